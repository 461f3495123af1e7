"""Pure-Python list model of one (request, layer) cache.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).  Written independently of
``hs_oracle.c`` to pin it on exhaustive tiny traces: instead of stamps and a
sort it keeps the LRU as a Python list of slots, least recent first, and
moves slots to the recent end as they are used.

Rule, read from "HiSparse 深度解析" (gentlecold.top) §3.3 and §3.5: a miss
takes the least recent slot that does not hold a position selected in this
step (never-used slots are the least recent of all, lowest index first);
misses are served in list order; after the step the slots filled by misses
move to the recent end, then the slots hit in this step (hits rank newer than
fetched misses).  Slots that become recent together are ordered by slot index.
The newest token (§3.4) sits in slot B outside the list; an LRU slot that
holds the same position is treated as not selected.
"""
from __future__ import annotations


class ListCache:
    def __init__(self, B: int, newest_slot: bool = False):
        self.B = B
        self.newest_slot = newest_slot
        self.order = list(range(B))       # least recent first
        self.holds = [None] * B           # position held by each slot
        self.newest = None

    def append(self, pos: int) -> None:
        self.newest = pos

    def resolve(self, sel):
        """Returns (out, hits, misses, plan) for the selection ``sel``."""
        sel = [int(p) for p in sel]
        if len(set(sel)) != len(sel):
            raise ValueError("duplicate position")
        # the newest token is served from slot B, never through an LRU slot
        chosen = set(sel) - ({self.newest} if self.newest_slot else set())
        where = {p: s for s, p in enumerate(self.holds) if p is not None}
        out = [None] * len(sel)
        hit_slots, miss_idx = [], []
        for i, p in enumerate(sel):
            if self.newest_slot and p == self.newest:
                out[i] = self.B
            elif p in where:
                out[i] = where[p]
                hit_slots.append(where[p])
            else:
                miss_idx.append(i)
        free = [s for s in self.order if self.holds[s] is None or self.holds[s] not in chosen]
        if len(free) < len(miss_idx):
            raise ValueError("selection larger than the buffer")
        filled, plan = [], []
        for j, i in enumerate(miss_idx):
            s = free[j]
            self.holds[s] = sel[i]
            out[i] = s
            filled.append(s)
            plan.append((sel[i], s))
        for group in (sorted(filled), sorted(hit_slots)):
            for s in group:
                self.order.remove(s)
                self.order.append(s)
        return out, len(sel) - len(miss_idx), len(miss_idx), plan
