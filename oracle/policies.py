"""Offline replacement-policy comparator for one (request, layer) cache.

TEST INFRASTRUCTURE and offline analysis (see ``oracle/__init__.py``): plain
CPU code, never called by the GPU path.

"HiSparse 深度解析" (gentlecold.top) §3.3 compares, on selection traces,
keeping only the current top-k (B = k), FIFO, Random, LRU and Belady's offline
optimum at B = 2k, and LRU at B = 4k.  This module replays the seeded
synthetic traces under each of those policies and counts misses.

Model shared by every policy.  A cache holds at most B positions.  At each
step every selected position must be resident afterwards.  A selected
position already resident is a hit.  Every other selected position is a miss
and takes a victim slot: an empty slot if any is left, else a resident slot
whose position is not selected in this step.  Misses are served in selection
order, and the victims are taken in ascending order of the policy's eviction
key (empty slots first, in slot order):

- ``lru``     (stamp, slot).  A miss at step t stamps its slot 2t-1; a hit
              stamps 2t, so hits rank more recent than this step's misses
              (the cache's own rule, §3.3).
- ``fifo``    (fetch time, slot).  A miss stamps its slot with (t, j) for the
              j-th miss of step t; hits leave the stamp alone.
- ``random``  a fresh uniformly random key per slot and step, drawn from a
              seeded generator (a uniformly random victim set).
- ``belady``  (-next use, slot): the resident position selected again latest
              (never again ranks latest of all) goes first.
- ``topk``    ("swap-vanilla") B = k: after a step only the current
              selection is resident, so every policy behaves the same.

With the newest-token slot (§3.4), the just-appended position is served from
a slot outside the cache and counts as a hit; it is removed from the step's
selection before any policy sees it.
"""
from __future__ import annotations

import argparse
import sys
import time

import numpy as np

POLICIES = ("topk", "fifo", "random", "lru", "belady")
_NEVER = np.iinfo(np.int64).max


def next_use(trace) -> list:
    """For each step t and entry i, the first later step selecting trace[t][i] (or _NEVER)."""
    steps = len(trace)
    sizes = [len(s) for s in trace]
    pos = np.concatenate([np.asarray(s, np.int64) for s in trace]) if steps else np.empty(0, np.int64)
    step = np.repeat(np.arange(steps, dtype=np.int64), sizes)
    order = np.lexsort((step, pos))          # by position, then step
    nxt = np.full(pos.size, _NEVER, np.int64)
    same = pos[order][1:] == pos[order][:-1]
    nxt[order[:-1][same]] = step[order][1:][same]
    return np.split(nxt, np.cumsum(sizes)[:-1])


def simulate(trace, B: int, policy: str, newest=None, seed: int = 0, return_slots: bool = False):
    """Misses per step of ``trace`` (a list of selections) under ``policy``.

    ``newest``: per-step newest position (or None); it is a hit outside the cache.
    With ``return_slots`` also returns the position held by each slot at the end (-1 empty).
    """
    if policy not in POLICIES:
        raise ValueError("unknown policy %r" % policy)
    steps = len(trace)
    sels = []
    for t in range(steps):
        s = np.asarray(trace[t], np.int64)
        if newest is not None and newest[t] is not None:
            s = s[s != newest[t]]
        if np.unique(s).size != s.size:
            raise ValueError("duplicate position at step %d" % t)
        sels.append(s)
    if policy == "topk":
        B = max((s.size for s in sels), default=0)
    nu = next_use(sels) if policy == "belady" else None
    rng = np.random.Generator(np.random.PCG64(seed)) if policy == "random" else None
    holds = np.full(B, -1, np.int64)          # position in each slot (-1 empty)
    key = np.zeros(B, np.int64)               # eviction key (lower goes first)
    where: dict[int, int] = {}
    misses = np.zeros(steps, np.int64)
    for t in range(steps):
        s = sels[t]
        if s.size > B:
            raise ValueError("selection larger than the buffer at step %d" % t)
        slot = np.array([where.get(int(p), -1) for p in s], np.int64)
        hit = slot >= 0
        miss_idx = np.nonzero(~hit)[0]
        m = miss_idx.size
        misses[t] = m
        if policy == "random":
            key = rng.random(B)
        taken = np.zeros(B, bool)
        taken[slot[hit]] = True
        cand = np.nonzero(~taken)[0]
        empty = holds[cand] < 0
        # empty slots first in slot order, then the policy's key, ties by slot
        order = np.lexsort((cand, key[cand], ~empty))
        victims = cand[order[:m]]
        for j, (i, v) in enumerate(zip(miss_idx, victims)):
            old = int(holds[v])
            if old >= 0:
                del where[old]
            p = int(s[i])
            holds[v] = p
            where[p] = int(v)
        if policy == "lru":
            key[victims] = 2 * (t + 1) - 1
            key[slot[hit]] = 2 * (t + 1)
        elif policy == "fifo":
            key[victims] = (t + 1) * (B + 1) + np.arange(m)
        elif policy == "belady":
            # -next use: the furthest next selection is evicted first
            key[victims] = -nu[t][miss_idx]
            key[slot[hit]] = -nu[t][hit]
    return (misses, holds) if return_slots else misses


def workload_traces(w, requests=None, layers=None, steps=None):
    """Yields (r, l, trace, newest) for the independent caches of workload ``w``."""
    from synth.traces import selection_trace
    steps = w.steps if steps is None else steps
    requests = range(w.R) if requests is None else requests
    layers = [l for l in range(w.L) if l % w.group == 0] if layers is None else layers
    for r in requests:
        for l in layers:
            tr = selection_trace(w, r, l, steps)
            if w.block_tokens > 1:
                bt = w.block_tokens
                tr = [(np.asarray(row, np.int64)[:, None] * bt + np.arange(bt)).ravel() for row in tr]
            newest = [w.ctx + t for t in range(steps)] if w.append else None
            yield r, l, tr, newest


def compare(w, sizes, requests=None, layers=None, steps=None, seed=0) -> list:
    """Rows (policy, B, steady-state miss rate, cold-step misses) over the caches of ``w``.

    The steady-state rate counts steps 2.. (the first step of an empty cache misses everything).
    """
    rows = []
    tot = {}
    sel_total = 0
    cold = {}
    for r, l, tr, newest in workload_traces(w, requests, layers, steps):
        sel_total += sum(len(x) for x in tr[1:])
        for pol, B in sizes:
            ms = simulate(tr, B, pol, newest, seed=seed)
            tot[(pol, B)] = tot.get((pol, B), 0) + int(ms[1:].sum())
            cold[(pol, B)] = cold.get((pol, B), 0) + int(ms[0])
    for pol, B in sizes:
        rows.append((pol, B, tot[(pol, B)] / max(sel_total, 1), cold[(pol, B)]))
    return rows


def main(argv=None) -> int:
    import synth
    ap = argparse.ArgumentParser(description="offline replacement-policy comparison on the seeded traces")
    ap.add_argument("--workload", default="long", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--requests", type=int, default=None, help="first n requests only")
    ap.add_argument("--steps", type=int, default=None)
    args = ap.parse_args(argv)
    w = synth.WORKLOADS[args.workload]
    k = w.k
    sizes = [("topk", k), ("fifo", 2 * k), ("random", 2 * k), ("lru", 2 * k), ("belady", 2 * k),
             ("lru", 4 * k), ("belady", 4 * k)]
    reqs = range(min(w.R, args.requests)) if args.requests else None
    t0 = time.time()
    rows = compare(w, sizes, requests=reqs, steps=args.steps)
    print("workload %s: k=%d, %d steps, requests %s" % (w.name, k, args.steps or w.steps,
                                                         "all" if reqs is None else len(reqs)))
    print("%-8s %6s %10s %12s" % ("policy", "B", "miss rate", "cold misses"))
    for pol, B, rate, c in rows:
        print("%-8s %6d %9.2f%% %12d" % (pol, B, 100 * rate, c))
    print("(%.1f s)" % (time.time() - t0), file=sys.stderr)
    return 0


if __name__ == "__main__":
    sys.exit(main())
