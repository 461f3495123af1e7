"""Seeded top-k selection traces.

A trace is the sequence of selections S_1, S_2, ... of one (request, layer)
cache.  Each selection is an ordered list of distinct entries (token
positions, or block ids when the workload selects blocks).  The model, per
step t with N selectable units:

1. kept   = the entries of S_{t-1}, each kept with probability keep_p, in the
            order they had in S_{t-1};
2. forced = the last ``forced_last`` units (ascending), or the just-appended
            token when ``force_newest``; forced entries always stay, and kept
            entries beyond the room left are dropped from the end;
3. fresh  = draws until the list holds kb entries: each draw is uniform over
            [0, N) with probability ``uniform_frac``, else N-1-d with
            d = Zipf(zipf_a) - 1 (a draw with d >= N is discarded); draws
            already present are discarded;
4. the list kept ++ forced ++ fresh is shuffled by a seeded permutation.

The generator of cache (r, l) of workload ``cfg_id`` is
``numpy.random.Generator(PCG64(SeedSequence([cfg_id, r, l])))``.
With ``all_hit`` every step after the first repeats the first selection.
"""
from __future__ import annotations

import numpy as np


def selection_trace(w, r: int, l: int, steps: int | None = None, all_hit: bool = False,
                    kb: int | None = None) -> np.ndarray:
    """int32 [steps][kb] selection entries of cache (r, l) of workload ``w``."""
    steps = w.steps if steps is None else steps
    kb = w.kb if kb is None else kb
    bt = w.block_tokens
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.cfg_id, r, l])))
    n_max = (w.ctx + (steps if w.append else 0)) // bt
    member = np.zeros(n_max, dtype=bool)
    out = np.empty((steps, kb), dtype=np.int32)
    prev = np.empty(0, dtype=np.int64)
    for t in range(steps):
        if all_hit and t > 0:
            out[t] = out[0]
            continue
        n_units = (w.ctx + (t + 1 if w.append else 0)) // bt
        if n_units < kb:
            raise ValueError("context holds fewer units than the selection size")
        kept = prev[rng.random(prev.size) < w.keep_p]
        if w.forced_last:
            forced = np.arange(n_units - w.forced_last, n_units, dtype=np.int64)
        elif w.force_newest:
            forced = np.array([n_units - 1], dtype=np.int64)
        else:
            forced = np.empty(0, dtype=np.int64)
        member[forced] = True
        kept = kept[~member[kept]][: kb - forced.size]
        member[kept] = True
        parts = [kept, forced]
        need = kb - kept.size - forced.size
        while need > 0:
            n = max(2 * need, 16)
            if w.uniform_frac >= 1.0:
                cand = rng.integers(0, n_units, n)
            elif w.uniform_frac <= 0.0:
                d = rng.zipf(w.zipf_a, n) - 1
                cand = (n_units - 1 - d)[d < n_units]
            else:
                coin = rng.random(n) < w.uniform_frac
                uni = rng.integers(0, n_units, n)
                d = rng.zipf(w.zipf_a, n) - 1
                ok = coin | (d < n_units)
                cand = np.where(coin, uni, n_units - 1 - np.minimum(d, n_units - 1))[ok]
            cand = cand[~member[cand]]
            _, first = np.unique(cand, return_index=True)
            cand = cand[np.sort(first)][:need]
            member[cand] = True
            parts.append(cand)
            need -= cand.size
        sel = np.concatenate(parts)
        member[sel] = False
        sel = rng.permutation(sel)
        out[t] = sel
        prev = sel
    return out


def trace_stats(trace: np.ndarray) -> dict:
    """Step-to-step reuse of a trace: mean |S_t & S_{t-1}| / kb over t >= 1."""
    if trace.shape[0] < 2:
        return {"reuse": float("nan")}
    reuse = [np.intersect1d(trace[t], trace[t - 1]).size / trace.shape[1]
             for t in range(1, trace.shape[0])]
    return {"reuse": float(np.mean(reuse))}


def verify_rows(w, r: int, l: int, steps: int, rows: int, keep: float = 0.9) -> np.ndarray:
    """int32 [steps][rows][kb] selections of the verification rows of speculative steps.

    Row 0 of step t is ``selection_trace``'s selection; row q > 0 keeps each entry of row
    q-1 with probability ``keep`` (in order), then draws fresh entries as the trace model
    does (uniform over the context with probability ``uniform_frac``, else recency-Zipf),
    then is shuffled.  Generator: PCG64(SeedSequence([cfg_id, r, l, 0x5BEC])).
    """
    base = selection_trace(w, r, l, steps)
    kb = base.shape[1]
    bt = w.block_tokens
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.cfg_id, r, l, 0x5BEC])))
    out = np.empty((steps, rows, kb), dtype=np.int32)
    for t in range(steps):
        n_units = (w.ctx + (t + 1 if w.append else 0)) // bt
        out[t, 0] = base[t]
        for q in range(1, rows):
            prev = out[t, q - 1].astype(np.int64)
            kept = prev[rng.random(kb) < keep]
            member = set(kept.tolist())
            fresh = []
            while len(kept) + len(fresh) < kb:
                if rng.random() < w.uniform_frac:
                    c = int(rng.integers(0, n_units))
                else:
                    d = int(rng.zipf(w.zipf_a)) - 1
                    if d >= n_units:
                        continue
                    c = n_units - 1 - d
                if c not in member:
                    member.add(c)
                    fresh.append(c)
            out[t, q] = rng.permutation(np.concatenate([kept, np.array(fresh, np.int64)]))
    return out
