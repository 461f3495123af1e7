"""Seeded resident-page layouts for the resident tier in front of the hot slots.

Input generation only: which logical pages of each request sit in the device's
regular paged KV cache at each step, and where.  Model, per request r:

* the pages ever resident are the last ``window_tokens`` of the prefill
  context plus each older prefill page with probability ``old_frac``;
* each gets a physical page; requests own disjoint physical ranges, in a
  seeded random order inside each range;
* at step t, the oldest ``t // spill_every`` pages of the window have been
  spilled (no longer resident), and each older page is absent with
  probability ``churn`` (drawn per step), so pages both leave and return.

``all_resident`` makes every prefill page resident at every step (a short
request that fits the device pool).  Generator of request r:
``numpy.random.Generator(PCG64(SeedSequence([cfg_id, r, 0x5E5])))``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class ResidentSpec:
    page_tokens: int = 64
    window_tokens: int = 8192
    old_frac: float = 0.05
    churn: float = 0.1
    spill_every: int = 4
    all_resident: bool = False


def resident_layout(w, steps: int, spec: ResidentSpec, max_positions: int | None = None):
    """Returns (phys int32 [R][n_pages], masks bool [steps][R][n_pages], total_pages).

    phys[r][pg] is the physical page of logical page pg of request r (-1 when the page
    is never resident); the block table of step t is where(masks[t], phys, -1).  The
    table covers ``max_positions`` positions (default: the workload's over ``steps``).
    """
    P = spec.page_tokens
    n_pages = -(-(max_positions or w.max_positions(steps)) // P)
    ctx_pages = w.ctx // P
    phys = np.full((w.R, n_pages), -1, np.int32)
    masks = np.zeros((steps, w.R, n_pages), bool)
    base = 0
    for r in range(w.R):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.cfg_id, r, 0x5E5])))
        if spec.all_resident:
            ever = np.arange(ctx_pages)
            win = ever
        else:
            w0 = max(0, ctx_pages - spec.window_tokens // P)
            win = np.arange(w0, ctx_pages)
            old = np.nonzero(rng.random(w0) < spec.old_frac)[0]
            ever = np.concatenate([old, win])
        phys[r, ever] = base + rng.permutation(ever.size).astype(np.int32)
        base += ever.size
        for t in range(steps):
            if spec.all_resident:
                masks[t, r, ever] = True
                continue
            keep_win = win[min(win.size, t // spec.spill_every):]
            masks[t, r, keep_win] = True
            old_now = old[rng.random(old.size) >= spec.churn]
            masks[t, r, old_now] = True
    return phys, masks, base
