"""Resident tier in front of the hot slots, on the GPU through the C ABI, against the oracle.

"HiSparse 深度解析" (gentlecold.top) §6.5 and "HiSparse local KV offload
architecture" (docs.vllm.ai), "Hot lookup and LRU": resident page first, then
hot slot, then pinned host.  Every step compares the published rows and the
counts bit for bit with ``Cache.resolve_tiered``; metadata and hot bytes are
compared at the end; attention reads resident and hot rows alike.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest
import torch

import hierarchical_kv_cache_amd as hk
import oracle
import synth
from harness import SCALE, Pair
from synth.resident import ResidentSpec

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attn_check(p, step, layers, heads=16):
    """Attention over the published rows: hot slots 0..B, resident rows above."""
    w = p.w
    q = synth.queries(w.R, w.L, step, heads=heads)
    d_q = torch.from_numpy(q.view(np.int16)).to("cuda")
    out = torch.empty((w.R, heads, 512), dtype=torch.float32, device="cuda")
    worst = 0.0
    for l in layers:
        a = l - l % w.group
        ai = p.anchors.index(a)
        hk.hs_wait_layer(p.h, l, 0)
        hk.hs_sparse_attn(p.h, l, d_q[:, l].contiguous().data_ptr(), heads, 512, p.d_out[ai].data_ptr(),
                          out.data_ptr(), SCALE, 0, 0)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        slots = p.d_out[ai].cpu().numpy()
        for r in range(w.R):
            hot = p.caches[(r, l)].hot if l == a else p.ohot_shared[(r, l)]
            rows = np.concatenate([hot, p.res_pool[l]])
            ref = oracle.attention.sparse_decode_attention(q[r, l], rows, slots[r], SCALE)
            err = np.abs(o[r] - ref).max() / np.abs(ref).max()
            worst = max(worst, err)
            assert err <= 2e-3, (r, l, err)
    return worst


def run(p, steps, attn_every=0):
    tot = np.zeros(3, np.int64)
    for t in range(steps):
        log("step %d" % t)
        res = p.step_gpu_and_oracle()
        for v in res.values():
            tot += (v[1], v[2], v[5])
        if attn_every and (t % attn_every == attn_every - 1):
            attn_check(p, t, range(p.w.L))
    p.check_state()
    return tot


def test_long_with_resident_window():
    w = W["long"]
    p = Pair(w, steps=16, resident=ResidentSpec(window_tokens=16384, old_frac=0.05))
    hits, misses, res = run(p, 16, attn_every=8)
    log("long+resident: hits %d misses %d resident %d" % (hits, misses, res))
    assert res > 0 and misses > 0 and hits > 0
    p.close()


def test_batched_with_resident_pages():
    w = W["batched"].scaled(L=2)
    p = Pair(w, steps=6, resident=ResidentSpec(window_tokens=4096, old_frac=0.1, churn=0.2, spill_every=2))
    run(p, 6, attn_every=3)
    p.close()


def test_capacity_blocks_with_resident_pages():
    w = W["capacity"].scaled(ctx=131072)
    p = Pair(w, steps=8, resident=ResidentSpec(window_tokens=16384, old_frac=0.1))
    run(p, 8)
    p.close()


def test_shared_layers_with_resident_pages():
    w = W["shared"].scaled(R=2, L=8, ctx=16384)
    p = Pair(w, steps=4, resident=ResidentSpec(window_tokens=2048, old_frac=0.2))
    run(p, 4, attn_every=2)
    p.check_hot()
    p.close()


def test_all_resident_returns_early_and_changes_nothing():
    """A short request whose pages are all resident: every call publishes resident rows,
    reports top_k resident entries, and leaves the hot metadata in its admission state."""
    w = W["batched"].scaled(R=4, L=2, ctx=8192, k=512, B=1024)
    p = Pair(w, steps=5, resident=ResidentSpec(all_resident=True))
    run(p, 5, attn_every=5)
    for key in p.caches:
        st = p.caches[key].export()
        assert (st["slot_pos"] == -1).all() and st["step"] == 0
    p.close()


def test_alternating_all_resident_and_hot_steps():
    """Steps served entirely by the resident tier (the kernel returns early and keeps its
    metadata half) interleaved with steps through the hot slots."""
    w = W["tiny"].scaled(R=3, steps=12)
    p = Pair(w, steps=12, wgs=3, resident=ResidentSpec(page_tokens=16, all_resident=True))
    full = p.masks.copy()
    for t in range(12):
        p.masks[t] = full[t] if t % 3 == 1 else (full[t] & (t % 3 == 2) & (np.arange(full.shape[2]) % 2 == 0))
    res = [0, 0, 0]
    for t in range(12):
        out = p.step_gpu_and_oracle()
        for v in out.values():
            res[0] += v[1]; res[1] += v[2]; res[2] += v[5]
    p.check_state()
    assert res[2] > 0 and res[1] > 0
    p.close()


def test_resident_row_outside_the_pool_is_an_error():
    w = W["tiny"].scaled(R=2)
    p = Pair(w, steps=4, resident=ResidentSpec(page_tokens=64, window_tokens=1024))
    p.step_gpu_and_oracle()
    torch.cuda.synchronize()
    before = [p.caches[(r, 0)].export() for r in range(2)]
    # request 1's first resident page points past the pool
    tab = p.table(1)
    pg = int(np.nonzero(tab[1] >= 0)[0][0])
    tab[1, pg] = p.res_rows // 64
    p.d_table.copy_(torch.from_numpy(tab))
    sel = p.trace[1, 0].copy()
    x = pg * 64 + 3
    if x not in sel[1]:
        sel[1, 0] = x
    d_sel = torch.from_numpy(sel).cuda()
    d_ctx = torch.full((2,), w.ctx, dtype=torch.int32, device="cuda")
    hk.hs_resolve(p.h, 0, d_sel.data_ptr(), d_ctx.data_ptr(), p.d_out[0].data_ptr(), p.d_stats.data_ptr(), 0, 0,
                  p.compute.cuda_stream)
    st = p.d_stats.cpu().numpy()
    assert st[1, 2] & hk.HS_ERR_RESIDENT and (p.d_out[0][1] == -1).all().item()
    with pytest.raises(oracle.OracleError) as e:
        p.caches[(1, 0)].resolve_tiered(sel[1], w.ctx, tab[1], 6, p.res_rows, p.ohost[1][0])
    assert e.value.code & oracle.ERR_RESIDENT
    # request 0 resolved normally: feed the oracle the same call
    p.caches[(0, 0)].resolve_tiered(sel[0], w.ctx, tab[0], 6, p.res_rows, p.ohost[0][0])
    assert st[0, 2] == 0
    after = p.caches[(1, 0)].export()
    assert np.array_equal(after["slot_pos"], before[1]["slot_pos"])
    p.t = 2
    p.check_state(hot=False)
    p.close()


def test_unbind_returns_to_the_two_level_path():
    w = W["tiny"].scaled(R=2)
    p = Pair(w, steps=6, resident=ResidentSpec(page_tokens=64, window_tokens=1024))
    for _ in range(3):
        p.step_gpu_and_oracle()
    hk.hs_bind_resident(p.h, 0, 0, 0, 0, 0)
    # the oracle follows with an empty table from now on
    p.masks[3:] = False
    for _ in range(3):
        p.step_gpu_and_oracle()
    p.check_state()
    p.close()
