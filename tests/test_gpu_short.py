"""Short-sequence fast path on the GPU through the C ABI, against the oracle.

"HiSparse 深度解析" (gentlecold.top) §5.3-§5.5: a request whose tokens fit the
device buffer keeps them there in order; RESOLVE returns their own slots with
no host IO until the context outgrows B, then the normal path takes over.
Requests are admitted at different lengths, grow one token per step by
write-through appends, and cross B during the test; every step is compared bit
for bit with the oracle, the metadata and hot bytes at the end.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import hierarchical_kv_cache_amd as hk
import oracle
import synth

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def export(c, R, B):
    sp = torch.empty((R, B), dtype=torch.int32, device="cuda")
    lru = torch.empty((R, B), dtype=torch.int32, device="cuda")
    nw = torch.empty((R,), dtype=torch.int32, device="cuda")
    hk.hs_export_state(c.h, 0, sp.data_ptr(), lru.data_ptr(), 0, nw.data_ptr(), 0)
    torch.cuda.synchronize()
    return sp.cpu().numpy(), lru.cpu().numpy(), nw.cpu().numpy()


@pytest.mark.parametrize("rows", [1, 2])
def test_short_requests_cross_into_the_normal_path(rows):
    R, L, B, k = 3, 2, 256, 64
    ctx0 = [150, 200, 256]
    steps = 120
    lmax = max(ctx0) + steps + 1
    cfg = hk.make_config(R, L, lmax, k, B, newest_slot=True, wgs_per_request=3,
                         verify_rows=rows if rows > 1 else 0)
    Bc = cfg.buffer_slots
    c = hk.HiSparse(cfg)
    for r in range(R):
        synth.fill_request(c.host_pool_address(r), r, L, lmax, ctx0[r])
    ohost = [np.empty((L, lmax, 1152), np.uint8) for _ in range(R)]
    for r in range(R):
        synth.fill_request(ohost[r], r, L, lmax, ctx0[r])
    caches = [oracle.Cache(Bc, lmax, 1152, newest_slot=True) for _ in range(R)]
    for r in range(R):
        hk.hs_admit_short(c.h, r, ctx0[r], 0)
        caches[r].admit_short(ctx0[r], ohost[r][0])
    rng = np.random.default_rng(7 + rows)
    dev = torch.device("cuda")
    side = torch.cuda.Stream()
    shape = (R, rows, k) if rows > 1 else (R, k)
    out = torch.empty(shape, dtype=torch.int32, device=dev)
    st = torch.zeros((R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    ctx = list(ctx0)
    fast = slow = 0
    for t in range(steps):
        pos = np.array(ctx, np.int32)  # the new token of each request
        recs = synth.records_at(R, L, pos)  # [R][L][rec]: request r's record at pos[r]
        d_new = torch.from_numpy(recs).to(dev)
        d_pos = torch.from_numpy(pos).to(dev)
        hk.hs_writeback(c.h, d_new.data_ptr(), d_pos.data_ptr(), torch.cuda.current_stream().cuda_stream,
                     side.cuda_stream)
        for r in range(R):
            caches[r].append(int(pos[r]), recs[r, 0], ohost[r][0])
            ctx[r] += 1
        sel = np.empty((R, rows, k), np.int32)
        for r in range(R):
            base = rng.choice(ctx[r] - 1, size=k - 1, replace=False)
            for q in range(rows):
                row = np.concatenate([[ctx[r] - 1], base if q == 0 else rng.choice(ctx[r] - 1, k - 1, replace=False)])
                sel[r, q] = rng.permutation(row)
        d_ctx = torch.tensor(ctx, dtype=torch.int32, device=dev)
        d_sel = torch.from_numpy(sel if rows > 1 else sel[:, 0].copy()).to(dev)
        if rows > 1:
            hk.hs_resolve_rows(c.h, 0, rows, d_sel.data_ptr(), d_ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0,
                               torch.cuda.current_stream().cuda_stream)
        else:
            hk.hs_resolve(c.h, 0, d_sel.data_ptr(), d_ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0,
                          torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        got, s = out.cpu().numpy(), st.cpu().numpy()
        for r in range(R):
            if rows > 1:
                o, hh, mm, rr, pp, ps, nu = caches[r].resolve_rows(sel[r], ctx[r], ohost[r][0])
            else:
                o, hh, mm, pp, ps = caches[r].resolve(sel[r, 0], ctx[r], ohost[r][0])
            if ctx[r] <= Bc:
                fast += 1
            else:
                slow += 1
            assert s[r, 2] == 0 and s[r, 0] == hh and s[r, 1] == mm, (t, r, s[r], hh, mm)
            assert np.array_equal(got[r], o), (t, r)
    log("short: %d fast-path calls, %d normal" % (fast, slow))
    assert fast > 0 and slow > 0
    sp, lru, nw = export(c, R, Bc)
    hot = c.hot.cpu().numpy()
    for r in range(R):
        e = caches[r].export()
        assert np.array_equal(sp[r], e["slot_pos"]) and np.array_equal(lru[r], e["lru"]) and nw[r] == e["newest_pos"]
        occ = np.nonzero(e["slot_pos"] >= 0)[0]
        assert np.array_equal(hot[r, 0, occ], caches[r].hot[occ])
        # layer 1 is never resolved here: admission and appends filled its B slots in order
        assert all(np.array_equal(hot[r, 1, s_], synth.record(r, 1, s_)) for s_ in range(0, Bc, 17))
    c.close()


def test_fast_path_range_error_and_reset():
    R, B, k, lmax = 2, 128, 16, 512
    c = hk.HiSparse(hk.make_config(R, 1, lmax, k, B))
    for r in range(R):
        synth.fill_request(c.host_pool_address(r), r, 1, lmax, lmax)
    for r in range(R):
        hk.hs_admit_short(c.h, r, 100, 0)
    dev = torch.device("cuda")
    sel = np.stack([np.arange(k), np.arange(k) + 90]).astype(np.int32)  # request 1 reaches 105 >= 100
    out = torch.empty((R, k), dtype=torch.int32, device=dev)
    st = torch.zeros((R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    ctx = torch.full((R,), 100, dtype=torch.int32, device=dev)
    hk.hs_resolve(c.h, 0, torch.from_numpy(sel).to(dev).data_ptr(), ctx.data_ptr(), out.data_ptr(), st.data_ptr(),
                  0, 0, 0)
    torch.cuda.synchronize()
    got, s = out.cpu().numpy(), st.cpu().numpy()
    assert np.array_equal(got[0], sel[0]) and s[0, 0] == k and s[0, 2] == 0
    assert (got[1] == -1).all() and s[1, 2] == hk.HS_ERR_RANGE
    # the records are in their own slots
    hot = c.hot.cpu().numpy()
    assert all(np.array_equal(hot[0, 0, p], synth.record(0, 0, p)) for p in range(0, 100, 7))
    # a reset request is no longer short: the normal path misses everything
    hk.hs_reset_request(c.h, 0, 0)
    hk.hs_resolve(c.h, 0, torch.from_numpy(sel).to(dev).data_ptr(), ctx.data_ptr(), out.data_ptr(), st.data_ptr(),
                  0, 0, 0)
    torch.cuda.synchronize()
    assert st.cpu().numpy()[0, 1] == k
    c.close()
