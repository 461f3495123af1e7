"""Speculative multi-row RESOLVE on the GPU through the C ABI, against the oracle.

"HiSparse 深度解析" (gentlecold.top) §6.5 comparison table and "HiSparse local
KV offload architecture" (docs.vllm.ai), speculative decoding: the verification
rows of one step are resolved as the union of their selections in first-
reference order.  Every step compares every row's published slots and the
union's counts bit for bit with ``Cache.resolve_rows``; metadata and hot bytes
are compared at the end.
"""
from __future__ import annotations

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


def run(p, steps):
    tot = np.zeros(3, np.int64)
    for t in range(steps):
        res = p.step_gpu_and_oracle()
        for v in res.values():
            tot += (v[1], v[2], v[5])
    p.check_state()
    return tot


@pytest.mark.parametrize("rows,wgs", [(2, 0), (3, 3), (4, 1)])
def test_tiny_rows(rows, wgs):
    w = W["tiny"].scaled(R=3, B=64 * rows + 8)
    p = Pair(w, steps=12, wgs=wgs, rows=rows)
    run(p, 12)
    p.close()


def test_long_four_rows_with_write_through():
    """MTP with three draft tokens: four rows of k = 2048, B = 5 k (the pages' default)."""
    w = W["long"].scaled(L=2, B=5 * 2048)
    p = Pair(w, steps=8, rows=4)
    h, m, r = run(p, 8)
    log("long 4 rows: hits %d misses %d" % (h, m))
    p.close()


def test_long_and_short_unions_in_one_call():
    """Unions on both sides of 4096 entries in the same call: a union of at most 4 x 1024
    entries is resolved by the launch with 4 list entries per thread, a longer one by the launch
    with 8 (each request's workgroups return at entry in the other launch).  4 rows of k = 2048
    into B = 10240 (12 slots per thread); request 0's rows keep 90 % of the row before (union
    about 2650), request 1's 30 % (about 6300); 12 steps, past the buffer-fill point of request 1."""
    w = W["long"].scaled(R=2, L=1, B=5 * 2048, append=False, force_newest=False)
    p = Pair(w, steps=12, rows=4, rows_keep=(0.9, 0.3))
    short = long_ = 0
    for t in range(12):
        res = p.step_gpu_and_oracle()
        for (r, l), v in res.items():
            n = int(v[1]) + int(v[2]) + int(v[5])
            short += n <= 4096
            long_ += n > 4096
        if t in (5, 11):
            p.check_state()
    log("unions <= 4096: %d, > 4096: %d; occupied slots evicted %d" % (short, long_, p.evicted))
    assert short >= 12 and long_ >= 12, (short, long_)
    assert p.evicted > 0
    p.check_hot()
    p.close()


@pytest.mark.parametrize("rows,B,keep", [(3, 8192, 0.9), (3, 8192, 0.2), (4, 16384, 0.9), (4, 16384, 0.25)])
def test_union_kernel_layouts(rows, B, keep):
    """The union RESOLVE kernel at 8 and 16 slots per thread (resolve_union_kernel<8, 8> and
    <16, 8>): rows x k 2048 > 4096 entries of capacity, the union short (rows keep 90 % of the
    row before: the 4-entries-per-thread body) or long (25-20 %: past 4096 entries, the full
    body); 6 steps, the state after the last."""
    w = W["long"].scaled(L=1, B=B, append=False, force_newest=False)
    p = Pair(w, steps=6, rows=rows, rows_keep=keep)
    sizes = []
    for _ in range(6):
        for (r, l), v in p.step_gpu_and_oracle().items():
            sizes.append(int(v[1]) + int(v[2]) + int(v[5]))
    log("rows %d B %d keep %.2f: union sizes %s" % (rows, B, keep, sizes))
    assert (max(sizes) > 4096) == (keep < 0.5), sizes
    p.check_state()
    p.close()


def test_batched_rows():
    w = W["batched"].scaled(R=8, L=2, k=1024, B=3 * 1024)
    p = Pair(w, steps=5, rows=3)
    run(p, 5)
    p.close()


def test_rows_with_shared_layers_and_resident_tier():
    w = W["shared"].scaled(R=2, L=4, ctx=16384, k=512, B=2048, group=2)
    p = Pair(w, steps=4, rows=2, resident=ResidentSpec(window_tokens=2048, old_frac=0.2))
    run(p, 4)
    p.check_hot()
    p.close()


def test_rows_capacity_blocks():
    w = W["capacity"].scaled(ctx=131072, k=1024, B=2 * 1024)
    p = Pair(w, steps=4, rows=2)
    run(p, 4)
    p.close()


def test_attention_per_row():
    """Each verification row's attention reads its own published slots."""
    w = W["batched"].scaled(R=4, L=1, k=512, B=1536, heads=16)
    p = Pair(w, steps=2, rows=3)
    run(p, 2)
    q = synth.queries(w.R, 3, 1, heads=16)  # one query set per row
    slots = p.d_out[0].cpu().numpy()  # [R][rows][k]
    out = torch.empty((w.R, 16, 512), dtype=torch.float32, device="cuda")
    for row in range(3):
        d_q = torch.from_numpy(q[:, row].view(np.int16).copy()).cuda()
        d_slots = torch.from_numpy(np.ascontiguousarray(slots[:, row])).cuda()
        hk.hs_sparse_attn(p.h, 0, d_q.data_ptr(), 16, 512, d_slots.data_ptr(), out.data_ptr(), SCALE, 0, 0)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        for r in range(w.R):
            ref = oracle.attention.sparse_decode_attention(q[r, row], p.caches[(r, 0)].hot, slots[r, row], SCALE)
            assert np.abs(o[r] - ref).max() <= 2e-3 * np.abs(ref).max()
    p.close()


def test_duplicate_inside_a_row_is_an_error_repeats_across_rows_are_not():
    R, k, B, lmax = 3, 32, 128, 4096
    cfg = hk.make_config(R, 1, lmax, k, B, verify_rows=3, wgs_per_request=2)
    c = hk.HiSparse(cfg)
    for r in range(R):
        synth.fill_request(c.host_pool_address(r), r, 1, lmax, lmax)
    caches = [oracle.Cache(B, lmax, 1152) for _ in range(R)]
    rng = np.random.default_rng(1)
    dev = torch.device("cuda")
    out = torch.empty((R, 3, k), dtype=torch.int32, device=dev)
    st = torch.zeros((R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    ctx = torch.full((R,), lmax, dtype=torch.int32, device=dev)
    for step in range(6):
        sel = np.stack([np.stack([rng.choice(lmax, k, replace=False) for _ in range(3)]) for _ in range(R)]).astype(np.int32)
        sel[:, 1, :8] = sel[:, 0, :8]              # repeats across rows: shared slots
        if step % 2 == 1:
            sel[1, 2, 5] = sel[1, 2, 9]            # a duplicate inside row 2 of request 1
        hk.hs_resolve_rows(c.h, 0, 3, torch.from_numpy(sel).cuda().data_ptr(), ctx.data_ptr(), out.data_ptr(),
                           st.data_ptr(), 0, 0, 0)
        torch.cuda.synchronize()
        got, s = out.cpu().numpy(), st.cpu().numpy()
        for r in range(R):
            try:
                ref = caches[r].resolve_rows(sel[r], lmax, c.host_pool(r)[0])
            except oracle.OracleError as e:
                assert s[r, 2] == e.code and (got[r] == -1).all(), (step, r)
                continue
            assert s[r, 2] == 0 and s[r, 0] == ref[1] and s[r, 1] == ref[2], (step, r, s[r], ref[1:3])
            assert np.array_equal(got[r], ref[0]), (step, r)
            assert np.array_equal(got[r][1, :8], got[r][0, :8])
    c.close()


def test_one_launch_errors_and_padded_requests():
    """The one-launch rows kernel (3 rows of k 2048 into B 8192: the union's capacity needs more
    than 4 list entries per thread and its LDS fits): a duplicate inside a row and a position
    out of range make only their request's rows -1 with the error and leave its state alone;
    repeats across rows share slots; a request past num_reqs is untouched.  Every other request's
    slots and counts against the oracle, 8 steps, and the state at the end."""
    R, k, B, rows = 3, 2048, 8192, 3
    lmax = 65536
    cfg = hk.make_config(R, 1, lmax, k, B, verify_rows=rows)
    c = hk.HiSparse(cfg)
    for r in range(R):
        synth.fill_request(c.host_pool_address(r), r, 1, lmax, lmax)
    caches = [oracle.Cache(B, lmax, 1152) for _ in range(R)]
    rng = np.random.default_rng(7)
    dev = torch.device("cuda")
    out = torch.full((R, rows, k), -7, dtype=torch.int32, device=dev)
    st = torch.zeros((R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    ctx = torch.full((R,), lmax, dtype=torch.int32, device=dev)
    prev = [rng.choice(lmax, k, replace=False) for _ in range(R)]
    n_err = n_ok = n_pad = 0
    for step in range(8):
        nreq = R - 1 if step in (3, 6) else R  # request 2 padded in two steps
        sel = np.empty((R, rows, k), np.int32)
        for r in range(R):
            for q in range(rows):
                row = prev[r].copy()
                fresh = rng.choice(lmax, k, replace=False)
                keep = rng.random(k) < 0.8
                cand = np.where(keep, row, -1)
                used = set(int(x) for x in cand if x >= 0)
                fi = iter(int(x) for x in fresh if int(x) not in used)
                sel[r, q] = [int(x) if x >= 0 else next(fi) for x in cand]
                prev[r] = sel[r, q].copy()
        if step % 3 == 1:
            sel[1, 2, 5] = sel[1, 2, 9]        # a duplicate inside row 2 of request 1
        if step % 3 == 2:
            sel[0, 1, 100] = lmax + 3          # a position out of range in request 0
        d_nr = torch.tensor([nreq], dtype=torch.int32, device=dev)
        out.fill_(-7)
        before = out.clone()
        hk.hs_resolve_rows(c.h, 0, rows, torch.from_numpy(sel).cuda().data_ptr(), ctx.data_ptr(), out.data_ptr(),
                           st.data_ptr(), d_nr.data_ptr(), 0, 0)
        torch.cuda.synchronize()
        got, s = out.cpu().numpy(), st.cpu().numpy()
        for r in range(R):
            if r >= nreq:
                assert np.array_equal(got[r], before[r].cpu().numpy()), (step, r)  # untouched
                n_pad += 1
                continue
            try:
                ref = caches[r].resolve_rows(sel[r], lmax, c.host_pool(r)[0])
            except oracle.OracleError as e:
                assert s[r, 2] == e.code and (got[r] == -1).all(), (step, r, s[r])
                n_err += 1
                continue
            assert s[r, 2] == 0 and s[r, 0] == ref[1] and s[r, 1] == ref[2], (step, r, s[r], ref[1:3])
            assert np.array_equal(got[r], ref[0]), (step, r)
            n_ok += 1
    assert n_err >= 4 and n_ok >= 12 and n_pad == 2, (n_err, n_ok, n_pad)
    # the state at the end: slot maps and LRU orders against the oracle (a failed step changed nothing)
    sp = torch.empty((R, B), dtype=torch.int32, device=dev)
    lru = torch.empty((R, B), dtype=torch.int32, device=dev)
    nw = torch.empty((R,), dtype=torch.int32, device=dev)
    hk.hs_export_state(c.h, 0, sp.data_ptr(), lru.data_ptr(), 0, nw.data_ptr(), 0)
    torch.cuda.synchronize()
    sp, lru = sp.cpu().numpy(), lru.cpu().numpy()
    for r in range(R):
        ex = caches[r].export()
        assert np.array_equal(sp[r], ex["slot_pos"]), ("slot_pos", r)
        assert np.array_equal(lru[r], ex["lru"]), ("lru", r)
    c.close()


def test_rows_refused_without_verify_rows():
    cfg = hk.make_config(1, 1, 1024, 64, 128)
    c = hk.HiSparse(cfg)
    d = torch.zeros((1, 2, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(hk.HsError):
        hk.hs_resolve_rows(c.h, 0, 2, d.data_ptr(), d.data_ptr(), d.data_ptr(), 0, 0, 0, 0)
    c.close()
