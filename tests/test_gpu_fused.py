"""hs_resolve_attn: RESOLVE and the sparse attention over the published slots in one kernel.

Every step: slots, counts and (at the end) the slot map, LRU order, page table and hot
bytes bit for bit against the oracle, as for hs_resolve; the attention output within
2e-3 * max|o_ref| of float64 attention over the records of the selected positions.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu]

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import hierarchical_kv_cache_amd as hk  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from harness import Pair, SCALE  # noqa: E402
from synth.resident import ResidentSpec  # noqa: E402

W = synth.WORKLOADS


def log(msg):
    print(msg, flush=True)


def run(p: Pair, steps=None, expect_fused=True):
    assert (hk.hs_resolve_attn_wgs(p.h) > 0) == expect_fused, hk.hs_resolve_attn_wgs(p.h)
    for _ in range(p.steps if steps is None else steps):
        p.step_gpu_and_oracle()
    p.check_state()
    log("  worst attention rel err %.2e" % p.worst_attn)


@pytest.mark.parametrize("B", [64, 128, 256])
def test_tiny_one_chunk(B):
    """k = 64: one fetch workgroup per request writes the output itself (no merge)."""
    w = W["tiny"].scaled(R=3, B=B)
    log("tiny R=3 B=%d" % B)
    p = Pair(w, fused_heads=16)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == 2
        run(p)
    finally:
        p.close()


@pytest.mark.parametrize("k,heads", [(100, 5), (1000, 16), (130, 1), (65, 3)])
def test_ragged_chunks(k, heads):
    """Shares of 50, 62-63, 43-44 and 32-33 entries; fewer than 16 heads."""
    w = W["tiny"].scaled(k=k, B=max(128, k + 40), R=3, forced_last=min(16, k), steps=6)
    log("ragged k=%d heads=%d" % (k, heads))
    p = Pair(w, fused_heads=heads)
    try:
        run(p)
    finally:
        p.close()


def test_long_with_write_through():
    """The long-request shape (k 2048, B 4096, 33 workgroups), newest slot via write-through."""
    w = W["long"].scaled(L=2, steps=6)
    log("long L=2 steps=6")
    p = Pair(w, fused_heads=16)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == 33
        run(p)
    finally:
        p.close()


@pytest.mark.parametrize("k,B,fp8", [(4096, 4096, False), (3000, 6000, False), (4096, 4096, True)])
def test_four_entries_per_thread(k, B, fp8):
    """Lists longer than 2048 entries (4 per thread in workgroup 0: resolve_kernel<4, 4, true>,
    <8, 4, true> and the FP8 kernel <4, 4>), 2 requests of the long shape, write-through; 8
    steps, the buffer filled and evicting from the third."""
    w = W["long"].scaled(R=2, L=1, k=k, B=B, ctx=65536, steps=8, keep_p=0.6)
    log("k=%d B=%d fp8=%s" % (k, B, fp8))
    p = Pair(w, fused_heads=16, fp8=fp8)
    try:
        run(p)
        assert p.evicted > 0, p.evicted
    finally:
        p.close()


def test_batched_four_requests():
    w = W["batched"].scaled(R=4, L=2, steps=4, B=4096)
    log("batched R=4 L=2 B=4096")
    p = Pair(w, fused_heads=16)
    try:
        run(p)
    finally:
        p.close()


def test_capacity_blocks():
    w = W["capacity"].scaled(R=2, L=2, ctx=262144, steps=4)
    log("capacity blocks R=2 L=2 ctx=262144")
    p = Pair(w, fused_heads=16)
    try:
        run(p)
    finally:
        p.close()


def test_resident_tier():
    """Resident rows read from the resident pool, hot rows and misses in one tile."""
    w = W["long"].scaled(L=2, ctx=65536, steps=5)
    log("long with a resident window")
    p = Pair(w, fused_heads=16, resident=ResidentSpec(page_tokens=64, window_tokens=16384, old_frac=0.1,
                                                      spill_every=1, churn=0.05))
    try:
        run(p)
    finally:
        p.close()


def test_shared_layers_anchor_fused():
    """Anchors through the fused call (with the miss plan), shared layers through the replay and
    hs_sparse_attn on the anchor's slots."""
    w = W["shared"].scaled(R=2, L=4, ctx=16384, steps=3)
    log("shared R=2 L=4")
    p = Pair(w, fused_heads=16)
    try:
        run(p)
        p.check_hot()
    finally:
        p.close()


def test_padded_requests_untouched():
    w = W["tiny"].scaled(R=4, steps=4)
    p = Pair(w, fused_heads=16)
    try:
        sentinel = torch.full_like(p.d_att, 7.0)
        p.d_att.copy_(sentinel)
        for _ in range(3):
            p.step_gpu_and_oracle(num_reqs=3)
        torch.cuda.synchronize()
        assert torch.equal(p.d_att[:, 3], sentinel[:, 3])
        p.check_state(requests=range(3))
    finally:
        p.close()


@pytest.mark.parametrize("R,wgs", [(3, 5), (60, 3)])
def test_errors_give_nan_rows_and_leave_state(R, wgs):
    """A duplicate in one request: its error bits, its output rows NaN, nothing of it changes;
    the other requests resolve and attend as usual.  With 60 requests the fetch workgroups
    attend two tiles each."""
    k, B, lmax, ctx = 256, 512, 8192, 6000
    cfg = hk.make_config(R, 1, lmax, k, B)
    c = hk.HiSparse(cfg)
    try:
        assert hk.hs_resolve_attn_wgs(c.h) == wgs
        for r in range(R):
            synth.fill_request(c.host_pool_address(r), r, 1, lmax, lmax)
        caches = [oracle.Cache(B, lmax, 1152) for _ in range(R)]
        dev = torch.device("cuda")
        out = torch.empty((R, k), dtype=torch.int32, device=dev)
        st = torch.zeros((R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
        att = torch.empty((R, 16, 512), dtype=torch.float32, device=dev)
        d_ctx = torch.full((R,), ctx, dtype=torch.int32, device=dev)
        rng = np.random.default_rng(3)
        for t in range(4):
            sels = [rng.choice(ctx, k, replace=False).astype(np.int32) for _ in range(R)]
            bad = t % 2 == 1
            if bad:
                sels[1][200] = sels[1][7]
            q = synth.queries(R, 1, t)
            d_q = torch.from_numpy(q[:, 0].copy().view(np.int16)).to(dev)
            d_sel = torch.from_numpy(np.stack(sels)).to(dev)
            hk.hs_resolve_attn(c.h, 0, d_sel.data_ptr(), d_ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0,
                               d_q.data_ptr(), 16, 512, att.data_ptr(), SCALE, 0)
            torch.cuda.synchronize()
            got, s, o = out.cpu().numpy(), st.cpu().numpy(), att.cpu().numpy()
            for r in range(R):
                if bad and r == 1:
                    with pytest.raises(oracle.OracleError) as e:
                        caches[r].resolve(sels[r], ctx, c.host_pool(r)[0])
                    assert s[r, 2] == e.value.code == hk.HS_ERR_DUP
                    assert (got[r] == -1).all() and np.isnan(o[r]).all()
                    continue
                ref = caches[r].resolve(sels[r], ctx, c.host_pool(r)[0])[0]
                assert s[r, 2] == 0 and np.array_equal(got[r], ref), (t, r)
                o_ref = oracle.attention.sparse_decode_attention(q[r, 0], caches[r].hot, ref, SCALE)
                assert np.abs(o[r] - o_ref).max() <= 2e-3 * np.abs(o_ref).max(), (t, r)
    finally:
        c.close()


@pytest.mark.parametrize("streams", ["two", "one"])
def test_short_requests_cross_into_the_normal_path(streams):
    """Short requests (slot = position) through the fused call, growing by write-through
    appends past B (on a backup stream, or in the append kernel on the compute stream)."""
    w = W["tiny"].scaled(R=2, ctx=200, B=256, k=64, forced_last=16, steps=80, append=True)
    p = Pair(w, fused_heads=16, append_streams=streams)
    try:
        for r in range(w.R):
            hk.hs_admit_short(p.h, r, w.ctx, p.compute.cuda_stream)
            for l in p.anchors:
                p.caches[(r, l)].admit_short(w.ctx, p.ohost[r][l])
        run(p)
    finally:
        p.close()


def test_fp8_records_long():
    """FP8 latent-KV records (656 bytes) through the fused kernel: the codes are turned into
    bf16 in the tile, the scores and P V apply the block scales; the misses staged and copied
    as raw records."""
    w = W["long"].scaled(L=2, steps=4, ctx=32768)
    log("fp8 long L=2")
    p = Pair(w, fused_heads=16, fp8=True)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == 33
        run(p)
    finally:
        p.close()


def test_fp8_records_several_tiles():
    w = W["batched"].scaled(R=32, L=1, steps=3, B=4096)
    log("fp8 batched R=32: 8 workgroups of 5 tiles")
    p = Pair(w, fused_heads=16, fp8=True)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == 8
        run(p)
    finally:
        p.close()


def test_fp8_records_resident_tier_and_ragged():
    """FP8 records from the resident pool and the hot slots, eight requests (two tiles per
    fetch workgroup), k = 1000 (ragged shares)."""
    w = W["long"].scaled(R=8, L=1, ctx=65536, k=1000, steps=4, append=False, force_newest=False)
    log("fp8 R=8 k=1000 with a resident window")
    p = Pair(w, fused_heads=16, fp8=True, resident=ResidentSpec(page_tokens=64, window_tokens=16384,
                                                                old_frac=0.1, spill_every=1, churn=0.05))
    try:
        run(p)
    finally:
        p.close()


def test_fp8_records_shared_layers():
    w = W["shared"].scaled(R=2, L=4, ctx=16384, steps=3)
    log("fp8 shared R=2 L=4")
    p = Pair(w, fused_heads=16, fp8=True)
    try:
        run(p)
        p.check_hot()
    finally:
        p.close()


def test_configuration_without_the_fused_kernel():
    """130 requests x 2 workgroups exceed one wave of workgroups even with one fetch
    workgroup per request: the call makes hs_resolve and hs_sparse_attn, with the same
    results."""
    w = W["tiny"].scaled(R=130, steps=3)
    log("tiny R=130: two calls")
    p = Pair(w, fused_heads=16)
    try:
        run(p, expect_fused=False)
    finally:
        p.close()


@pytest.mark.parametrize("R,k,tiles", [(32, 2048, 5), (8, 2048, 2), (16, 1000, 2), (40, 2048, 7)])
def test_fetch_workgroups_over_several_tiles(R, k, tiles):
    """Fetch workgroups that attend several 64-row tiles with a running maximum, sum and
    output: the batched shape (32 requests, 7 shares of 292-293 entries, the last tile of a
    share partly filled), shares of exactly two tiles, a ragged second tile (125-entry
    shares) and 40 requests (5 shares of 409-410 entries)."""
    w = W["batched"].scaled(R=R, L=1, k=k, B=4096, steps=3)
    S = -(-k // (64 * tiles))
    assert R * (S + 1) <= 256 and (tiles == 1 or R * (-(-k // (64 * (tiles - 1))) + 1) > 256)
    log("batched R=%d k=%d: %d fetch workgroups of %d tiles per request" % (R, k, S, tiles))
    p = Pair(w, fused_heads=16)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == S + 1
        run(p)
    finally:
        p.close()


@pytest.mark.parametrize("fp8", [False, True])
def test_fused_matches_separate_calls(fp8):
    """The same trace through hs_resolve + hs_sparse_attn on one handle and hs_resolve_attn on
    another: identical slots every step, and the same attention output bit for bit (one
    request: both split the list into the same 32 chunks of 64 entries, attend them with the
    same tile functions and merge them with the same function), bf16 or FP8 records."""
    w = W["long"].scaled(L=1, steps=4, ctx=32768)
    a = Pair(w, fused_heads=16, fp8=fp8)
    b = Pair(w, fp8=fp8)
    try:
        q_all = [synth.queries(w.R, w.L, t) for t in range(w.steps)]
        out_b = torch.empty((w.R, 16, 512), dtype=torch.float32, device="cuda")
        for t in range(w.steps):
            a.step_gpu_and_oracle()
            b.step_gpu_and_oracle()
            d_q = torch.from_numpy(q_all[t][:, 0].copy().view(np.int16)).to("cuda")
            hk.hs_sparse_attn(b.h, 0, d_q.data_ptr(), 16, 512, b.d_out[0].data_ptr(), out_b.data_ptr(), SCALE, 0,
                              b.compute.cuda_stream)
            torch.cuda.synchronize()
            assert torch.equal(a.d_out, b.d_out)
            oa, ob = a.d_att[0].cpu().numpy(), out_b.cpu().numpy()
            assert np.array_equal(oa, ob), (t, float(np.abs(oa - ob).max()))
    finally:
        a.close()
        b.close()


def test_graph_capture_replays_match_oracle():
    """hs_resolve_attn of every layer captured once in a HIP graph reading fixed input buffers,
    replayed for 8 steps with eager input copies and unrelated eager work between replays;
    every replay agrees with the oracle."""
    w = W["batched"].scaled(R=4, L=2, ctx=16384)
    steps = 8
    p = Pair(w, steps=steps)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) > 0
        dev = torch.device("cuda")
        s = torch.cuda.Stream()
        sel_buf = torch.empty_like(p.d_trace[0])
        q_all = np.stack([synth.queries(w.R, w.L, t) for t in range(steps)])  # [t][R][L][16][576]
        d_q_all = torch.from_numpy(q_all.view(np.int16)).to(dev).permute(0, 2, 1, 3, 4).contiguous()
        q_buf = torch.empty_like(d_q_all[0])
        ctx = torch.full((w.R,), w.ctx, dtype=torch.int32, device=dev)
        out = torch.empty((w.L, w.R, 16, 512), dtype=torch.float32, device=dev)
        stats = torch.zeros((w.L, w.R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for ai, l in enumerate(p.anchors):
                hk.hs_resolve_attn(p.h, l, sel_buf[ai].data_ptr(), ctx.data_ptr(), p.d_out[ai].data_ptr(),
                                   stats[ai].data_ptr(), 0, 0, q_buf[l].data_ptr(), 16, 512, out[l].data_ptr(),
                                   SCALE, s.cuda_stream)
        torch.cuda.synchronize()
        for t in range(steps):
            sel_buf.copy_(p.d_trace[t])
            q_buf.copy_(d_q_all[t])
            noise = torch.randn(4096, device=dev).sum()  # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.isfinite(noise)
            got, st, o = p.d_out.cpu().numpy(), stats.cpu().numpy(), out.cpu().numpy()
            for ai, l in enumerate(p.anchors):
                for r in range(w.R):
                    ref, hits, misses, _, _ = p.caches[(r, l)].resolve(p.trace[t, ai, r], w.ctx, p.ohost[r][l])
                    assert np.array_equal(got[ai, r], ref), (t, l, r)
                    assert tuple(st[ai, r, :3]) == (hits, misses, 0), (t, l, r)
                    o_ref = oracle.attention.sparse_decode_attention(q_all[t, r, l], p.caches[(r, l)].hot, ref, SCALE)
                    assert np.abs(o[l, r] - o_ref).max() <= 2e-3 * np.abs(o_ref).max(), (t, l, r)
            p.t += 1
        p.check_state()
    finally:
        p.close()


def test_graph_capture_with_write_through_on_the_compute_stream():
    """hs_writeback without a backup stream (one kernel, no event) and hs_resolve_attn of every
    layer captured once in a HIP graph that reads fixed input buffers, replayed for 6 decode
    steps with eager input copies and unrelated eager work between replays; every replay
    agrees with the oracle, and the written-through records reach the host pool."""
    w = W["long"].scaled(R=2, L=2, ctx=16384, steps=6)
    steps = w.steps
    p = Pair(w, steps=steps)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) > 0
        dev = torch.device("cuda")
        s = torch.cuda.Stream()
        sel_buf = torch.empty_like(p.d_trace[0])
        q_all = np.stack([synth.queries(w.R, w.L, t) for t in range(steps)])  # [t][R][L][16][576]
        d_q_all = torch.from_numpy(q_all.view(np.int16)).to(dev).permute(0, 2, 1, 3, 4).contiguous()
        q_buf = torch.empty_like(d_q_all[0])
        recs_all = [synth.records_at(w.R, w.L, [w.ctx + t] * w.R) for t in range(steps)]
        new_buf = torch.empty((w.R, w.L, synth.RECORD_BYTES), dtype=torch.uint8, device=dev)
        pos_buf = torch.empty((w.R,), dtype=torch.int32, device=dev)
        ctx = torch.empty((w.R,), dtype=torch.int32, device=dev)
        out = torch.empty((w.L, w.R, 16, 512), dtype=torch.float32, device=dev)
        stats = torch.zeros((w.L, w.R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            hk.hs_writeback(p.h, new_buf.data_ptr(), pos_buf.data_ptr(), s.cuda_stream, 0)
            for ai, l in enumerate(p.anchors):
                hk.hs_resolve_attn(p.h, l, sel_buf[ai].data_ptr(), ctx.data_ptr(), p.d_out[ai].data_ptr(),
                                   stats[ai].data_ptr(), 0, 0, q_buf[l].data_ptr(), 16, 512, out[l].data_ptr(),
                                   SCALE, s.cuda_stream)
        torch.cuda.synchronize()
        for t in range(steps):
            pos = w.ctx + t
            sel_buf.copy_(p.d_trace[t])
            q_buf.copy_(d_q_all[t])
            new_buf.copy_(torch.from_numpy(recs_all[t]))
            pos_buf.fill_(pos)
            ctx.fill_(pos + 1)
            noise = torch.randn(4096, device=dev).sum()  # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.isfinite(noise)
            got, st, o = p.d_out.cpu().numpy(), stats.cpu().numpy(), out.cpu().numpy()
            for ai, l in enumerate(p.anchors):
                for r in range(w.R):
                    p.caches[(r, l)].append(pos, recs_all[t][r, l], p.ohost[r][l])
                    ref, hits, misses, _, _ = p.caches[(r, l)].resolve(p.trace[t, ai, r], pos + 1, p.ohost[r][l])
                    assert np.array_equal(got[ai, r], ref), (t, l, r)
                    assert tuple(st[ai, r, :3]) == (hits, misses, 0), (t, l, r)
                    o_ref = oracle.attention.sparse_decode_attention(q_all[t, r, l], p.caches[(r, l)].hot, ref, SCALE)
                    assert np.abs(o[l, r] - o_ref).max() <= 2e-3 * np.abs(o_ref).max(), (t, l, r)
            p.t += 1
            p.newest = pos
        p.check_state()
        for t in range(steps):
            for r in range(w.R):
                for l in range(w.L):
                    assert np.array_equal(p.gpu.host_pool(r)[l, w.ctx + t], recs_all[t][r, l]), (t, r, l)
    finally:
        p.close()


def test_several_tiles_with_resident_tier():
    """Eight requests (two tiles per fetch workgroup): resident rows, hot rows and misses
    across tile boundaries."""
    w = W["long"].scaled(R=8, L=1, ctx=65536, steps=4, append=False, force_newest=False)
    log("long R=8 with a resident window: 17 workgroups of 2 tiles")
    p = Pair(w, fused_heads=16, resident=ResidentSpec(page_tokens=64, window_tokens=16384, old_frac=0.1,
                                                      spill_every=1, churn=0.05))
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == 17
        run(p)
    finally:
        p.close()


def test_several_tiles_capacity_blocks():
    w = W["capacity"].scaled(R=8, L=1, ctx=262144, steps=4)
    log("capacity blocks R=8: 17 workgroups of 2 tiles")
    p = Pair(w, fused_heads=16)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == 17
        run(p)
    finally:
        p.close()


def test_several_tiles_shared_layers():
    w = W["shared"].scaled(R=8, L=4, ctx=16384, steps=3)
    log("shared R=8 L=4: anchors with 17 workgroups of 2 tiles")
    p = Pair(w, fused_heads=16)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == 17
        run(p)
        p.check_hot()
    finally:
        p.close()


def test_several_tiles_padded_requests_untouched():
    w = W["batched"].scaled(R=32, L=1, steps=3, B=4096)
    p = Pair(w, fused_heads=16)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == 8
        sentinel = torch.full_like(p.d_att, 7.0)
        p.d_att.copy_(sentinel)
        for _ in range(3):
            p.step_gpu_and_oracle(num_reqs=21)
        torch.cuda.synchronize()
        assert torch.equal(p.d_att[:, 21:], sentinel[:, 21:])
        p.check_state(requests=range(21))
    finally:
        p.close()
