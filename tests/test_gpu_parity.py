"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Slot maps, LRU orders, page tables, hit/miss counts and copied bytes must match
bit for bit; attention within 2e-3 * max|o_ref| per (request, layer) (bf16 in,
fp32 accumulate).
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

W = synth.WORKLOADS


def log(msg):
    print(msg, flush=True)


# ---- worked example of the pages -------------------------------------------------------

def test_example_a_through_the_c_abi(golden):
    """gentlecold.top §3.5, B=8, k=4 walk-through, run on the GPU."""
    g = dict(golden("example_a.txt"))
    B, newest = int(g["B"][0]), int(g["newest"][0])
    toks = [int(x) for x in g["before_tokens"]]
    cfg = hk.make_config(1, 1, 64, 4, B, newest_slot=True)
    c = hk.HiSparse(cfg)
    synth.fill_request(c.host_pool_address(0), 0, 1, 64, newest)
    dev = torch.device("cuda")
    out = torch.empty((1, 4), dtype=torch.int32, device=dev)
    st = torch.zeros((1, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    side = torch.cuda.Stream()

    def resolve(sel, ctx):
        d_sel = torch.tensor([sel], dtype=torch.int32, device=dev)
        d_ctx = torch.tensor([ctx], dtype=torch.int32, device=dev)
        hk.hs_resolve(c.h, 0, d_sel.data_ptr(), d_ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0, 0)
        torch.cuda.synchronize()
        return out.cpu().numpy()[0].tolist(), st.cpu().numpy()[0].tolist()

    resolve(toks[:4], newest)
    resolve(toks[4:], newest)
    rec = torch.from_numpy(synth.records_at(1, 1, [newest])).to(dev)
    pos = torch.tensor([newest], dtype=torch.int32, device=dev)
    hk.hs_writeback(c.h, rec.data_ptr(), pos.data_ptr(), 0, side.cuda_stream)
    slots, stats = resolve([int(x) for x in g["selection"]], newest + 1)
    assert slots == [int(x) for x in g["expect_slots"]]
    assert stats[:3] == [int(g["expect_hits"][0]), int(g["expect_misses"][0]), 0]
    lru = torch.empty((1, B), dtype=torch.int32, device=dev)
    sp = torch.empty((1, B), dtype=torch.int32, device=dev)
    hk.hs_export_state(c.h, 0, sp.data_ptr(), lru.data_ptr(), 0, 0, 0)
    torch.cuda.synchronize()
    assert lru.cpu().numpy()[0].tolist() == [int(x) for x in g["expect_lru"]]
    assert sp.cpu().numpy()[0].tolist() == [25, 11, 12, 13, 14, 15, 16, 17]
    hot = c.hot[0, 0].cpu().numpy()
    assert np.array_equal(hot[0], synth.record(0, 0, 25))   # t25 fetched into s0
    assert np.array_equal(hot[B], synth.record(0, 0, 30))   # newest slot
    torch.cuda.synchronize()
    # write-through reached the host pool
    assert np.array_equal(c.host_pool(0)[0, 30], synth.record(0, 0, 30))
    c.close()


NEWEST_IN_LRU = [([[1, 2], [2, 3], [1, 2]], [None, 2, 2]),
                 ([[0, 1, 2], [2, 4, 5], [5, 0, 2]], [None, 2, 5])]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("seqs,newest,B", [(s, n, B) for s, n in NEWEST_IN_LRU for B in (2, 3, 4, 6)
                                           if B >= len(s[0])])
def test_newest_position_also_in_an_lru_slot(seqs, newest, B, fused):
    """The corner case the pages leave open ("HiSparse 深度解析" (gentlecold.top) §3.4, §5.2
    name the reserved newest slot but not a newest position that an LRU slot already holds):
    a write-through of such a position.  Reading, as in the oracle: slot B serves it and the
    LRU slot holding it counts as not selected (evictable).  Slots, hit/miss counts, slot
    map, LRU order and page table through the C ABI against the oracle after every step; through
    the fused call also the attention over the published slots against float64 attention."""
    k = len(seqs[0])
    U, lmax = 9, 16
    cfg = hk.make_config(1, 1, lmax, k, B, newest_slot=True)
    c = hk.HiSparse(cfg)
    synth.fill_request(c.host_pool_address(0), 0, 1, lmax, lmax)
    host = np.stack([synth.record(0, 0, q) for q in range(lmax)])
    oc = oracle.Cache(B, lmax, synth.RECORD_BYTES, newest_slot=True)
    dev = torch.device("cuda")
    out = torch.empty((1, k), dtype=torch.int32, device=dev)
    st = torch.zeros((1, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    d_ctx = torch.tensor([U], dtype=torch.int32, device=dev)
    sp = torch.empty((1, B), dtype=torch.int32, device=dev)
    lru = torch.empty((1, B), dtype=torch.int32, device=dev)
    pt = torch.empty((1, lmax), dtype=torch.int32, device=dev)
    att = torch.empty((1, 16, 512), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    for t, sel in enumerate(seqs):
        log("newest-in-LRU case B=%d fused=%d step %d sel %s newest %s" % (B, fused, t, sel, newest[t]))
        if newest[t] is not None:
            oc.append(newest[t], host[newest[t]], None)
            rec = torch.from_numpy(synth.records_at(1, 1, [newest[t]])).to(dev)
            pos = torch.tensor([newest[t]], dtype=torch.int32, device=dev)
            hk.hs_writeback(c.h, rec.data_ptr(), pos.data_ptr(), 0, side.cuda_stream)
        o, hits, misses, _, _ = oc.resolve(np.asarray(sel, np.int32), U, host)
        d_sel = torch.tensor([sel], dtype=torch.int32, device=dev)
        if fused:
            q = synth.queries(1, 1, t)[0, 0]
            d_q = torch.from_numpy(q.view(np.int16).copy()).to(dev)
            hk.hs_resolve_attn(c.h, 0, d_sel.data_ptr(), d_ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0,
                               d_q.data_ptr(), 16, 512, att.data_ptr(), SCALE, 0)
        else:
            hk.hs_resolve(c.h, 0, d_sel.data_ptr(), d_ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0, 0)
        hk.hs_export_state(c.h, 0, sp.data_ptr(), lru.data_ptr(), pt.data_ptr(), 0, 0)
        torch.cuda.synchronize()
        stats = st.cpu().numpy()[0].tolist()
        assert out.cpu().numpy()[0].tolist() == o.tolist(), (t, sel)
        assert stats[:3] == [hits, misses, 0], (t, stats)
        e = oc.export()
        assert sp.cpu().numpy()[0].tolist() == e["slot_pos"].tolist(), t
        assert lru.cpu().numpy()[0].tolist() == e["lru"].tolist(), t
        assert pt.cpu().numpy()[0].tolist() == oc.page_table.tolist(), t
        hot = c.hot[0, 0].cpu().numpy()
        for i, s_ in enumerate(o.tolist()):
            assert np.array_equal(hot[s_], host[sel[i]]), (t, i, s_)
        if fused:
            K = oracle.attention.bf16_to_f64(np.ascontiguousarray(host[sel]).view(np.uint16))
            ref = oracle.attention.sparse_decode_attention_rows(q, K, SCALE)
            got = att.cpu().numpy()[0]
            assert np.abs(got - ref).max() <= 2e-3 * np.abs(ref).max(), t
    c.close()


# ---- the workloads ---------------------------------------------------------------------

@pytest.mark.parametrize("B,wgs", [(64, 1), (100, 3), (128, 0), (128, 7), (256, 2)])
def test_tiny_every_step(B, wgs):
    """Tiny workload (1 x 1, ctx 4096, k 64, 32 steps) at several B and workgroup counts:
    slots, counts, slot map, LRU, page table and hot bytes after every step."""
    w = W["tiny"].scaled(B=B)
    log("tiny B=%d wgs=%d" % (B, wgs))
    p = Pair(w, wgs=wgs)
    for _ in range(w.steps):
        p.step_gpu_and_oracle()
        p.check_state()
    p.close()


@pytest.mark.parametrize("streams", ["two", "one"])
def test_long_with_write_through_scaled(streams):
    """Long-request shape (k 2048, B 4096, one token appended and written through per step,
    always selected) on 2 layers and a 16K context, state checked every step; the
    write-through on a backup stream or in the append kernel on the compute stream."""
    w = W["long"].scaled(L=2, ctx=16384, steps=12)
    log("long scaled, write-through on %s stream(s)" % streams)
    p = Pair(w, append_streams=streams)
    for _ in range(w.steps):
        p.step_gpu_and_oracle()
        p.check_state()
    # the appended tokens are on the host, in the pinned pool the GPU wrote
    for t in range(w.steps):
        pos = w.ctx + t
        for l in range(w.L):
            assert np.array_equal(p.gpu.host_pool(0)[l, pos], synth.record(0, l, pos))
    p.close()


def test_write_through_modes_alternating():
    """Write-through alternating between the backup stream and the one-kernel mode every step
    (a one-stream append must wait for a backup that may still read slot B): state checked
    every step, every appended record in the host pool at the end."""
    w = W["long"].scaled(L=2, ctx=8192, steps=10)
    log("write-through modes alternating")
    p = Pair(w)
    for t in range(w.steps):
        p.append_streams = "one" if t % 2 else "two"
        p.step_gpu_and_oracle()
        p.check_state()
    torch.cuda.synchronize()
    for t in range(w.steps):
        pos = w.ctx + t
        for l in range(w.L):
            assert np.array_equal(p.gpu.host_pool(0)[l, pos], synth.record(0, l, pos))
    p.close()


def test_long_full_size():
    """The long-request workload at full size (1 x 8 layers, ctx 131072, k 2048, B 4096) for
    24 steps: every slot vector and count each step, the whole state every 8 steps."""
    w = W["long"]
    log("long full size")
    p = Pair(w, steps=24)
    for t in range(24):
        p.step_gpu_and_oracle()
        if t % 8 == 7:
            p.check_state()
    p.close()


@pytest.mark.parametrize("B", synth.BATCHED_B_SWEEP)
def test_batched_sweep(B):
    """Batched shape: 32 requests resolved in one launch per layer, B in {2048, 4096, 8192};
    2 of the 16 layers, 4 steps."""
    w = W["batched"].scaled(L=2, B=B)
    log("batched B=%d" % B)
    p = Pair(w, steps=4)
    for _ in range(4):
        p.step_gpu_and_oracle()
    p.check_state()
    p.close()


def test_shared_index_prefetch_scaled():
    """Shared-index shape: 8 layers = 2 x (anchor + 3 shared), 4 requests, ctx 16384; the
    shared layers follow the anchor's plan with their own records on a side stream."""
    w = W["shared"].scaled(R=4, L=8, ctx=16384)
    log("shared scaled")
    p = Pair(w, steps=6)
    for _ in range(6):
        p.step_gpu_and_oracle()
        p.check_state()
    p.check_hot(layers=range(w.L))
    p.close()


@pytest.mark.parametrize("R", [1, 3, 40, 1100])
def test_shared_replay_request_counts(R):
    """The replay kernel over one, a few and many requests: up to 1024 requests the launch
    strides over all requests' misses at once; 1100 requests take the per-request split
    (each workgroup takes every grid-th request)."""
    w = W["shared"].scaled(R=R, L=4, ctx=8192, k=256, B=512) if R <= 40 else \
        W["shared"].scaled(R=R, L=4, ctx=512, k=64, B=128)
    log("shared replay R=%d" % R)
    p = Pair(w, steps=5)
    try:
        for _ in range(5):
            p.step_gpu_and_oracle()
        p.check_state()
        p.check_hot(layers=range(w.L))
    finally:
        p.close()


def test_capacity_blocks_scaled():
    """Block-id selections (32 blocks of 64 tokens), recency-Zipf trace, on 2 x 2 caches with
    a 64K context; blocks are expanded in the kernel."""
    w = W["capacity"].scaled(R=2, L=2, ctx=65536)
    log("capacity scaled")
    p = Pair(w, steps=8)
    for _ in range(8):
        p.step_gpu_and_oracle()
        p.check_state()
    p.close()


# ---- semantics at the edges -------------------------------------------------------------

def _single(B=16, k=8, newest=False, lmax=256, wgs=2):
    cfg = hk.make_config(2, 1, lmax, k, B, newest_slot=newest, wgs_per_request=wgs)
    c = hk.HiSparse(cfg)
    for r in range(2):
        synth.fill_request(c.host_pool_address(r), r, 1, lmax, lmax)
    return c


def test_bad_selections_set_error_and_change_nothing():
    dev = torch.device("cuda")
    c = _single()
    out = torch.empty((2, 8), dtype=torch.int32, device=dev)
    st = torch.zeros((2, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    ctx = torch.tensor([200, 200], dtype=torch.int32, device=dev)
    good = torch.tensor([list(range(8)), list(range(50, 58))], dtype=torch.int32, device=dev)
    hk.hs_resolve(c.h, 0, good.data_ptr(), ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0, 0)
    sp0 = torch.empty((2, 16), dtype=torch.int32, device=dev)
    lru0 = torch.empty((2, 16), dtype=torch.int32, device=dev)
    hk.hs_export_state(c.h, 0, sp0.data_ptr(), lru0.data_ptr(), 0, 0, 0)
    bad = torch.tensor([[1, 2, 3, 4, 5, 6, 7, 3], [50, 51, 52, 53, 54, 55, 56, 250]], dtype=torch.int32,
                       device=dev)
    hk.hs_resolve(c.h, 0, bad.data_ptr(), ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0, 0)
    torch.cuda.synchronize()
    s = st.cpu().numpy()
    assert s[0, 2] == hk.HS_ERR_DUP and s[1, 2] == hk.HS_ERR_RANGE
    assert (out.cpu().numpy() == -1).all()
    sp1 = torch.empty_like(sp0)
    lru1 = torch.empty_like(lru0)
    hk.hs_export_state(c.h, 0, sp1.data_ptr(), lru1.data_ptr(), 0, 0, 0)
    torch.cuda.synchronize()
    assert torch.equal(sp0, sp1) and torch.equal(lru0, lru1)
    # the oracle agrees on the error bits
    oc = oracle.Cache(16, 256, 1152)
    with pytest.raises(oracle.OracleError) as e:
        oc.resolve(bad.cpu().numpy()[0], 200, np.zeros((256, 1152), np.uint8))
    assert e.value.code == hk.HS_ERR_DUP
    with pytest.raises(oracle.OracleError) as e:
        oc.resolve(bad.cpu().numpy()[1], 200, np.zeros((256, 1152), np.uint8))
    assert e.value.code == hk.HS_ERR_RANGE
    c.close()


def test_padded_requests_are_untouched():
    """A device request count below R leaves the padded requests exactly as they were
    (gentlecold.top §5.5: padded blocks of a captured batch return early)."""
    w = W["tiny"].scaled(R=3)
    p = Pair(w, wgs=2)
    p.step_gpu_and_oracle()
    for _ in range(4):
        p.step_gpu_and_oracle(num_reqs=2)
    p.check_state(requests=[0, 1])
    # request 2 still has its state after step 1 only
    sp = torch.empty((3, w.B), dtype=torch.int32, device="cuda")
    hk.hs_export_state(p.h, 0, sp.data_ptr(), 0, 0, 0, 0)
    torch.cuda.synchronize()
    oc = oracle.Cache(w.B, p.lmax, 1152)
    oc.resolve(p.trace[0, 0, 2], w.ctx, p.ohost[2][0])
    assert np.array_equal(sp.cpu().numpy()[2], oc.export()["slot_pos"])
    p.close()


@pytest.mark.parametrize("mode", ["resolve", "fused", "rows"])
def test_empty_batch_changes_nothing(mode):
    """A device request count of 0 (a captured batch with every request padded, gentlecold.top
    §5.5) leaves every request as it was, through hs_resolve, hs_resolve_attn and
    hs_resolve_rows, the write-through of that step aside; the steps after it match the
    oracle, which skips that step for every request."""
    w = W["tiny"].scaled(R=3, steps=6, B=192 if mode == "rows" else 128)  # rows: B >= 3 k
    kw = {"fused": {"fused_heads": 16}, "rows": {"rows": 3}}.get(mode, {})
    p = Pair(w, wgs=2, **kw)
    log("empty batch through %s" % mode)
    p.step_gpu_and_oracle()
    p.step_gpu_and_oracle()
    p.step_gpu_and_oracle(num_reqs=0)
    p.check_state()
    for _ in range(3):
        p.step_gpu_and_oracle()
    p.check_state()
    p.close()


def test_skip_io_moves_metadata_not_bytes():
    """The timing aid (gentlecold.top §4.4 no-IO oracle): same metadata, no record bytes."""
    w = W["tiny"]
    a = Pair(w)
    b = Pair(w)
    b.gpu.hot.fill_(0x5A)
    for _ in range(6):
        ra = a.step_gpu_and_oracle()
        rb = b.step_gpu_and_oracle(flags=hk.HS_SKIP_IO)
    a.check_state(hot=True)
    b.check_state(hot=False)
    torch.cuda.synchronize()
    assert (b.gpu.hot.cpu().numpy() == 0x5A).all()
    a.close()
    b.close()


def test_reset_request_returns_to_admission_state():
    w = W["tiny"].scaled(R=2)
    p = Pair(w)
    for _ in range(3):
        p.step_gpu_and_oracle()
    hk.hs_reset_request(p.h, 1, 0)
    sp = torch.empty((2, w.B), dtype=torch.int32, device="cuda")
    lru = torch.empty((2, w.B), dtype=torch.int32, device="cuda")
    hk.hs_export_state(p.h, 0, sp.data_ptr(), lru.data_ptr(), 0, 0, 0)
    torch.cuda.synchronize()
    assert (sp.cpu().numpy()[1] == -1).all()
    assert lru.cpu().numpy()[1].tolist() == list(range(w.B))
    assert np.array_equal(sp.cpu().numpy()[0], p.caches[(0, 0)].export()["slot_pos"])
    p.close()


def test_shared_layer_is_refused_by_resolve():
    cfg = hk.make_config(1, 4, 4096, 64, 128, layer_group=4)
    c = hk.HiSparse(cfg)
    x = torch.zeros((1, 64), dtype=torch.int32, device="cuda")
    with pytest.raises(hk.HsError) as e:
        hk.hs_resolve(c.h, 1, x.data_ptr(), x.data_ptr(), x.data_ptr(), 0, 0, 0, 0)
    assert e.value.code == hk.HS_ESTATE
    c.close()


# ---- the sparse-attention consumer -------------------------------------------------------

def _attn_check(p, step, layers, heads=16):
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
            att = oracle.attention.sparse_decode_attention_fp8 if p.fp8 else oracle.attention.sparse_decode_attention
            ref = att(q[r, l], hot, slots[r], SCALE)
            err = np.abs(o[r] - ref).max() / np.abs(ref).max()
            worst = max(worst, err)
            assert err <= 2e-3, (r, l, err)
    return worst


def test_attention_batched():
    w = W["batched"].scaled(L=2)
    p = Pair(w, steps=2)
    for t in range(2):
        p.step_gpu_and_oracle()
        worst = _attn_check(p, t, range(w.L))
    log("attention batched worst rel err %.2e" % worst)
    p.close()


def test_attention_single_request_and_shared_layers():
    w = W["shared"].scaled(R=2, L=4, ctx=16384)
    p = Pair(w, steps=2)
    for t in range(2):
        p.step_gpu_and_oracle()
        worst = _attn_check(p, t, range(w.L))
    log("attention shared worst rel err %.2e" % worst)
    p.close()


@pytest.mark.parametrize("k,heads,fp8", [(64, 16, False), (100, 5, False), (1000, 16, False), (65, 3, False),
                                        (65, 3, True), (1000, 16, True)])
def test_attention_ragged(k, heads, fp8):
    """Entry counts that leave a ragged last tile (k = 65: a chunk with one entry), and fewer
    than 16 heads; bf16 and FP8 records."""
    w = W["tiny"].scaled(k=k, B=max(128, k + 40), R=3, forced_last=min(16, k))
    p = Pair(w, steps=3, fp8=fp8)
    for t in range(3):
        p.step_gpu_and_oracle()
        _attn_check(p, t, [0], heads=heads)
    p.close()


def test_duplicates_in_many_patterns_then_valid_steps():
    """Duplicate and out-of-range entries in varied places (home-bucket contests, the
    compare-and-swap fallback, the newest slot); every request's error bits match the
    oracle, nothing changes, and later valid steps still agree with the oracle."""
    R, k, B, lmax = 8, 256, 512, 8192
    cfg = hk.make_config(R, 1, lmax, k, B, newest_slot=True, wgs_per_request=3)
    c = hk.HiSparse(cfg)
    for r in range(R):
        synth.fill_request(c.host_pool_address(r), r, 1, lmax, lmax)
    caches = [oracle.Cache(B, lmax, 1152, newest_slot=True) for _ in range(R)]
    dev = torch.device("cuda")
    out = torch.empty((R, k), dtype=torch.int32, device=dev)
    st = torch.zeros((R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    side = torch.cuda.Stream()
    rng = np.random.default_rng(5)
    ctx = 6000
    d_ctx = torch.full((R,), ctx, dtype=torch.int32, device=dev)

    def step(sels, newest=None):
        if newest is not None:
            recs = synth.records_at(R, 1, [newest] * R)
            d_new = torch.from_numpy(recs).to(dev)
            d_pos = torch.full((R,), newest, dtype=torch.int32, device=dev)
            hk.hs_writeback(c.h, d_new.data_ptr(), d_pos.data_ptr(), 0, side.cuda_stream)
            for r in range(R):
                caches[r].append(newest, recs[r, 0], None)
        d_sel = torch.from_numpy(np.stack(sels).astype(np.int32)).to(dev)
        hk.hs_resolve(c.h, 0, d_sel.data_ptr(), d_ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0, 0)
        torch.cuda.synchronize()
        got, s = out.cpu().numpy(), st.cpu().numpy()
        for r in range(R):
            try:
                ref = caches[r].resolve(sels[r], ctx, c.host_pool(r)[0])[0]
                assert s[r, 2] == 0 and np.array_equal(got[r], ref), r
            except oracle.OracleError as e:
                assert s[r, 2] == e.code, (r, s[r], e.code)
                assert (got[r] == -1).all()
        sp = torch.empty((R, B), dtype=torch.int32, device=dev)
        lru = torch.empty((R, B), dtype=torch.int32, device=dev)
        hk.hs_export_state(c.h, 0, sp.data_ptr(), lru.data_ptr(), 0, 0, 0)
        torch.cuda.synchronize()
        for r in range(R):
            ex = caches[r].export()
            assert np.array_equal(sp.cpu().numpy()[r], ex["slot_pos"]) and \
                np.array_equal(lru.cpu().numpy()[r], ex["lru"]), r

    def fresh():
        return [rng.choice(ctx - 1, size=k, replace=False) for _ in range(R)]

    step(fresh())
    for trial in range(6):
        sels = fresh()
        for r in range(R):
            kind = (trial + r) % 5
            if kind == 0:   # one pair
                a, b = rng.choice(k, 2, replace=False)
                sels[r][b] = sels[r][a]
            elif kind == 1:  # a triple
                a, b, d = rng.choice(k, 3, replace=False)
                sels[r][b] = sels[r][d] = sels[r][a]
            elif kind == 2:  # many pairs
                idx = rng.choice(k, 40, replace=False)
                sels[r][idx[20:]] = sels[r][idx[:20]]
            elif kind == 3:  # out of range
                sels[r][rng.integers(k)] = ctx + 5
            # kind 4: valid
        step(sels)
        step(fresh())
    # the newest position selected twice is a duplicate too
    sels = fresh()
    for r in range(R):
        sels[r][0] = sels[r][1] = ctx - 1
    step(sels, newest=ctx - 1)
    step(fresh())
    c.close()


@pytest.mark.parametrize("B,k,keep,wgs", [(12000, 512, 0.85, 2), (16384, 2048, 0.85, 2), (16384, 8192, 0.5, 0),
                                          (4096, 4096, 0.6, 0), (6000, 3000, 0.6, 0)])
def test_large_lists_and_buffers(B, k, keep, wgs):
    """Large buffers and lists in the kernel's blocked layout: B = 12000 (12 slots per thread),
    B = 16384 (16 slots per thread) with 2 and 8 list entries per thread (B = 16384 and
    top_k = 8192 are the largest the library takes on this device), and lists of 4096 and 3000
    entries (4 per thread) into B = 4096 and 6000.  The list of 8192 fills its buffer at
    the third step and then evicts (with the default 32 workgroups per request: at 2, each
    wave's miss list would have to hold half the list, more LDS than a workgroup has); so do
    the lists of 4096 and 3000.  State compared after every step."""
    w = W["tiny"].scaled(B=B, k=k, ctx=65536, steps=6, R=2, keep_p=keep)
    p = Pair(w, wgs=wgs)
    for _ in range(w.steps):
        p.step_gpu_and_oracle()
        p.check_state()
    if k >= 3000:
        assert p.evicted > 0, p.evicted
    log("B=%d k=%d: occupied slots evicted %d" % (B, k, p.evicted))
    p.close()


@pytest.mark.parametrize("k", [8256, 16384])
def test_top_k_beyond_the_lds_is_refused(k):
    """A top_k whose RESOLVE tables do not fit a workgroup's 160 KB of LDS (above 8192) is
    refused by hs_create with HS_EINVAL and a message naming the bytes; nothing is launched."""
    cfg = hk.make_config(1, 1, 65536, k, 16384)
    with pytest.raises(hk.HsError) as e:
        hk.HiSparse(cfg)
    assert e.value.code == hk.HS_EINVAL and "LDS" in str(e.value), str(e.value)


def test_graph_capture_replays_match_oracle():
    """RESOLVE + attention of every layer captured once in a HIP graph that reads fixed input
    buffers (the pages run the kernel inside the decode CUDA graph, gentlecold.top §3.5), then
    replayed for 8 steps with eager input copies and unrelated eager work between replays;
    every replay agrees with the oracle."""
    w = W["batched"].scaled(R=4, L=2, ctx=16384)
    steps = 8
    p = Pair(w, steps=steps)
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
            hk.hs_resolve(p.h, l, sel_buf[ai].data_ptr(), ctx.data_ptr(), p.d_out[ai].data_ptr(),
                          stats[ai].data_ptr(), 0, 0, s.cuda_stream)
            hk.hs_sparse_attn(p.h, l, q_buf[l].data_ptr(), 16, 512, p.d_out[ai].data_ptr(),
                              out[l].data_ptr(), SCALE, 0, s.cuda_stream)
    torch.cuda.synchronize()
    for t in range(steps):
        sel_buf.copy_(p.d_trace[t])
        q_buf.copy_(d_q_all[t])
        noise = torch.randn(4096, device=dev).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        got = p.d_out.cpu().numpy()
        st = stats.cpu().numpy()
        o = out.cpu().numpy()
        for ai, l in enumerate(p.anchors):
            for r in range(w.R):
                ref, hits, misses, _, _ = p.caches[(r, l)].resolve(p.trace[t, ai, r], w.ctx, p.ohost[r][l])
                assert np.array_equal(got[ai, r], ref), (t, l, r)
                assert tuple(st[ai, r, :3]) == (hits, misses, 0), (t, l, r)
                o_ref = oracle.attention.sparse_decode_attention(q_all[t, r, l], p.caches[(r, l)].hot, ref, SCALE)
                assert np.abs(o[l, r] - o_ref).max() <= 2e-3 * np.abs(o_ref).max(), (t, l, r)
        p.t += 1
    p.check_state()
    p.close()
