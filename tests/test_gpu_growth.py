"""On-demand growth of the device buffer (HS_CFG_HOT_ON_DEMAND) on the GPU, through the C ABI.

"HiSparse 深度解析" (gentlecold.top) §5.4: the device buffer grows as a short request grows
(_grow_device_buffers), so it does not hold all B slots from the start; §5.3: a request longer
than B holds the full B.  Short requests are admitted at different lengths into a hot buffer
with no device memory behind it, grown ahead of their appends, and carried across B; every step
is compared bit for bit with the oracle (which has no notion of growth: growth must not change
any result), the attention within 2e-3 of float64, and the device memory behind the buffer
with oracle.growth after every growth.  Then the capacity errors: a short request whose context
outgrew its capacity and a request on the normal path before all B slots are backed get
HS_ERR_CAPACITY and change nothing.  (The error cases keep every slot they could touch backed by
device memory: a capacity one below B, or a short capacity whose 64 KiB chunks reach past the
slots in question.)
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu]

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import hierarchical_kv_cache_amd as hk  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402
from oracle import growth  # noqa: E402

CHUNK = 1 << 16
SCALE = 576 ** -0.5
REC = 1152


def log(msg):
    print(msg, file=sys.stderr, flush=True)


_hip = ctypes.CDLL("libamdhip64.so")
_hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
_hip.hipMemcpy.restype = ctypes.c_int


def read_slots(c, r, l, slots, B, L):
    """Records of the given (backed) slots of (r, l), copied device to host one by one."""
    out = np.empty((len(slots), REC), np.uint8)
    for n, s in enumerate(slots):
        addr = c.hot_address + ((r * L + l) * (B + 1) + int(s)) * REC
        assert _hip.hipMemcpy(out[n].ctypes.data, addr, REC, 2) == 0  # device to host
    return out


def export(c, l, R, B, lmax):
    sp = torch.empty((R, B), dtype=torch.int32, device="cuda")
    lru = torch.empty((R, B), dtype=torch.int32, device="cuda")
    pt = torch.empty((R, lmax), dtype=torch.int32, device="cuda")
    nw = torch.empty((R,), dtype=torch.int32, device="cuda")
    hk.hs_export_state(c.h, l, sp.data_ptr(), lru.data_ptr(), pt.data_ptr(), nw.data_ptr(), 0)
    torch.cuda.synchronize()
    return sp.cpu().numpy(), lru.cpu().numpy(), pt.cpu().numpy(), nw.cpu().numpy()


def attention_ref(q, ohost_l, sel):
    K = oracle.attention.bf16_to_f64(np.ascontiguousarray(ohost_l[sel.astype(np.int64)]).view(np.uint16))
    return oracle.attention.sparse_decode_attention_rows(q, K, SCALE)


def test_hot_buffer_grows_with_short_requests():
    R, L, B, k, heads = 3, 2, 1024, 64, 4
    ctx0 = [950, 1000, 70]  # requests 0 and 1 cross B during the run, request 2 stays short
    steps = 130
    lmax = max(ctx0) + steps + 1
    cfg = hk.make_config(R, L, lmax, k, B, newest_slot=True, wgs_per_request=3, hot_on_demand=True)
    c = hk.HiSparse(cfg)
    assert c.hot is None and c.hot_address != 0
    assert hk.hs_hot_backed_bytes(c.h) == 0
    for r in range(R):
        synth.fill_request(c.host_pool_address(r), r, L, lmax, ctx0[r])
    ohost = [np.empty((L, lmax, REC), np.uint8) for _ in range(R)]
    for r in range(R):
        synth.fill_request(ohost[r], r, L, lmax, ctx0[r])
    caches = {(r, l): oracle.Cache(B, lmax, REC, newest_slot=True) for r in range(R) for l in range(L)}
    caps = {}
    cs = torch.cuda.current_stream().cuda_stream

    def grow(r, slots):
        hk.hs_grow_request(c.h, r, slots, cs)
        caps[r] = max(caps.get(r, 0), slots)
        want = growth.backed_bytes(caps, L, B, REC, CHUNK)
        got = hk.hs_hot_backed_bytes(c.h)
        assert got == want, ("backed bytes", r, slots, got, want)

    with pytest.raises(hk.HsError):  # admission needs the slots backed first
        hk.hs_admit_short(c.h, 0, ctx0[0], cs)
    for r in range(R):
        grow(r, min(B, (ctx0[r] + 1 + 31) // 32 * 32))
        hk.hs_admit_short(c.h, r, ctx0[r], cs)
        for l in range(L):
            caches[(r, l)].admit_short(ctx0[r], ohost[r][l])
    full = -(-R * L * (B + 1) * REC // CHUNK) * CHUNK
    log("backed after admission: %d of %d bytes" % (hk.hs_hot_backed_bytes(c.h), full))
    assert hk.hs_hot_backed_bytes(c.h) < full

    rng = np.random.default_rng(11)
    dev = torch.device("cuda")
    out = torch.empty((L, R, k), dtype=torch.int32, device=dev)
    st = torch.zeros((L, R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    att = torch.empty((L, R, heads, 512), dtype=torch.float32, device=dev)
    ctx = list(ctx0)
    fast = slow = grows = 0
    worst = 0.0
    for t in range(steps):
        # grow ahead of the append: position ctx[r] needs slot ctx[r] while short, all B after
        for r in range(R):
            need = min(B, ctx[r] + 1)
            if need > caps[r]:
                grow(r, min(B, max(need, caps[r] + 32)))
                grows += 1
        pos = np.array(ctx, np.int32)
        recs = synth.records_at(R, L, pos)
        d_new, d_pos = torch.from_numpy(recs).to(dev), torch.from_numpy(pos).to(dev)
        hk.hs_writeback(c.h, d_new.data_ptr(), d_pos.data_ptr(), cs, cs)
        for r in range(R):
            for l in range(L):
                caches[(r, l)].append(int(pos[r]), recs[r, l], ohost[r][l])
            ctx[r] += 1
        sel = np.empty((L, R, k), np.int32)
        for l in range(L):
            for r in range(R):
                row = np.concatenate([[ctx[r] - 1], rng.choice(ctx[r] - 1, size=k - 1, replace=False)])
                sel[l, r] = rng.permutation(row)
        d_ctx = torch.tensor(ctx, dtype=torch.int32, device=dev)
        d_sel = torch.from_numpy(sel).to(dev)
        q = synth.queries(R, L, t, heads=heads)
        d_q = torch.from_numpy(q.view(np.int16)).to(dev).permute(1, 0, 2, 3).contiguous()  # [L][R][H][576]
        # layer 0 through the fused call, layer 1 through the two calls
        hk.hs_resolve_attn(c.h, 0, d_sel[0].data_ptr(), d_ctx.data_ptr(), out[0].data_ptr(), st[0].data_ptr(), 0, 0,
                           d_q[0].data_ptr(), heads, 512, att[0].data_ptr(), SCALE, cs)
        hk.hs_resolve(c.h, 1, d_sel[1].data_ptr(), d_ctx.data_ptr(), out[1].data_ptr(), st[1].data_ptr(), 0, 0, cs)
        hk.hs_sparse_attn(c.h, 1, d_q[1].data_ptr(), heads, 512, out[1].data_ptr(), att[1].data_ptr(), SCALE, 0, cs)
        torch.cuda.synchronize()
        got, s, a = out.cpu().numpy(), st.cpu().numpy(), att.cpu().numpy()
        for l in range(L):
            for r in range(R):
                o, hh, mm, _, _ = caches[(r, l)].resolve(sel[l, r], ctx[r], ohost[r][l])
                assert s[l, r, 2] == 0 and s[l, r, 0] == hh and s[l, r, 1] == mm, (t, l, r, s[l, r], hh, mm)
                assert np.array_equal(got[l, r], o), (t, l, r)
                ref = attention_ref(q[r, l], ohost[r][l], sel[l, r])
                err = np.abs(a[l, r] - ref).max() / np.abs(ref).max()
                worst = max(worst, err)
                assert err <= 2e-3, (t, l, r, err)
                if ctx[r] <= B:
                    fast += 1
                else:
                    slow += 1
    log("growth: %d fast-path and %d normal resolves, %d growths, worst attention %.2e, backed %d of %d bytes"
        % (fast, slow, grows, worst, hk.hs_hot_backed_bytes(c.h), full))
    assert fast > 0 and slow > 0 and grows > 0
    # request 2 never needed all B slots: its layers' unused chunks hold no device memory
    assert caps[2] < B // 4 and hk.hs_hot_backed_bytes(c.h) < full * 0.8
    for l in range(L):
        sp, lru, pt, nw = export(c, l, R, B, lmax)
        for r in range(R):
            e = caches[(r, l)].export()
            assert np.array_equal(sp[r], e["slot_pos"]) and np.array_equal(lru[r], e["lru"]), (l, r)
            assert nw[r] == e["newest_pos"] and np.array_equal(pt[r], caches[(r, l)].page_table), (l, r)
            occ = np.nonzero(e["slot_pos"] >= 0)[0]
            assert occ.max() < caps[r]  # only backed slots hold positions
            assert np.array_equal(read_slots(c, r, l, occ, B, L), caches[(r, l)].hot[occ]), (l, r)
    c.close()


def test_capacity_errors_change_nothing():
    """A short request whose context outgrew its capacity, and a request on the normal path whose
    capacity is one below B, get HS_ERR_CAPACITY (NaN attention rows through the fused call) and
    change nothing; the other request is unaffected; once grown, the normal path runs and equals
    the oracle."""
    R, L, B, k, lmax, heads = 2, 1, 256, 32, 1024, 2
    cfg = hk.make_config(R, L, lmax, k, B, newest_slot=True, wgs_per_request=2, hot_on_demand=True)
    c = hk.HiSparse(cfg)
    for r in range(R):
        synth.fill_request(c.host_pool_address(r), r, L, lmax, lmax)
    ohost = [np.empty((L, lmax, REC), np.uint8) for _ in range(R)]
    for r in range(R):
        synth.fill_request(ohost[r], r, L, lmax, lmax)
    cs = torch.cuda.current_stream().cuda_stream
    dev = torch.device("cuda")
    # request 0: short, 100 tokens, capacity 100 (its chunks back slots up to 113)
    hk.hs_grow_request(c.h, 0, 100, cs)
    hk.hs_admit_short(c.h, 0, 100, cs)
    # request 1: on the normal path from the start, capacity B - 1 (its chunks back every slot)
    hk.hs_grow_request(c.h, 1, B - 1, cs)
    # one append each: request 0's position 100 lies past its capacity (only slot B and the host
    # pool take it); request 1's newest token is position 900
    pos = np.array([100, 900], np.int32)
    recs = synth.records_at(R, L, pos)
    hk.hs_writeback(c.h, torch.from_numpy(recs).to(dev).data_ptr(), torch.from_numpy(pos).to(dev).data_ptr(), cs, cs)
    torch.cuda.synchronize()
    before = export(c, 0, R, B, lmax)
    ctx = torch.tensor([101, 901], dtype=torch.int32, device=dev)
    rng = np.random.default_rng(3)
    sel = np.stack([rng.permutation(np.concatenate([[100], rng.choice(100, k - 1, replace=False)])),
                    rng.permutation(np.concatenate([[900], rng.choice(900, k - 1, replace=False)]))]).astype(np.int32)
    d_sel = torch.from_numpy(sel).to(dev)
    out = torch.empty((R, k), dtype=torch.int32, device=dev)
    st = torch.zeros((R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    q = torch.from_numpy(synth.queries(R, 1, 0, heads=heads)[:, 0].view(np.int16)).to(dev)
    att = torch.empty((R, heads, 512), dtype=torch.float32, device=dev)
    for fused in (False, True):
        if fused:
            hk.hs_resolve_attn(c.h, 0, d_sel.data_ptr(), ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0,
                               q.data_ptr(), heads, 512, att.data_ptr(), SCALE, cs)
        else:
            hk.hs_resolve(c.h, 0, d_sel.data_ptr(), ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0, cs)
        torch.cuda.synchronize()
        s, o = st.cpu().numpy(), out.cpu().numpy()
        assert s[0, 2] == hk.HS_ERR_CAPACITY and s[1, 2] == hk.HS_ERR_CAPACITY, s
        assert (o == -1).all()
        if fused:
            assert torch.isnan(att).all()
        after = export(c, 0, R, B, lmax)
        assert all(np.array_equal(x, y) for x, y in zip(before, after))
    # request 1 grown to B: the normal path runs and matches the oracle's first step
    hk.hs_grow_request(c.h, 1, B, cs)
    hk.hs_resolve(c.h, 0, d_sel.data_ptr(), ctx.data_ptr(), out.data_ptr(), st.data_ptr(), 0, 0, cs)
    torch.cuda.synchronize()
    s, o = st.cpu().numpy(), out.cpu().numpy()
    oc = oracle.Cache(B, lmax, REC, newest_slot=True)
    oc.append(900, recs[1, 0], ohost[1][0])
    ref, hh, mm, _, _ = oc.resolve(sel[1], 901, ohost[1][0])
    assert s[1, 2] == 0 and s[1, 0] == hh and s[1, 1] == mm and np.array_equal(o[1], ref)
    assert s[0, 2] == hk.HS_ERR_CAPACITY  # request 0 is still past its capacity
    c.close()
