"""A resolve workgroup that reads the page table after its launch's workgroup 0 has published.

The workgroups of one resolve launch do not wait for each other, and workgroup 0 updates
the page table in place while its siblings may still be reading it.  A sibling that starts
late therefore sees the entries of this launch's misses already set.  These tests put every
workgroup of a launch in that position, deterministically: the launch is run once, the
metadata is restored to its state before the launch except for the page table, which keeps
what the launch wrote, the hot buffer is restored (so the victim slots hold the evicted
records again), and the same launch is run again.  Both runs must agree byte for byte: slots,
counts, the whole workspace and the hot buffer.

(The fused call, hs_resolve_attn, does not write the page table while its resolve kernel
runs: its second kernel applies the updates, so no workgroup of the fused kernel can meet
an entry of its own launch.)
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu]

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import hierarchical_kv_cache_amd as hk  # noqa: E402
import synth  # noqa: E402
from harness import Pair, SCALE  # noqa: E402

W = synth.WORKLOADS


def log(msg):
    print(msg, flush=True)


def replay_with_published_page_table(p: Pair, t0: int):
    """Runs steps 0..t0 (checked against the oracle), then re-runs step t0 as described above
    (through hs_resolve_attn when the pair drives the fused call)."""
    w = p.w
    for _ in range(t0):
        p.step_gpu_and_oracle()
    ws, hot = p.gpu.workspace, p.gpu.hot
    torch.cuda.synchronize()
    ws0, hot0 = ws.clone(), hot.clone()
    p.t = t0
    res = p.step_gpu_and_oracle()
    misses = sum(int(v[2]) for v in res.values())
    torch.cuda.synchronize()
    out1, stats1 = p.d_out.clone(), p.d_stats.clone()
    ws1, hot1 = ws.clone(), hot.clone()
    # the metadata as it was before the launch, with the page tables the launch wrote
    ws.copy_(ws0)
    for l in p.anchors:
        off = hk.hs_page_table(p.h, l) - ws.data_ptr()
        n = w.R * p.lmax * 8
        ws[off:off + n].copy_(ws1[off:off + n])
    hot.copy_(hot0)
    torch.cuda.synchronize()
    out2 = torch.full_like(p.d_out, -7)
    stats2 = torch.full_like(p.d_stats, -7)
    d_ctx = torch.full((w.R,), p.w.ctx, dtype=torch.int32, device=p.dev)
    if p.fused_heads:
        att1 = p.d_att.clone()
        q = synth.queries(w.R, w.L, t0, heads=p.fused_heads)
        d_q = torch.from_numpy(q.view(np.int16)).to(p.dev)
        att2 = torch.full_like(p.d_att, -7.0)
    for ai, l in enumerate(p.anchors):
        fl = hk.HS_RECORD_PLAN if w.group > 1 else 0
        if p.fused_heads:
            dq = d_q[:, l].contiguous()
            hk.hs_resolve_attn(p.h, l, p.d_trace[t0, ai].data_ptr(), d_ctx.data_ptr(), out2[ai].data_ptr(),
                               stats2.data_ptr(), 0, fl, dq.data_ptr(), p.fused_heads, 512, att2[ai].data_ptr(),
                               SCALE, p.compute.cuda_stream)
            torch.cuda.synchronize()
        else:
            hk.hs_resolve(p.h, l, p.d_trace[t0, ai].data_ptr(), d_ctx.data_ptr(), out2[ai].data_ptr(),
                          stats2.data_ptr(), 0, fl, p.compute.cuda_stream)
        if ai == len(p.anchors) - 1:
            assert torch.equal(stats2, stats1), (stats2.cpu().numpy(), stats1.cpu().numpy())
    torch.cuda.synchronize()
    assert torch.equal(out2, out1)
    if p.fused_heads:  # the same records in the same order: the same attention, bit for bit
        assert torch.equal(att2, att1)
    assert int(stats1[:, 2].abs().sum()) == 0
    assert torch.equal(ws, ws1), "workspace differs from the first run"
    assert torch.equal(hot, hot1), "hot buffer differs from the first run"
    p.check_state()
    return misses


@pytest.mark.parametrize("wgs", [1, 4, 32])
@pytest.mark.parametrize("t0", [0, 6])
def test_tiny_published_page_table(wgs, t0):
    w = W["tiny"].scaled(R=3, steps=8)
    log("tiny R=3 wgs=%d t0=%d" % (wgs, t0))
    p = Pair(w, wgs=wgs)
    try:
        misses = replay_with_published_page_table(p, t0)
        assert misses > 0
    finally:
        p.close()


def test_batched_published_page_table():
    w = W["batched"].scaled(R=4, L=2, steps=3, B=4096)
    log("batched R=4 L=2 B=4096 t0=2")
    p = Pair(w)
    try:
        assert replay_with_published_page_table(p, 2) > 0
    finally:
        p.close()


def test_capacity_blocks_published_page_table():
    w = W["capacity"].scaled(R=2, L=1, ctx=65536, steps=3)
    log("capacity blocks R=2 ctx=65536 t0=2")
    p = Pair(w)
    try:
        assert replay_with_published_page_table(p, 2) > 0
    finally:
        p.close()

