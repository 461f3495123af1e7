"""RESOLVE past the buffer-fill point, at the shapes the decode step runs: every step's misses
beyond the empty slots evict slots that hold positions ("HiSparse 深度解析" (gentlecold.top)
§3.3: victims are the least recent slots not selected now; §3.5 worked example).

Each test runs long enough that the hot buffer fills and then keeps running, asserts that
occupied slots were evicted (counted from the oracle's misses: empty slots are taken first,
so a step with m misses and e empty slots evicts max(0, m - e) occupied ones), and compares
with the oracle: slots and counts (and bytes_fetched) every step, the attention output of the
fused call every step, the slot map, LRU order, page table and hot bytes at the checkpoints.
"""
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu]

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import hierarchical_kv_cache_amd as hk  # noqa: E402
import synth  # noqa: E402
from harness import Pair  # noqa: E402

W = synth.WORKLOADS


def log(msg):
    print(msg, flush=True)


def drive(p: Pair, steps: int, check_at=(), every_step_state=False, hot_requests=None, hot_layers=None):
    t0 = time.time()
    for i in range(steps):
        p.step_gpu_and_oracle()
        if every_step_state or (i + 1) in check_at:
            p.check_state(hot=False)
            p.check_hot(layers=hot_layers, requests=hot_requests)
    first = min(p.evicted_at) + 1 if p.evicted_at else None
    log("  %d steps in %.1f s; occupied slots evicted: %d (first at step %s, in %d steps); worst attention %.2e"
        % (steps, time.time() - t0, p.evicted, first, len(p.evicted_at), p.worst_attn))
    return first


def test_fused_long_full_shape_past_fill():
    """hs_resolve_attn at the long request's full shape (1 x 8 layers, ctx 131072, k 2048,
    B 4096, 16 heads, the write-through in the append kernel), 28 steps: the buffer fills at
    about step 9, so 19 steps evict through the fused kernel and its finish kernel."""
    w = W["long"]
    log("fused long 1x8 B=4096, 28 steps")
    p = Pair(w, steps=28, fused_heads=16, append_streams="one")
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == 33
        first = drive(p, 28, check_at=(12, 20, 28))
        assert p.evicted > 0 and first is not None and 28 - first >= 15, (p.evicted, first)
    finally:
        p.close()


def test_fused_batched_past_fill():
    """hs_resolve_attn at 32 requests (k 2048, B 4096, 16 heads: 7 fetch workgroups of 5
    tiles per request), 2 of the 16 layers, 20 steps: the buffers fill at about step 10."""
    w = W["batched"].scaled(L=2, B=4096)
    log("fused batched 32x2 B=4096, 20 steps")
    p = Pair(w, steps=20, fused_heads=16)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) == 8
        first = drive(p, 20, check_at=(12, 20), hot_requests=[0, 13, 31])
        assert p.evicted > 0 and first is not None and 20 - first >= 6, (p.evicted, first)
    finally:
        p.close()


def test_fused_fp8_past_fill():
    """hs_resolve_attn with FP8 records (656 bytes: the fused kernel's FP8 tiles, the staged raw
    records and the finish kernel's copies of them) at the long request's shape (k 2048, B 4096,
    2 of the 8 layers, write-through) and at 32 requests (one layer), past the buffer-fill point:
    24 and 20 steps, the state at checkpoints and the attention every step."""
    for w, steps, label in ((W["long"].scaled(L=2), 24, "fp8 fused long 1x2"),
                            (W["batched"].scaled(L=1, B=4096), 20, "fp8 fused batched 32x1")):
        log("%s B=4096, %d steps" % (label, steps))
        p = Pair(w, steps=steps, fused_heads=16, fp8=True)
        try:
            assert hk.hs_resolve_attn_wgs(p.h) > 0
            first = drive(p, steps, check_at=(12, steps), hot_requests=[0, w.R - 1])
            assert p.evicted > 0 and first is not None and steps - first >= 6, (p.evicted, first)
        finally:
            p.close()


def test_fused_batched_b8192_past_fill():
    """hs_resolve_attn at 32 requests with B 8192 (8 slots per thread in the resolving
    workgroup), one layer, 36 steps: the buffers fill at about step 28."""
    w = W["batched"].scaled(L=1, B=8192)
    log("fused batched 32x1 B=8192, 36 steps")
    p = Pair(w, steps=36, fused_heads=16)
    try:
        assert hk.hs_resolve_attn_wgs(p.h) > 0
        first = drive(p, 36, check_at=(30, 36), hot_requests=[0, 7, 31])
        assert p.evicted > 0 and first is not None and 36 - first >= 4, (p.evicted, first)
    finally:
        p.close()


@pytest.mark.parametrize("fused", [False, True])
def test_eight_slots_per_thread_every_step(fused):
    """B = 5120 (8 slots per thread), k 2048, 2 requests, reuse 0.5 so that about 1000 entries
    miss per step and the buffers fill at step 4; 14 steps, the slot map, LRU order, page table
    and hot bytes compared after every step, through hs_resolve and through hs_resolve_attn."""
    w = W["batched"].scaled(R=2, L=1, B=5120, keep_p=0.5)
    log("B=5120 R=2 keep 0.5, %s" % ("hs_resolve_attn" if fused else "hs_resolve"))
    p = Pair(w, steps=14, fused_heads=16 if fused else 0)
    try:
        first = drive(p, 14, every_step_state=True)
        assert p.evicted > 0 and first is not None and first <= 6, (p.evicted, first)
    finally:
        p.close()


@pytest.mark.parametrize("B", [2052, 3000, 3002])
@pytest.mark.parametrize("fused", [False, True])
def test_four_slots_per_thread_partial_tail(B, fused):
    """4 slots per thread where the last threads' runs of slots lie past B (B = 2052 and 3000:
    every thread loads a whole 16-byte group of the slot map and LRU order, the ones past the end
    reading the last group and ignoring it; B = 3002, not a multiple of 4: element loads), k 2048,
    2 requests, reuse 0.5, the state after every step for 10 steps past the buffer-fill point,
    through hs_resolve and hs_resolve_attn."""
    w = W["batched"].scaled(R=2, L=1, B=B, keep_p=0.5)
    log("B=%d R=2 keep 0.5, %s" % (B, "hs_resolve_attn" if fused else "hs_resolve"))
    p = Pair(w, steps=10, fused_heads=16 if fused else 0)
    try:
        first = drive(p, 10, every_step_state=True)
        assert p.evicted > 0 and first is not None and first <= 4, (p.evicted, first)
    finally:
        p.close()


def test_rows_sixteen_slots_per_thread_past_fill():
    """hs_resolve_rows: 4 verification rows of k 2048 into B = 10240 slots (16 slots per
    thread, the union of about 2650 positions resolved as one list), the long request with
    write-through, 2 layers, 18 steps: the buffers fill at about step 11."""
    w = W["long"].scaled(B=10240, L=2)
    log("rows=4 B=10240 1x2, 18 steps")
    p = Pair(w, steps=18, rows=4)
    try:
        first = drive(p, 18, check_at=(12, 18))
        assert p.evicted > 0 and first is not None and 18 - first >= 4, (p.evicted, first)
    finally:
        p.close()


def test_rows_eight_slots_per_thread_every_step():
    """hs_resolve_rows: 2 rows of k 2048 into B = 5120 (8 slots per thread), reuse 0.6, the
    state compared after every step for 12 steps."""
    w = W["batched"].scaled(R=2, L=1, B=5120, keep_p=0.6)
    log("rows=2 B=5120 R=2 keep 0.6, 12 steps")
    p = Pair(w, steps=12, rows=2)
    try:
        first = drive(p, 12, every_step_state=True)
        assert p.evicted > 0 and first is not None, (p.evicted, first)
    finally:
        p.close()
