"""FP8 latent-KV records on the GPU through the C ABI, against the oracle.

"HiSparse 深度解析" (gentlecold.top) §5.5: the KV dtype may be fp8_e4m3 (a
FlashMLA-style layout).  RESOLVE moves the 656-byte records as opaque bytes
(compared bit for bit); the attention consumer dequantises them (code times
its block's scale, rounded to bf16) and is compared with the float64 oracle
within the 2e-3 relative bound.  The decode itself is checked exactly with a
one-entry selection and q = 0, where attention returns the value row.
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
from oracle import attention as A

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def crafted(codes: np.ndarray, scales) -> np.ndarray:
    rec = np.zeros(656, np.uint8)
    rec[:512] = codes
    rec[512:528] = np.asarray(scales, np.float32).view(np.uint8)
    rec[528:] = (np.arange(64, dtype=np.float32) / 8 - 4).view(np.uint32).__rshift__(16).astype(np.uint16).view(np.uint8)
    return rec


def test_every_e4m3_code_decodes_exactly():
    """Records holding each of the 254 finite codes with exactly representable scales:
    attention over one entry with q = 0 returns the dequantised value row."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    recs = [crafted(np.resize(finite, 512), [1.0, 1.0, 1.0, 1.0]),
            crafted(np.resize(finite[::-1], 512), [0.125, 2.0, 1.0, 0.5])]
    n = len(recs)
    cfg = hk.make_config(1, 1, n, 1, 2, fp8=True)
    c = hk.HiSparse(cfg)
    pool = c.host_pool(0)
    for i, rec in enumerate(recs):
        pool[0, i] = rec
    dev = torch.device("cuda")
    out = torch.empty((1, 1), dtype=torch.int32, device=dev)
    q = torch.zeros((1, 16, 576), dtype=torch.int16, device=dev)
    o = torch.empty((1, 16, 512), dtype=torch.float32, device=dev)
    ctx = torch.full((1,), n, dtype=torch.int32, device=dev)
    for i, rec in enumerate(recs):
        sel = torch.tensor([[i]], dtype=torch.int32, device=dev)
        hk.hs_resolve(c.h, 0, sel.data_ptr(), ctx.data_ptr(), out.data_ptr(), 0, 0, 0, 0)
        hk.hs_sparse_attn(c.h, 0, q.data_ptr(), 16, 512, out.data_ptr(), o.data_ptr(), 1.0, 0, 0)
        torch.cuda.synchronize()
        got = o.cpu().numpy()[0]
        exp = A.fp8_records_to_f64(rec[None])[0, :512]
        for h in range(16):
            assert np.array_equal(got[h].astype(np.float64), exp), (i, h)
    c.close()


def fp8_attn_check(p, step, layers, heads=16):
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
            rows = np.concatenate([hot, p.res_pool[l]]) if p.resident is not None else hot
            ref = A.sparse_decode_attention_fp8(q[r, l], rows, slots[r], SCALE)
            err = np.abs(o[r] - ref).max() / np.abs(ref).max()
            worst = max(worst, err)
            assert err <= 2e-3, (r, l, err)
    return worst


def test_fp8_long_with_write_through():
    w = W["long"].scaled(L=2)
    p = Pair(w, steps=12, fp8=True)
    for t in range(12):
        p.step_gpu_and_oracle()
        if t % 4 == 3:
            log("fp8 long step %d worst rel err %.2e" % (t, fp8_attn_check(p, t, range(w.L))))
    p.check_state()
    p.close()


def test_fp8_batched():
    w = W["batched"].scaled(L=2)
    p = Pair(w, steps=4, fp8=True)
    for t in range(4):
        p.step_gpu_and_oracle()
    log("fp8 batched worst rel err %.2e" % fp8_attn_check(p, 3, range(w.L)))
    p.check_state()
    p.close()


def test_fp8_shared_layers_and_resident_tier():
    from synth.resident import ResidentSpec
    w = W["shared"].scaled(R=2, L=8, ctx=16384)
    p = Pair(w, steps=3, fp8=True, resident=ResidentSpec(window_tokens=2048, old_frac=0.2))
    for t in range(3):
        p.step_gpu_and_oracle()
    fp8_attn_check(p, 2, range(w.L))
    p.check_state()
    p.check_hot()
    p.close()


@pytest.mark.parametrize("k,heads", [(64, 16), (100, 5)])
def test_fp8_ragged(k, heads):
    w = W["tiny"].scaled(k=k, B=max(128, k + 40), R=3, forced_last=min(16, k))
    p = Pair(w, steps=3, fp8=True)
    for t in range(3):
        p.step_gpu_and_oracle()
        fp8_attn_check(p, t, [0], heads=heads)
    p.close()
