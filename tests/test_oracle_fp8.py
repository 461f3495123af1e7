"""Pins of the oracle's FP8 record decoding and attention -- CPU only.

"HiSparse 深度解析" (gentlecold.top) §5.5 lists bfloat16 and fp8_e4m3 as the KV
dtypes, fp8 served by a FlashMLA-style kernel; the record read here is that
layout: 512 E4M3 codes in four blocks of 128 with a float32 scale each, then
64 bf16 rope values.  The E4M3 decode is pinned by torch's float8_e4m3fn type
(an independent library routine) on all 256 codes and by values the format
fixes; the attention by the bf16 path on records whose values are exact in both
formats.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as A


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = A.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("code,value", [(0x7E, 448.0), (0xFE, -448.0), (0x38, 1.0), (0xB8, -1.0),
                                        (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
                                        (0x00, 0.0), (0x3C, 1.5), (0x40, 2.0)])
def test_e4m3_values_fixed_by_the_format(code, value):
    assert A.e4m3_to_f64(np.array([code], np.uint8))[0] == value


def test_fp8_record_layout():
    rec = synth.record(1, 2, 3, synth.FP8_RECORD_BYTES)
    vals = A.fp8_records_to_f64(rec[None])[0]
    scales = rec[512:528].copy().view(np.float32)
    codes = torch.from_numpy(rec[:512].copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(vals[:512], (codes.reshape(4, 128) * scales[:, None]).ravel())
    assert np.array_equal(vals[512:], A.bf16_to_f64(rec[528:].copy().view(np.uint16)))
    # the quantiser saturates each block at its max: some code of every block is +-448
    assert all(np.abs(codes.reshape(4, 128)[b]).max() == 448.0 for b in range(4))


def test_fp8_attention_equals_bf16_attention_on_shared_values():
    """Records built so that every value is exact in both formats (scale 1, values that are
    E4M3 numbers): the FP8 and the bf16 attention agree exactly."""
    rng = np.random.default_rng(3)
    n, k, H = 20, 12, 16
    codes = rng.integers(0, 256, size=(n, 512), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38  # no NaN
    fp8 = np.zeros((n, 656), np.uint8)
    fp8[:, :512] = codes
    fp8[:, 512:528] = np.ones((n, 4), np.float32).view(np.uint8)
    rope = rng.integers(0, 2 ** 16, size=(n, 64), dtype=np.uint16)
    rope[(rope & 0x7F80) == 0x7F80] = 0x3F80  # no inf / NaN
    fp8[:, 528:] = rope.view(np.uint8)
    vals = A.e4m3_to_f64(codes)
    bf = np.zeros((n, 576), np.uint16)
    bf[:, :512] = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # exact in bf16
    bf[:, 512:] = rope
    q = (rng.standard_normal((H, 576)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    slots = rng.choice(n, size=k, replace=False)
    a = A.sparse_decode_attention_fp8(q, fp8, slots, 0.05)
    b = A.sparse_decode_attention(q, bf.view(np.uint8), slots, 0.05)
    assert np.array_equal(a, b)
