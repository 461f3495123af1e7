"""Float64 sparse decode attention over the published slots.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

The consumer reads, for each selected entry i, the record in slot out[i]
of the (request, layer) hot buffer ("HiSparse 深度解析" (gentlecold.top)
§5.4: sparse attention reads the physical slots aligned with the top-k
order).  A record holds 576 bf16 values: scores use all 576 (the key), the
output mixes the first 512 (the value), so H query heads share one latent
KV row per token.  s = scale * q K^T, p = softmax over the k entries,
o = p V, all in float64 from the bf16 bytes.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact)."""
    u16 = np.ascontiguousarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64, from the format's definition: sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
    (mantissa * 2^-9); exponent 15 with mantissa 7 is NaN (there is no infinity)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def fp8_records_to_f64(rows: np.ndarray) -> np.ndarray:
    """uint8 [n][656] FP8 records -> float64 [n][576]: the 512 E4M3 codes times their block's
    float32 scale (blocks of 128), then the 64 bf16 values."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    codes = e4m3_to_f64(rows[:, :512]).reshape(n, 4, 128)
    scales = rows[:, 512:528].copy().view(np.float32).astype(np.float64).reshape(n, 4, 1)
    rope = bf16_to_f64(rows[:, 528:656].copy().view(np.uint16))
    return np.concatenate([(codes * scales).reshape(n, 512), rope], axis=1)


def sparse_decode_attention_rows(q: np.ndarray, K: np.ndarray, scale: float, dv: int = 512) -> np.ndarray:
    """q: uint16 [H][D] bf16 queries; K: float64 [k][D] the selected keys (values are their
    first dv dims).  Returns float64 [H][dv]."""
    Q = bf16_to_f64(q)
    V = K[:, :dv]
    s = scale * (Q @ K.T)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ V


def sparse_decode_attention_fp8(q: np.ndarray, hot: np.ndarray, slots: np.ndarray, scale: float,
                                dv: int = 512) -> np.ndarray:
    """The same attention over FP8 records: hot is uint8 [S][656]."""
    K = fp8_records_to_f64(hot[np.asarray(slots, dtype=np.int64)])
    return sparse_decode_attention_rows(q, K, scale, dv)


def sparse_decode_attention(q: np.ndarray, hot: np.ndarray, slots: np.ndarray, scale: float,
                            dv: int = 512) -> np.ndarray:
    """q: uint16 [H][D] bf16 queries; hot: uint8 [S][2*D] slot bytes;
    slots: [k] slot per selected entry.  Returns float64 [H][dv]."""
    Q = bf16_to_f64(q)
    rows = np.ascontiguousarray(hot[np.asarray(slots, dtype=np.int64)]).view(np.uint16)
    K = bf16_to_f64(rows)
    V = K[:, :dv]
    s = scale * (Q @ K.T)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ V
