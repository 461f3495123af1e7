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
