"""Seeded synthetic inputs for the hierarchical KV cache: workloads, selection
traces, KV records and query vectors.

This package holds no step of the cache method.  Both the CPU oracle and the
HIP path read what it produces, and nothing in it depends on either.

* ``WORKLOADS`` describes the five workloads (tiny, long, batched, shared,
  capacity) by shape and trace model.
* ``selection_trace`` produces the per-step top-k selection of one
  (request, layer) cache.
* ``fill_request`` / ``record`` / ``records_at`` / ``queries`` produce bf16
  bytes from a counter-based SplitMix64 + Box-Muller generator (definition in
  ``records.c``); values are N(0,1) rounded to bf16.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

from .traces import selection_trace, trace_stats  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_records.so")
_lib = None

RECORD_BYTES = 1152  # 576 bf16 per token: 512 value dims + 64 rope dims (scores use all 576)
FP8_RECORD_BYTES = 656  # 512 e4m3 codes + 4 float32 block scales + 64 bf16 rope dims
POISON = 0xFF        # byte of host positions not yet written (bf16 NaN pattern)
RECORD_SEED = 0
QUERY_SEED = 1


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int          # first component of every trace seed
    R: int               # requests
    L: int               # layers
    ctx: int             # context tokens at the first decode step
    k: int               # selected tokens per (request, layer, step)
    B: int               # hot slots per (request, layer)
    steps: int
    block_tokens: int = 1      # >1: selections are block ids of this many tokens
    keep_p: float = 0.87       # chance a selected entry stays selected next step
    forced_last: int = 0       # the last n positions are always selected
    uniform_frac: float = 0.5  # share of fresh draws uniform over context (rest Zipf over recency)
    zipf_a: float = 1.1
    append: bool = False       # one token appended per step, written through to host
    force_newest: bool = False # the just-appended token is always selected
    group: int = 1             # layers per anchor group (anchor + group-1 shared layers)
    heads: int = 0             # query heads of the sparse-attention consumer (0: none)

    @property
    def kb(self) -> int:
        """Selection entries per (request, layer, step)."""
        return self.k // self.block_tokens

    def max_positions(self, steps: int | None = None) -> int:
        s = self.steps if steps is None else steps
        return self.ctx + (s if self.append else 0)

    def host_bytes(self, steps: int | None = None) -> int:
        return self.R * self.L * self.max_positions(steps) * RECORD_BYTES

    def hot_bytes(self) -> int:
        return self.R * self.L * (self.B + 1) * RECORD_BYTES

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, R=1, L=1, ctx=4096, k=64, B=128, steps=32, keep_p=0.85,
                     forced_last=16, uniform_frac=1.0),
    "long": Workload("long", 2, R=1, L=8, ctx=131072, k=2048, B=4096, steps=256, keep_p=0.87,
                     uniform_frac=0.5, append=True, force_newest=True, heads=16),
    "batched": Workload("batched", 3, R=32, L=16, ctx=32768, k=2048, B=4096, steps=128,
                        keep_p=0.87, uniform_frac=0.5, heads=16),
    "shared": Workload("shared", 4, R=16, L=32, ctx=131072, k=2048, B=4096, steps=64, keep_p=0.87,
                       uniform_frac=0.5, group=4, heads=16),
    "capacity": Workload("capacity", 5, R=4, L=4, ctx=1048576, k=2048, B=4096, steps=64,
                         block_tokens=64, keep_p=0.8, uniform_frac=0.0),
}
BATCHED_B_SWEEP = (2048, 4096, 8192)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "records.c")
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        build()
    lib = ctypes.CDLL(_SO)
    i64, u64, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
    lib.synth_one.argtypes = [vp, u64, i64, i64, i64, i64]
    lib.synth_one.restype = None
    lib.synth_one_fp8.argtypes = [vp, u64, i64, i64, i64]
    lib.synth_one_fp8.restype = None
    lib.synth_fill_request.argtypes = [vp, i64, i64, i64, i64, i64, u64, ctypes.c_int, ctypes.c_int]
    lib.synth_fill_request.restype = ctypes.c_int
    lib.synth_records_at.argtypes = [vp, i64, i64, vp, i64, u64]
    lib.synth_records_at.restype = None
    _lib = lib
    return lib


def build() -> None:
    """Compile the record generator with gcc (plain C, no GPU code)."""
    src = os.path.join(_HERE, "records.c")
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-Wall", "-o", tmp, src, "-lm",
                           "-lpthread"])
    os.replace(tmp, _SO)


def _ptr(buf) -> int:
    if isinstance(buf, int):
        return buf
    if isinstance(buf, np.ndarray):
        if not buf.flags["C_CONTIGUOUS"]:
            raise ValueError("buffer must be C-contiguous")
        return buf.ctypes.data
    raise TypeError("expected a numpy array or an integer address")


def record(r: int, l: int, pos: int, rec_bytes: int = RECORD_BYTES, seed: int = RECORD_SEED):
    """The KV record of (request r, layer l, position pos) as uint8 bytes: bf16 values, or
    the FP8 layout when rec_bytes is FP8_RECORD_BYTES."""
    out = np.empty(rec_bytes, np.uint8)
    if rec_bytes == FP8_RECORD_BYTES:
        _load().synth_one_fp8(out.ctypes.data, seed, r, l, pos)
    else:
        _load().synth_one(out.ctypes.data, seed, r, l, pos, rec_bytes // 2)
    return out


def records_at(R: int, L: int, pos, rec_bytes: int = RECORD_BYTES, seed: int = RECORD_SEED):
    """uint8 [R][L][rec_bytes]: the record of position pos[r] for every (r, l)."""
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64).reshape(R))
    out = np.empty((R, L, rec_bytes), np.uint8)
    _load().synth_records_at(out.ctypes.data, R, L, pos.ctypes.data, rec_bytes, seed)
    return out


def fill_request(buf, req: int, L: int, lmax: int, ctx: int, rec_bytes: int = RECORD_BYTES,
                 seed: int = RECORD_SEED, poison: int = POISON, nthreads: int | None = None):
    """Fill one request's host region [L][lmax][rec_bytes] (numpy array or address):
    positions < ctx get their records, the rest the poison byte."""
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    rc = _load().synth_fill_request(_ptr(buf), req, L, lmax, ctx, rec_bytes, seed, poison,
                                    nthreads)
    if rc != 0:
        raise RuntimeError("synth_fill_request failed (%d)" % rc)


def queries(R: int, L: int, step: int, heads: int = 16, dim: int = 576, seed: int = QUERY_SEED):
    """bf16 query vectors of one decode step as uint16 [R][L][heads][dim]."""
    out = np.empty((R, L, heads, dim), np.uint16)
    lib = _load()
    for r in range(R):
        for l in range(L):
            lib.synth_one(out[r, l].ctypes.data, seed, r, l, step, heads * dim)
    return out
