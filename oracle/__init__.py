"""CPU oracle of the hierarchical KV cache and of its sparse-attention consumer.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``hierarchical_kv_cache_amd``) and imports nothing
from it; the only inputs both sides share come from ``synth``.

* ``Cache``        -- one (request, layer) cache; plain C model in
                      ``hs_oracle.c`` (stamp-based LRU, sort per step).
* ``expand_blocks``, ``replay`` -- block-id expansion and shared-layer copy.
* ``brute``        -- an independently written pure-Python model used to pin
                      ``Cache`` on exhaustive tiny traces.
* ``attention``    -- float64 NumPy sparse decode attention.
* ``policies``     -- offline replacement-policy comparator (topk, FIFO,
                      Random, LRU, Belady) on the seeded traces; also a
                      command-line analysis tool (``python -m oracle.policies``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import attention, brute  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_hso.so")
_lib = None

ERR_DUP, ERR_RANGE, ERR_CAPACITY, ERR_RESIDENT = 1, 2, 4, 8


class OracleError(ValueError):
    def __init__(self, code: int):
        names = [n for b, n in ((ERR_DUP, "duplicate position"), (ERR_RANGE, "position out of range"),
                                (ERR_CAPACITY, "selection larger than the buffer"),
                                (ERR_RESIDENT, "resident row outside the resident pool")) if code & b]
        super().__init__(", ".join(names) or "error %d" % code)
        self.code = code


def build() -> None:
    """Compile the C model with gcc."""
    src = os.path.join(_HERE, "hs_oracle.c")
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-Wall", "-o", tmp, src])
    os.replace(tmp, _SO)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "hs_oracle.c")
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        build()
    lib = ctypes.CDLL(_SO)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.hso_create.argtypes = [i32, i64, i32, i32]
    lib.hso_create.restype = vp
    lib.hso_destroy.argtypes = [vp]
    lib.hso_destroy.restype = None
    lib.hso_resolve.argtypes = [vp, vp, i32, i64, vp, vp, vp, vp, vp]
    lib.hso_resolve.restype = i32
    lib.hso_resolve_tiered.argtypes = [vp, vp, i32, i64, vp, i64, i32, i64, vp, vp, vp, vp, vp]
    lib.hso_resolve_tiered.restype = i32
    lib.hso_resolve_rows.argtypes = [vp, vp, i32, i32, i64, vp, i64, i32, i64, vp, vp, vp, vp, vp]
    lib.hso_resolve_rows.restype = i32
    lib.hso_admit_short.argtypes = [vp, i64, vp]
    lib.hso_admit_short.restype = i32
    lib.hso_append.argtypes = [vp, i64, vp, vp]
    lib.hso_append.restype = i32
    lib.hso_replay.argtypes = [vp, vp, i32, vp, vp, i32]
    lib.hso_replay.restype = None
    lib.hso_expand_blocks.argtypes = [vp, i32, i32, vp]
    lib.hso_expand_blocks.restype = None
    lib.hso_export.argtypes = [vp, vp, vp, vp]
    lib.hso_export.restype = None
    for name in ("hso_page_table", "hso_hot"):
        getattr(lib, name).argtypes = [vp]
        getattr(lib, name).restype = vp
    for name in ("hso_newest", "hso_step"):
        getattr(lib, name).argtypes = [vp]
        getattr(lib, name).restype = i64
    _lib = lib
    return lib


def _addr(buf) -> int:
    if isinstance(buf, int):
        return buf
    if not isinstance(buf, np.ndarray) or not buf.flags["C_CONTIGUOUS"]:
        raise TypeError("expected a C-contiguous numpy array or an address")
    return buf.ctypes.data


class Cache:
    """One (request, layer) cache: B LRU slots, optional newest slot at index B,
    page table over ``max_positions`` positions, host mirror of the slot bytes."""

    def __init__(self, B: int, max_positions: int, rec_bytes: int = 1152, newest_slot: bool = False):
        self._lib = _load()
        self.B, self.max_positions, self.rec_bytes = B, max_positions, rec_bytes
        self._h = self._lib.hso_create(B, max_positions, rec_bytes, 1 if newest_slot else 0)
        if not self._h:
            raise MemoryError("oracle cache allocation failed")

    def close(self):
        if self._h:
            self._lib.hso_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def resolve(self, sel, ctx_len: int, host):
        """Resolve one selection (token positions).  ``host`` is the layer's
        [max_positions][rec_bytes] record array (numpy uint8 or address).
        Returns (out, hits, misses, plan_pos, plan_slot); raises OracleError."""
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        k = sel.size
        out = np.empty(k, np.int32)
        ppos = np.empty(k, np.int32)
        pslot = np.empty(k, np.int32)
        counts = np.zeros(2, np.int32)
        err = self._lib.hso_resolve(self._h, sel.ctypes.data, k, ctx_len, _addr(host), out.ctypes.data,
                                    ppos.ctypes.data, pslot.ctypes.data, counts.ctypes.data)
        if err:
            raise OracleError(err)
        m = int(counts[1])
        return out, int(counts[0]), m, ppos[:m].copy(), pslot[:m].copy()

    def resolve_tiered(self, sel, ctx_len: int, rtable, page_shift: int, res_rows: int, host):
        """Resolve with the resident tier first (``hso_resolve_tiered``).  ``rtable`` is the
        request's int32 block table (resident page per logical page, -1 none).
        Returns (out, hits, misses, resident, plan_pos, plan_slot); raises OracleError."""
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        rt = np.ascontiguousarray(rtable, dtype=np.int32)
        k = sel.size
        out = np.empty(k, np.int32)
        ppos = np.empty(k, np.int32)
        pslot = np.empty(k, np.int32)
        counts = np.zeros(3, np.int32)
        err = self._lib.hso_resolve_tiered(self._h, sel.ctypes.data, k, ctx_len, rt.ctypes.data, rt.size,
                                           page_shift, res_rows, _addr(host), out.ctypes.data,
                                           ppos.ctypes.data, pslot.ctypes.data, counts.ctypes.data)
        if err:
            raise OracleError(err)
        m = int(counts[1])
        return out, int(counts[0]), m, int(counts[2]), ppos[:m].copy(), pslot[:m].copy()

    def resolve_rows(self, sel, ctx_len: int, host, rtable=None, page_shift: int = 0, res_rows: int = 0):
        """Resolve the verification rows ``sel`` [Q][k] of one speculative step together
        (``hso_resolve_rows``).  Returns (out [Q][k], hits, misses, resident, plan_pos,
        plan_slot, union_size); raises OracleError."""
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        Q, k = sel.shape
        out = np.empty((Q, k), np.int32)
        ppos = np.empty(Q * k, np.int32)
        pslot = np.empty(Q * k, np.int32)
        counts = np.zeros(4, np.int32)
        rt = None if rtable is None else np.ascontiguousarray(rtable, dtype=np.int32)
        err = self._lib.hso_resolve_rows(self._h, sel.ctypes.data, Q, k, ctx_len,
                                         None if rt is None else rt.ctypes.data, 0 if rt is None else rt.size,
                                         page_shift, res_rows, _addr(host), out.ctypes.data, ppos.ctypes.data,
                                         pslot.ctypes.data, counts.ctypes.data)
        if err:
            raise OracleError(err)
        m = int(counts[1])
        return out, int(counts[0]), m, int(counts[2]), ppos[:m].copy(), pslot[:m].copy(), int(counts[3])

    def admit_short(self, ctx_len: int, host):
        """Admission of a short request (``hso_admit_short``): positions 0 .. ctx_len-1 in
        slots 0 .. ctx_len-1, short-sequence fast path on while the context fits B."""
        err = self._lib.hso_admit_short(self._h, ctx_len, _addr(host))
        if err:
            raise OracleError(err)

    def append(self, pos: int, record: np.ndarray, host=None):
        rec = np.ascontiguousarray(record, dtype=np.uint8)
        err = self._lib.hso_append(self._h, pos, rec.ctypes.data, 0 if host is None else _addr(host))
        if err:
            raise OracleError(err)

    def export(self) -> dict:
        slot_pos = np.empty(self.B, np.int32)
        stamp = np.empty(self.B, np.int64)
        lru = np.empty(self.B, np.int32)
        self._lib.hso_export(self._h, slot_pos.ctypes.data, stamp.ctypes.data, lru.ctypes.data)
        return {"slot_pos": slot_pos, "stamp": stamp, "lru": lru,
                "newest_pos": int(self._lib.hso_newest(self._h)), "step": int(self._lib.hso_step(self._h))}

    @property
    def page_table(self) -> np.ndarray:
        """Live view of the page table (int32 [max_positions]; -1 = host only)."""
        p = self._lib.hso_page_table(self._h)
        return np.ctypeslib.as_array(ctypes.cast(p, ctypes.POINTER(ctypes.c_int32)),
                                     shape=(self.max_positions,))

    @property
    def hot(self) -> np.ndarray:
        """Live view of the slot bytes (uint8 [B+1][rec_bytes])."""
        p = self._lib.hso_hot(self._h)
        return np.ctypeslib.as_array(ctypes.cast(p, ctypes.POINTER(ctypes.c_uint8)),
                                     shape=(self.B + 1, self.rec_bytes))


def expand_blocks(blocks, block_tokens: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.int32)
    out = np.empty(blocks.size * block_tokens, np.int32)
    _load().hso_expand_blocks(blocks.ctypes.data, blocks.size, block_tokens, out.ctypes.data)
    return out


def replay(plan_pos, plan_slot, host, hot: np.ndarray, rec_bytes: int = 1152) -> None:
    plan_pos = np.ascontiguousarray(plan_pos, dtype=np.int32)
    plan_slot = np.ascontiguousarray(plan_slot, dtype=np.int32)
    _load().hso_replay(plan_pos.ctypes.data, plan_slot.ctypes.data, plan_pos.size, _addr(host),
                       _addr(hot), rec_bytes)
