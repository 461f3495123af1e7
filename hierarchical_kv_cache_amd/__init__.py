"""Python binding of libhisparse (hierarchical KV cache for top-k sparse-attention
decode on MI355X).

The functions below carry the C ABI's names (``include/hisparse.h``) and only
marshal arguments: integers are device or host addresses, streams are
``hipStream_t`` handles (``torch.cuda.Stream.cuda_stream``).  Every step of
the path runs in the HIP library; when it is missing, importing this package
raises instead of falling back to anything else.

``HiSparse`` is a convenience owner: it allocates the hot buffer and the
workspace as torch tensors (torch is only the device-memory and stream
provider) and forwards to the C calls.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import _build

LIB_PATH = _build.LIB

HS_OK, HS_EINVAL, HS_ENOMEM, HS_EHIP, HS_ESTATE = 0, -1, -2, -3, -4
HS_CFG_NEWEST_SLOT, HS_CFG_RECORD_FP8, HS_CFG_HOT_ON_DEMAND = 1, 2, 4
HS_RECORD_PLAN, HS_SKIP_IO = 1, 2
HS_ERR_DUP, HS_ERR_RANGE, HS_ERR_STATE, HS_ERR_RESIDENT, HS_ERR_CAPACITY = 1, 2, 4, 8, 16


class hs_config(ctypes.Structure):
    _fields_ = [
        ("num_requests", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("max_positions", ctypes.c_int64),
        ("record_bytes", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32),
        ("buffer_slots", ctypes.c_int32),
        ("layer_group", ctypes.c_int32),
        ("wgs_per_request", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("verify_rows", ctypes.c_int32),
    ]


HS_STATS_DTYPE = np.dtype([("hits", np.uint32), ("misses", np.uint32), ("error", np.uint32),
                           ("resident", np.uint32), ("bytes_fetched", np.uint64)])
# hs_stats in int32 words (24 bytes): hits, misses, error, resident, then bytes_fetched as two
# words (low, high)
HS_STATS_WORDS = 6
assert HS_STATS_DTYPE.itemsize == 4 * HS_STATS_WORDS

# every symbol include/hisparse.h declares
EXPORTS = (
    "hs_workspace_bytes", "hs_create", "hs_host_pool", "hs_hot_buffer", "hs_grow_request", "hs_hot_backed_bytes",
    "hs_resolve", "hs_resolve_rows", "hs_bind_resident",
    "hs_writeback",
    "hs_prefetch_shared",
    "hs_wait_layer", "hs_sparse_attn", "hs_sparse_attn_static", "hs_resolve_attn", "hs_resolve_attn_wgs", "hs_export_state", "hs_page_table", "hs_plan", "hs_admit_short",
    "hs_reset_request",
    "hs_destroy", "hs_last_error", "hs_resolve_wgs", "hs_probe_host_read", "hs_probe_copy",
    "hs_probe_host_records", "hs_probe_empty", "hs_timing_start", "hs_timing_read",
)


class HsError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (status %d)" % (msg, code))
        self.code = code


def _load():
    # torch ships a HIP runtime of its own: when torch is installed it is loaded first, so that
    # the library's libamdhip64 dependency resolves to that same runtime (two runtimes in one
    # process do not see each other's devices, streams or allocations)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError("libhisparse.so is not built: run hierarchical_kv_cache_amd._build.build() "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    cfgp = ctypes.POINTER(hs_config)
    sig = {
        "hs_workspace_bytes": (sz, [cfgp]),
        "hs_create": (i32, [cfgp, vp, vp, ctypes.POINTER(vp)]),
        "hs_host_pool": (vp, [vp, i32]),
        "hs_hot_buffer": (vp, [vp]),
        "hs_grow_request": (i32, [vp, i32, i32, vp]),
        "hs_hot_backed_bytes": (i64, [vp]),
        "hs_resolve": (i32, [vp, i32, vp, vp, vp, vp, vp, u32, vp]),
        "hs_resolve_rows": (i32, [vp, i32, i32, vp, vp, vp, vp, vp, u32, vp]),
        "hs_bind_resident": (i32, [vp, vp, i32, i32, vp, i64]),
        "hs_writeback": (i32, [vp, vp, vp, vp, vp]),
        "hs_prefetch_shared": (i32, [vp, i32, vp, vp]),
        "hs_wait_layer": (i32, [vp, i32, vp]),
        "hs_sparse_attn": (i32, [vp, i32, vp, i32, i32, vp, vp, ctypes.c_float, vp, vp]),
        "hs_sparse_attn_static": (i32, [vp, i32, vp, i32, i32, vp, vp, ctypes.c_float, vp, vp]),
        "hs_resolve_attn": (i32, [vp, i32, vp, vp, vp, vp, vp, u32, vp, i32, i32, vp, ctypes.c_float, vp]),
        "hs_resolve_attn_wgs": (i32, [vp]),
        "hs_export_state": (i32, [vp, i32, vp, vp, vp, vp, vp]),
        "hs_page_table": (vp, [vp, i32]),
        "hs_plan": (i32, [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp)]),
        "hs_admit_short": (i32, [vp, i32, i32, vp]),
        "hs_reset_request": (i32, [vp, i32, vp]),
        "hs_destroy": (i32, [vp]),
        "hs_last_error": (ctypes.c_char_p, []),
        "hs_resolve_wgs": (i32, [vp]),
        "hs_probe_host_read": (i32, [vp, sz, vp, i32, vp]),
        "hs_probe_copy": (i32, [vp, vp, sz, vp]),
        "hs_probe_host_records": (i32, [vp, i64, i32, vp, i32, vp, i32, vp]),
        "hs_probe_empty": (i32, [i32, vp]),
        "hs_timing_start": (i32, [vp, i32]),
        "hs_timing_read": (i32, [vp, vp, i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != HS_OK:
        raise HsError(status, _lib.hs_last_error().decode())


# ---- C ABI, same names -------------------------------------------------------------------

def hs_workspace_bytes(cfg: hs_config) -> int:
    n = _lib.hs_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise HsError(HS_EINVAL, _lib.hs_last_error().decode())
    return n


def hs_create(cfg: hs_config, d_hot: int, d_workspace: int) -> int:
    h = ctypes.c_void_p()
    _check(_lib.hs_create(ctypes.byref(cfg), d_hot, d_workspace, ctypes.byref(h)))
    return h.value


def hs_host_pool(h: int, request: int) -> int:
    return _lib.hs_host_pool(h, request) or 0


def hs_hot_buffer(h) -> int:
    return _lib.hs_hot_buffer(h) or 0


def hs_grow_request(h, request, slots, stream):
    _check(_lib.hs_grow_request(h, request, slots, stream or None))


def hs_hot_backed_bytes(h) -> int:
    return _lib.hs_hot_backed_bytes(h)


def hs_resolve(h, layer, d_sel, d_ctx_len, d_slots_out, d_stats, d_num_reqs, flags, stream):
    _check(_lib.hs_resolve(h, layer, d_sel, d_ctx_len, d_slots_out, d_stats or None, d_num_reqs or None,
                           flags, stream or None))


def hs_resolve_rows(h, layer, rows, d_sel, d_ctx_len, d_slots_out, d_stats, d_num_reqs, flags, stream):
    _check(_lib.hs_resolve_rows(h, layer, rows, d_sel, d_ctx_len, d_slots_out, d_stats or None, d_num_reqs or None,
                                flags, stream or None))


def hs_bind_resident(h, d_block_table, pages_per_request, page_tokens, d_resident_kv, resident_rows):
    _check(_lib.hs_bind_resident(h, d_block_table or None, pages_per_request, page_tokens, d_resident_kv or None,
                                 resident_rows))


def hs_writeback(h, d_new_kv, d_new_pos, compute, backup):
    _check(_lib.hs_writeback(h, d_new_kv, d_new_pos, compute or None, backup or None))


def hs_prefetch_shared(h, anchor_layer, compute, prefetch):
    _check(_lib.hs_prefetch_shared(h, anchor_layer, compute or None, prefetch or None))


def hs_wait_layer(h, layer, stream):
    _check(_lib.hs_wait_layer(h, layer, stream or None))


def hs_sparse_attn(h, layer, d_q, heads, value_dim, d_slots, d_out, scale, d_num_reqs, stream):
    _check(_lib.hs_sparse_attn(h, layer, d_q, heads, value_dim, d_slots, d_out, scale, d_num_reqs or None,
                               stream or None))


def hs_sparse_attn_static(h, layer, d_q, heads, value_dim, d_slots, d_out, scale, d_num_reqs, stream):
    _check(_lib.hs_sparse_attn_static(h, layer, d_q, heads, value_dim, d_slots, d_out, scale, d_num_reqs or None,
                                      stream or None))


def hs_resolve_attn(h, layer, d_sel, d_ctx_len, d_slots_out, d_stats, d_num_reqs, flags, d_q, heads, value_dim,
                    d_out, scale, stream):
    _check(_lib.hs_resolve_attn(h, layer, d_sel, d_ctx_len, d_slots_out, d_stats or None, d_num_reqs or None,
                                flags, d_q, heads, value_dim, d_out, scale, stream or None))


def hs_resolve_attn_wgs(h) -> int:
    return _lib.hs_resolve_attn_wgs(h)


def hs_export_state(h, layer, d_slot_pos, d_lru, d_page_table, d_newest, stream):
    _check(_lib.hs_export_state(h, layer, d_slot_pos or None, d_lru or None, d_page_table or None, d_newest or None,
                                stream or None))


def hs_page_table(h, layer) -> int:
    p = _lib.hs_page_table(h, layer)
    if not p:
        raise HsError(HS_EINVAL, "no page table for layer %d" % layer)
    return p


def hs_plan(h, layer):
    plan, counts = ctypes.c_void_p(), ctypes.c_void_p()
    _check(_lib.hs_plan(h, layer, ctypes.byref(plan), ctypes.byref(counts)))
    return plan.value, counts.value


def hs_admit_short(h, request, ctx_len, stream):
    _check(_lib.hs_admit_short(h, request, ctx_len, stream or None))


def hs_reset_request(h, request, stream):
    _check(_lib.hs_reset_request(h, request, stream or None))


def hs_destroy(h):
    _check(_lib.hs_destroy(h))


def hs_last_error() -> str:
    return _lib.hs_last_error().decode()


def hs_resolve_wgs(h) -> int:
    return _lib.hs_resolve_wgs(h)


def hs_probe_host_read(host_src, nbytes, d_sink, wgs, stream):
    _check(_lib.hs_probe_host_read(host_src, nbytes, d_sink, wgs, stream or None))


def hs_probe_copy(d_src, d_dst, nbytes, stream):
    _check(_lib.hs_probe_copy(d_src, d_dst, nbytes, stream or None))


def hs_probe_host_records(host_src, src_records, rec_bytes, d_index, n, d_dst, wgs, stream):
    _check(_lib.hs_probe_host_records(host_src, src_records, rec_bytes, d_index, n, d_dst, wgs,
                                      stream or None))


def hs_probe_empty(n, stream):
    _check(_lib.hs_probe_empty(n, stream or None))


def hs_timing_start(h, n):
    _check(_lib.hs_timing_start(h, n))


def hs_timing_read(h, n) -> np.ndarray:
    """Durations (µs) of the timed RESOLVE launches, in launch order."""
    out = np.zeros(max(0, n), np.float32)
    m = _lib.hs_timing_read(h, out.ctypes.data, n)
    if m < 0:
        raise HsError(m, _lib.hs_last_error().decode())
    return out[:m]


# ---- convenience owner --------------------------------------------------------------------

def make_config(R, L, max_positions, top_k, buffer_slots, record_bytes=1152, block_tokens=1, layer_group=1,
                wgs_per_request=0, newest_slot=False, fp8=False, verify_rows=0, hot_on_demand=False) -> hs_config:
    flags = (HS_CFG_NEWEST_SLOT if newest_slot else 0) | (HS_CFG_RECORD_FP8 if fp8 else 0) | \
        (HS_CFG_HOT_ON_DEMAND if hot_on_demand else 0)
    return hs_config(R, L, max_positions, 656 if fp8 else record_bytes, top_k, block_tokens, buffer_slots,
                     layer_group, wgs_per_request, flags, verify_rows)


class HiSparse:
    """Owns a handle plus the torch tensors it runs on (hot buffer, workspace)."""

    def __init__(self, cfg: hs_config, device="cuda"):
        import torch
        self.cfg = cfg
        self.R, self.L, self.B, self.k = cfg.num_requests, cfg.num_layers, cfg.buffer_slots, cfg.top_k
        self.rec = cfg.record_bytes
        self.max_positions = cfg.max_positions
        ws_bytes = hs_workspace_bytes(cfg)
        # with HS_CFG_HOT_ON_DEMAND the library reserves the hot buffer (hot_address; no tensor)
        on_demand = bool(cfg.flags & HS_CFG_HOT_ON_DEMAND)
        self.hot = None if on_demand else \
            torch.empty((self.R, self.L, self.B + 1, self.rec), dtype=torch.uint8, device=device)
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        self.h = hs_create(cfg, 0 if on_demand else self.hot.data_ptr(), self.workspace.data_ptr())
        self.hot_address = hs_hot_buffer(self.h)

    def host_pool(self, request: int) -> np.ndarray:
        """numpy view [L][max_positions][record_bytes] of request's pinned region."""
        addr = hs_host_pool(self.h, request)
        n = self.L * self.max_positions * self.rec
        buf = (ctypes.c_uint8 * n).from_address(addr)
        return np.frombuffer(buf, dtype=np.uint8).reshape(self.L, self.max_positions, self.rec)

    def host_pool_address(self, request: int) -> int:
        return hs_host_pool(self.h, request)

    @property
    def wgs(self) -> int:
        return hs_resolve_wgs(self.h)

    def close(self):
        if getattr(self, "h", None):
            hs_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
