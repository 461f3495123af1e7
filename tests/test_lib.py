"""CPU checks of the C-ABI library: it loads, and exports every symbol include/hisparse.h
declares (no compute calls: this host has no GPU)."""
import ctypes
import os
import re

import hierarchical_kv_cache_amd as hk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "hisparse.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(hk.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(hk.LIB_PATH)
    missing = [name for name in declared_functions() if not hasattr(lib, name)]
    assert not missing, missing


def test_workspace_sizing_and_validation_without_gpu():
    cfg = hk.make_config(R=32, L=16, max_positions=32768, top_k=2048, buffer_slots=4096)
    n = hk.hs_workspace_bytes(cfg)
    # page tables dominate: 32 * 16 * 32768 entries of 8 bytes (slot, generation)
    assert n >= 32 * 16 * 32768 * 8
    bad = hk.make_config(R=1, L=1, max_positions=4096, top_k=128, buffer_slots=64)  # B < k
    try:
        hk.hs_workspace_bytes(bad)
    except hk.HsError as e:
        assert e.code == hk.HS_EINVAL and "buffer_slots" in str(e)
    else:
        raise AssertionError("B < k accepted")
    bad = hk.make_config(R=1, L=1, max_positions=4096, top_k=96, buffer_slots=128, block_tokens=64)
    try:
        hk.hs_workspace_bytes(bad)
    except hk.HsError as e:
        assert "block_tokens" in str(e)
    else:
        raise AssertionError("block size not dividing k accepted")


def test_capacity_closed_form():
    """Device footprint per request is L * (B + 1) * record bytes, independent of the context
    ("推理系统基础设施手记（六）：HiSparse" (naphjohn.github.io) §2: HBM = N_l * B * W_KV * s;
    its worked figure: 4096 of 131072 tokens per layer, about 3.1 %, about 32x)."""
    import synth
    w = synth.WORKLOADS["long"]
    assert w.B / w.ctx == 4096 / 131072
    assert round(100 * w.B / w.ctx, 1) == 3.1 and w.ctx // w.B == 32
    assert w.hot_bytes() == w.R * w.L * (w.B + 1) * 1152
    assert synth.WORKLOADS["capacity"].host_bytes() == 4 * 4 * 1048576 * 1152


# The per-layer boundary the hot path is specified by: create, resolve, write-through of the
# new token, shared-layer prefetch, the layer wait, the attention consumer, state export,
# teardown.
CONTRACT = ("hs_workspace_bytes", "hs_create", "hs_host_pool", "hs_resolve", "hs_writeback",
            "hs_prefetch_shared", "hs_wait_layer", "hs_sparse_attn", "hs_export_state", "hs_destroy",
            "hs_last_error")


def declarations():
    """(name, the comment block right above the declaration) for every function declared."""
    text = open(os.path.join(ROOT, "include", "hisparse.h")).read()
    out = []
    for m in re.finditer(r"(/\*(?:(?!\*/).)*\*/)\s*\n(?:[a-z_0-9 ]+\*?\s*)(hs_[a-z_0-9]+)\s*\(", text, flags=re.S):
        out.append((m.group(2), m.group(1)))
    return out


def test_contract_names_are_exported():
    lib = ctypes.CDLL(hk.LIB_PATH)
    for name in CONTRACT:
        assert name in hk.EXPORTS and hasattr(lib, name), name
    assert not hasattr(lib, "hs_append"), "the write-through entry has one name, hs_writeback"


def test_stats_layout():
    """hs_stats: hits, misses, error, resident (uint32), then bytes_fetched (uint64)."""
    assert hk.HS_STATS_DTYPE.itemsize == 24
    assert hk.HS_STATS_DTYPE.fields["bytes_fetched"][1] == 16


def test_every_cache_declaration_cites_its_passage():
    """Each declaration of the cache's calls (not the measurement aids after the marker) has a
    comment above it that names a page section ([GC] / [VD] / [NJ] / [KJ] and a §)."""
    text = open(os.path.join(ROOT, "include", "hisparse.h")).read()
    cut = text.index("measurement aids")
    seen = set()
    for name, comment in declarations():
        pos = text.index(name + "(")
        if pos > cut or name in ("hs_last_error", "hs_resolve_wgs", "hs_resolve_attn_wgs", "hs_host_pool",
                                 "hs_page_table", "hs_plan", "hs_sparse_attn_static", "hs_hot_buffer",
                                 "hs_hot_backed_bytes"):
            continue
        seen.add(name)
        assert re.search(r"\[(GC|VD|NJ|KJ)\]", comment), (name, "no page cited")
    assert {"hs_wait_layer", "hs_export_state", "hs_destroy", "hs_workspace_bytes", "hs_writeback"} <= seen
