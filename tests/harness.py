"""Drives a workload through the HIP library (C ABI) and the CPU oracle side by side.

Test infrastructure: imports both sides; neither side imports the other.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import hierarchical_kv_cache_amd as hk
import oracle
import synth
from synth.resident import ResidentSpec, resident_layout

SCALE = 576 ** -0.5


def expand(sel_row, bt):
    return oracle.expand_blocks(sel_row, bt) if bt > 1 else np.asarray(sel_row, np.int32)


class Pair:
    """One HiSparse handle plus the matching oracle caches for a workload."""

    def __init__(self, w: synth.Workload, steps: int | None = None, wgs: int = 0, all_hit=False,
                 oracle_host_copy: bool | None = None, compare_hot=True, resident: ResidentSpec | None = None,
                 fp8: bool = False, rows: int = 1, fused_heads: int = 0, append_streams: str = "two",
                 rows_keep=0.9):
        self.w = w
        # hs_writeback's write-through: "two" (backup stream and events) or "one" (one kernel on
        # the compute stream); may be changed between steps
        self.append_streams = append_streams
        self.steps = w.steps if steps is None else steps
        self.lmax = w.max_positions(self.steps)
        self.R, self.L, self.B, self.k, self.kb = w.R, w.L, w.B, w.k, w.kb
        self.fp8 = fp8
        self.rec = synth.FP8_RECORD_BYTES if fp8 else synth.RECORD_BYTES
        self.compare_hot = compare_hot
        cfg = hk.make_config(w.R, w.L, self.lmax, w.k, w.B, record_bytes=self.rec,
                             block_tokens=w.block_tokens, layer_group=w.group, wgs_per_request=wgs,
                             newest_slot=w.append, fp8=fp8, verify_rows=rows if rows > 1 else 0)
        self.gpu = hk.HiSparse(cfg)
        self.h = self.gpu.h
        self.dev = torch.device("cuda")
        self.compute = torch.cuda.current_stream()
        self.side = torch.cuda.Stream()
        # host pools: the prefill records, written by the input generator
        for r in range(w.R):
            synth.fill_request(self.gpu.host_pool_address(r), r, w.L, self.lmax, w.ctx, rec_bytes=self.rec)
        # the oracle reads the same input bytes; with write-through the GPU also writes the
        # pinned pool, so the oracle then keeps a pool of its own
        if oracle_host_copy is None:
            oracle_host_copy = w.append
        if oracle_host_copy:
            self.ohost = []
            for r in range(w.R):
                a = np.empty((w.L, self.lmax, self.rec), np.uint8)
                synth.fill_request(a, r, w.L, self.lmax, w.ctx, rec_bytes=self.rec)
                self.ohost.append(a)
        else:
            self.ohost = [self.gpu.host_pool(r) for r in range(w.R)]
        self.anchors = [l for l in range(w.L) if l % w.group == 0]
        self.caches = {(r, l): oracle.Cache(w.B, self.lmax, self.rec, newest_slot=w.append)
                       for r in range(w.R) for l in self.anchors}
        self.ohot_shared = {(r, l): np.zeros((w.B + 1, self.rec), np.uint8)
                            for r in range(w.R) for l in range(w.L) if l % w.group}
        # selection traces, resident on the device: [steps][anchors][R][kb], or with
        # speculative verification rows [steps][anchors][R][rows][kb]
        self.rows = rows
        # fused RESOLVE + attention (hs_resolve_attn) with this many query heads; 0: hs_resolve
        self.fused_heads = fused_heads
        self.worst_attn = 0.0
        if fused_heads:
            self.d_att = torch.empty((len(self.anchors_of(w)), w.R, fused_heads, 512), dtype=torch.float32,
                                     device=self.dev)
        if rows > 1:
            from synth.traces import verify_rows
            # rows_keep: each row's chance of keeping an entry of the row before, for every
            # request or per request (the lower, the longer the union)
            keep = list(rows_keep) if hasattr(rows_keep, "__len__") else [rows_keep] * w.R
            tr = np.stack([np.stack([verify_rows(w, r, l, self.steps, rows, keep=keep[r]) for r in range(w.R)],
                                    axis=1) for l in self.anchors], axis=1)
        else:
            tr = np.stack([np.stack([synth.selection_trace(w, r, l, self.steps, all_hit=all_hit)
                                     for r in range(w.R)], axis=1) for l in self.anchors], axis=1)
        self.trace = tr
        self.d_trace = torch.from_numpy(tr).to(self.dev)
        out_shape = (len(self.anchors), w.R, rows, w.k) if rows > 1 else (len(self.anchors), w.R, w.k)
        self.d_out = torch.empty(out_shape, dtype=torch.int32, device=self.dev)
        self.d_stats = torch.zeros((w.R, hk.HS_STATS_WORDS), dtype=torch.int32, device=self.dev)
        self.t = 0
        self.newest = None
        # occupied LRU slots of each anchor cache, and how many misses so far took a slot that
        # held a position (an eviction): empty slots are taken first, so a step with m misses
        # and e empty slots evicts max(0, m - e) occupied ones (counted from the oracle's misses)
        self.occupied = {}
        self.evicted = 0
        self.evicted_at = {}
        self.resident = resident
        if resident is not None:
            self._bind_resident(resident)
        # the oracle's C calls release the GIL: independent caches resolve in parallel
        self.pool = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))

    def _bind_resident(self, spec: ResidentSpec):
        """Resident tier: the pool holds, at each resident page's rows, the records of that
        page's positions for every layer (copied from the prefill records)."""
        w = self.w
        P = spec.page_tokens
        self.page_shift = P.bit_length() - 1
        self.phys, self.masks, total = resident_layout(w, self.steps, spec)
        self.res_rows = max(1, total) * P
        pool = np.zeros((w.L, self.res_rows, self.rec), np.uint8)
        for r in range(w.R):
            pages = np.nonzero(self.phys[r] >= 0)[0]
            src = (pages[:, None] * P + np.arange(P)).ravel()
            dst = (self.phys[r][pages][:, None].astype(np.int64) * P + np.arange(P)).ravel()
            for l in range(w.L):
                pool[l, dst] = self.ohost[r][l][src]
        self.res_pool = pool
        self.d_res = torch.from_numpy(pool).to(self.dev)
        self.n_pages = self.phys.shape[1]
        self.d_table = torch.full((w.R, self.n_pages), -1, dtype=torch.int32, device=self.dev)
        hk.hs_bind_resident(self.h, self.d_table.data_ptr(), self.n_pages, P, self.d_res.data_ptr(), self.res_rows)

    @staticmethod
    def anchors_of(w):
        return [l for l in range(w.L) if l % w.group == 0]

    def table(self, t):
        return np.where(self.masks[t], self.phys, -1).astype(np.int32)

    # ---- one decode step ------------------------------------------------------------------
    def ctx_len(self):
        return self.w.ctx + (self.t + 1 if self.w.append else 0)

    def step_gpu_and_oracle(self, flags=0, check=True, num_reqs=None):
        w, t = self.w, self.t
        ctx = self.ctx_len()
        d_ctx = torch.full((w.R,), ctx, dtype=torch.int32, device=self.dev)
        results = {}
        if w.append:
            p = w.ctx + t
            recs = synth.records_at(w.R, w.L, [p] * w.R, rec_bytes=self.rec)
            d_new = torch.from_numpy(recs).to(self.dev)
            d_pos = torch.full((w.R,), p, dtype=torch.int32, device=self.dev)
            backup = self.side.cuda_stream if self.append_streams == "two" else self.compute.cuda_stream
            hk.hs_writeback(self.h, d_new.data_ptr(), d_pos.data_ptr(), self.compute.cuda_stream, backup)
            for r in range(w.R):
                for l in self.anchors:
                    self.caches[(r, l)].append(p, recs[r, l], self.ohost[r][l])
            self.newest = p
            self._keep = (d_new, d_pos)
        if self.resident is not None:
            tab = self.table(t)
            self.d_table.copy_(torch.from_numpy(tab))
        d_nr = None
        if num_reqs is not None:
            d_nr = torch.tensor([num_reqs], dtype=torch.int32, device=self.dev)
        if self.fused_heads:
            q = synth.queries(w.R, w.L, t, heads=self.fused_heads)
            d_q = torch.from_numpy(q.view(np.int16)).to(self.dev)
        for ai, l in enumerate(self.anchors):
            d_sel = self.d_trace[t, ai]
            fl = flags | (hk.HS_RECORD_PLAN if w.group > 1 else 0)
            if self.rows > 1:
                hk.hs_resolve_rows(self.h, l, self.rows, d_sel.data_ptr(), d_ctx.data_ptr(), self.d_out[ai].data_ptr(),
                                   self.d_stats.data_ptr(), d_nr.data_ptr() if d_nr is not None else 0, fl,
                                   self.compute.cuda_stream)
            elif self.fused_heads:
                dq = d_q[:, l].contiguous()
                hk.hs_resolve_attn(self.h, l, d_sel.data_ptr(), d_ctx.data_ptr(), self.d_out[ai].data_ptr(),
                                   self.d_stats.data_ptr(), d_nr.data_ptr() if d_nr is not None else 0, fl,
                                   dq.data_ptr(), self.fused_heads, 512, self.d_att[ai].data_ptr(), SCALE,
                                   self.compute.cuda_stream)
                self._keep_q = dq
            else:
                hk.hs_resolve(self.h, l, d_sel.data_ptr(), d_ctx.data_ptr(), self.d_out[ai].data_ptr(),
                              self.d_stats.data_ptr(), d_nr.data_ptr() if d_nr is not None else 0, fl,
                              self.compute.cuda_stream)
            if w.group > 1:
                hk.hs_prefetch_shared(self.h, l, self.compute.cuda_stream, self.side.cuda_stream)
            stats = self.d_stats.cpu().numpy().copy() if check else None
            nr = w.R if num_reqs is None else num_reqs

            def one(r, l=l, ai=ai):
                if self.rows > 1:
                    sel = np.stack([expand(row, w.block_tokens) for row in self.trace[t, ai, r]])
                    rt = tab[r] if self.resident is not None else None
                    o, hh, mm, rr, pp, ps, nu = self.caches[(r, l)].resolve_rows(
                        sel, ctx, self.ohost[r][l], rt, getattr(self, "page_shift", 0), getattr(self, "res_rows", 0))
                    res = (o, hh, mm, pp, ps, rr)
                    for ls in range(l + 1, min(l + w.group, w.L)):
                        oracle.replay(res[3], res[4], self.ohost[r][ls], self.ohot_shared[(r, ls)], self.rec)
                    return res
                pos = expand(self.trace[t, ai, r], w.block_tokens)
                if self.resident is not None:
                    o, hh, mm, rr, pp, ps = self.caches[(r, l)].resolve_tiered(
                        pos, ctx, tab[r], self.page_shift, self.res_rows, self.ohost[r][l])
                    res = (o, hh, mm, pp, ps, rr)
                else:
                    res = self.caches[(r, l)].resolve(pos, ctx, self.ohost[r][l]) + (0,)
                for ls in range(l + 1, min(l + w.group, w.L)):
                    oracle.replay(res[3], res[4], self.ohost[r][ls], self.ohot_shared[(r, ls)], self.rec)
                return res

            for r, res in zip(range(nr), self.pool.map(one, range(nr))):
                results[(r, l)] = res
                if self.resident is None:
                    occ = self.occupied.get((r, l), 0)
                    ev = max(0, int(res[2]) - (w.B - occ))
                    self.evicted += ev
                    if ev:
                        self.evicted_at[t] = self.evicted_at.get(t, 0) + ev
                    self.occupied[(r, l)] = min(w.B, occ + int(res[2]))
                if check:
                    assert stats[r, 0] == res[1] and stats[r, 1] == res[2] and stats[r, 2] == 0 \
                        and stats[r, 3] == res[5], (t, r, l, stats[r], res[1], res[2], res[5])
                    fetched = int(stats[r, 4].astype(np.uint32)) | (int(stats[r, 5].astype(np.uint32)) << 32)
                    want = 0 if flags & hk.HS_SKIP_IO else res[2] * self.rec
                    assert fetched == want, ("bytes_fetched", t, r, l, fetched, want)
            if check:
                got = self.d_out[ai].cpu().numpy()
                for r in range(nr):
                    exp = results[(r, l)][0]
                    if not np.array_equal(got[r], exp):
                        bad = np.argwhere(got[r] != exp)  # (entry) or (row, entry) indices
                        raise AssertionError("slots differ at step %d r %d l %d: %d entries, first %s"
                                             % (t, r, l, len(bad), [(tuple(int(x) for x in i), int(got[r][tuple(i)]),
                                                                     int(exp[tuple(i)])) for i in bad[:5]]))
                if self.fused_heads:
                    self._check_attention(t, ai, l, q, nr)
        for l in range(w.L):
            hk.hs_wait_layer(self.h, l, self.compute.cuda_stream)
        self.t += 1
        return results

    def _check_attention(self, t, ai, l, q, nr):
        """Fused attention output against float64 attention over the records of the selected
        positions (every selected entry's slot holds its position's bytes)."""
        w = self.w
        att = self.d_att[ai].cpu().numpy()
        for r in range(nr):
            pos = expand(self.trace[t, ai, r], w.block_tokens)
            recs = np.ascontiguousarray(self.ohost[r][l][pos.astype(np.int64)])
            K = oracle.attention.fp8_records_to_f64(recs) if self.fp8 else \
                oracle.attention.bf16_to_f64(recs.view(np.uint16))
            ref = oracle.attention.sparse_decode_attention_rows(q[r, l], K, SCALE)
            err = np.abs(att[r] - ref).max() / np.abs(ref).max()
            self.worst_attn = max(self.worst_attn, err)
            assert err <= 2e-3, ("attention", t, r, l, err)

    # ---- state comparison ---------------------------------------------------------------
    def check_state(self, layers=None, hot=True, page_table=True, requests=None):
        w = self.w
        torch.cuda.synchronize()
        layers = self.anchors if layers is None else layers
        requests = range(w.R) if requests is None else requests
        for l in layers:
            sp = torch.empty((w.R, w.B), dtype=torch.int32, device=self.dev)
            lru = torch.empty((w.R, w.B), dtype=torch.int32, device=self.dev)
            nw = torch.empty((w.R,), dtype=torch.int32, device=self.dev)
            ptx = torch.empty((w.R, self.lmax), dtype=torch.int32, device=self.dev) if page_table else None
            hk.hs_export_state(self.h, l, sp.data_ptr(), lru.data_ptr(), ptx.data_ptr() if page_table else 0,
                               nw.data_ptr(), self.compute.cuda_stream)
            torch.cuda.synchronize()
            sp, lru, nw = sp.cpu().numpy(), lru.cpu().numpy(), nw.cpu().numpy()
            if page_table:
                # the exported slots, and the raw 64-bit table's low halves, are the same
                pt = ptx.cpu().numpy()
                pt_addr = hk.hs_page_table(self.h, l)
                raw = torch.empty((w.R, self.lmax), dtype=torch.int64, device=self.dev)
                torch.cuda.synchronize()
                _copy_dev(pt_addr, raw)
                assert np.array_equal(page_table_slots(raw.cpu().numpy()), pt), ("page table export", l)
            for r in requests:
                st = self.caches[(r, l)].export()
                assert np.array_equal(sp[r], st["slot_pos"]), ("slot_pos", r, l)
                assert np.array_equal(lru[r], st["lru"]), ("lru", r, l)
                if w.append:
                    assert nw[r] == st["newest_pos"], ("newest", r, l)
                if page_table:
                    assert np.array_equal(pt[r], self.caches[(r, l)].page_table), ("page_table", r, l)
        if hot and self.compare_hot:
            self.check_hot(layers, requests)

    def check_hot(self, layers=None, requests=None):
        w = self.w
        torch.cuda.synchronize()
        layers = range(w.L) if layers is None else layers
        requests = range(w.R) if requests is None else requests
        for r in requests:
            for l in layers:
                a = l - l % w.group
                st = self.caches[(r, a)].export()
                occ = np.nonzero(st["slot_pos"] >= 0)[0]
                g = self.gpu.hot[r, l].cpu().numpy()
                ref = self.caches[(r, l)].hot if l == a else self.ohot_shared[(r, l)]
                if not np.array_equal(g[occ], ref[occ]):
                    bad = [int(s) for s in occ if not np.array_equal(g[s], ref[s])]
                    raise AssertionError("hot bytes differ r %d l %d: %d slots, first %s"
                                         % (r, l, len(bad), bad[:5]))
                # the bytes are the record of the position the slot holds (input generator)
                for s in occ[:: max(1, occ.size // 16)]:
                    assert np.array_equal(g[s], synth.record(r, l, int(st["slot_pos"][s]), self.rec)), (r, l, s)
                if w.append and st["newest_pos"] >= 0:
                    assert np.array_equal(g[w.B], synth.record(r, l, st["newest_pos"], self.rec))

    def close(self):
        torch.cuda.synchronize()
        self.pool.shutdown()
        self.gpu.close()


def page_table_slots(pt: np.ndarray) -> np.ndarray:
    """Slots of 64-bit page-table entries (the low 32 bits, int32; -1 = host only)."""
    return np.ascontiguousarray(pt).view(np.int32)[..., 0::2]


def _copy_dev(addr, dst: torch.Tensor):
    """Copy device memory at `addr` into `dst` (same byte size) with hipMemcpy via torch."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    rc = hip.hipMemcpy(dst.data_ptr(), addr, dst.numel() * dst.element_size(), 3)  # device to device
    assert rc == 0, rc
