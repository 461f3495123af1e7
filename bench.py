"""Benchmark of the per-layer RESOLVE hot path on one MI355X.

Workload (the headline): the batched decode step -- 32 requests x 16 layers,
32768-token contexts, 1152-byte bf16 records, k = 2048, B = 4096.  Per layer one
launch for all 32 requests resolves the selections (stage, mark, scan, fetch,
publish) and runs the sparse decode attention (16 heads) over the published
slots (hs_resolve_attn).  One step is all 16 layers.  Inputs (selection traces,
queries) are resident in HBM before the timed region starts.

Prints one JSON line.  `value` is resolved selections per second over the K
timed steps.  Also reported: the miss-fetch GB/s against the measured host-link
ceiling, the all-hit RESOLVE latency per layer (k = 2048, B = 4096) against the
launch bound, a roofline entry for the dominant kernel (against the host link,
which binds it here, and against HBM), the CPU oracle on this host's cores over
the same trace, and (without --quick) the other workloads and probes.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# the host link of an MI355X: PCIe 5.0 x16, 64 GB/s per direction (published)
HOST_LINK_PEAK_GBS = 64.0
REC = 1152


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=120)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the oracle timing")
    ap.add_argument("--quick", action="store_true", help="skip the secondary measurements")
    ap.add_argument("--measure", choices=sorted(SECONDARY), default=None,
                    help="run only this secondary measurement (and the 64 MiB copy that calibrates "
                         "the HBM-traffic counters) and print its figures as one JSON line")
    return ap.parse_args()


def addr(t, *idx):
    """Device address of t[idx] computed from the strides, without building the view (a
    torch view costs microseconds of host time per call, more than the launch it feeds)."""
    off = 0
    for i, st in zip(idx, t.stride()):
        off += i * st
    return t.data_ptr() + off * t.element_size()


def progress(msg):
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print("[bench] " + msg, file=sys.stderr, flush=True)


def sync_barrier(torch):
    torch.cuda.synchronize()


def profile_traffic(kernel: str, workload: str = "long"):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    (profiles/<kernel>_<workload>_traffic.txt), or None when the kernel's source changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
    h = hashlib.sha256()
    for src in rec.get("source_files", "").split():
        with open(os.path.join(ROOT, src), "rb") as g:
            h.update(g.read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return float(rec["bytes_per_launch"])


def profile_avg_us(kernel: str, workload: str = "long"):
    """Average duration of `kernel` in the committed rocprofv3 --kernel-trace --stats summary."""
    path = os.path.join(ROOT, "profiles", "kernel_trace_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        lines = f.readlines()
    for line in lines:  # the average over the timed steps' dispatches, where the summary gives it
        if line.startswith("timed_avg_us %s:" % kernel):
            return float(line.split(":", 1)[1])
    for line in lines:
        parts = line.split()
        if parts and not line.startswith("#") and \
                (parts[0] == kernel if "<" in kernel else parts[0].split("<")[0] == kernel):
            return float(parts[3])
    return None


def fill_pools(synth, cache, w, lmax):
    """The prefill records of every request into the library's pinned pool (the generator's C
    code runs several threads per request)."""
    for r in range(w.R):
        synth.fill_request(cache.host_pool_address(r), r, w.L, lmax, w.ctx)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: libhisparse has no multi-GPU path (each (request, layer) "
              "cache is independent; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import hierarchical_kv_cache_amd as hk
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.measure:
        calibration_copy(torch, hk, dev)
        print(json.dumps(SECONDARY[args.measure](torch, hk, synth, dev)))
        return
    t_start = time.time()
    # the host link's ceiling first (the headline's miss-fetch fraction is taken against it)
    link = measure_link(torch, hk, dev)
    progress("link ceiling %.1f GB/s" % link["ceiling_GBps"])
    w = synth.WORKLOADS["batched"].scaled(B=4096)
    head = batched_decode(torch, hk, synth, dev, w, args.warmup, args.steps, args)
    R, L, k, B = w.R, w.L, w.k, w.B
    K, W = args.steps, args.warmup
    detail = head["detail"]
    detail["link_ceiling_GBps"] = link["ceiling_GBps"]
    detail["link_dma_h2d_GBps"] = link["dma_GBps"]
    detail["link_zero_copy_GBps"] = link["zero_copy_GBps"]
    detail["link_random_records_GBps"] = link["random_records_GBps"]
    # the all-hit RESOLVE latency per layer at k 2048, B 4096 (part of the metric)
    detail.update(measure_all_hit(torch, hk, synth, dev))
    progress("all-hit RESOLVE %.2f / %.2f us per layer (1 / 32 requests)"
             % (detail["all_hit_us_per_layer_r1"], detail["all_hit_us_per_layer_r32"]))

    # ---- secondary measurements --------------------------------------------------------
    if args.quick:
        calibration_copy(torch, hk, dev)
    else:
        detail["long_decode"] = measure_long_decode(torch, hk, synth, dev)
        progress("long decode %.1f M selections/s" % (detail["long_decode"]["selections_per_s"] / 1e6))
        for fn in (measure_fetch, measure_fetch_heavy, measure_resident, measure_fp8, measure_rows, measure_short,
                   measure_capacity, measure_replay, measure_attention, measure_shared_step):
            detail.update(fn(torch, hk, synth, dev))
            progress(fn.__name__ + " done")
        detail["launch_latency_us"] = measure_empty(torch, hk)
        detail.update(measure_hbm(torch, hk, dev))
        detail["attention_r32_frac_of_scattered_read"] = (detail["attention_r32_GBps"]
                                                          / detail["hbm_scattered_records_read_GBps"])
        for key in ("batched_cold_fetch_GBps", "long_cold_fetch_GBps", "capacity_cold_fetch_GBps",
                    "capacity_steady_fetch_GBps", "replay_cold_GBps", "replay_steady_GBps",
                    "replay_cold_kernels_GBps", "replay_steady_kernels_GBps"):
            detail[key.replace("GBps", "frac_of_link")] = detail[key] / link["ceiling_GBps"]

    # ---- roofline of the dominant kernel -------------------------------------------------
    # The fused RESOLVE + attention kernel is the longest kernel of the step (the finish
    # kernel is short; see the kernel trace).  Per launch it moves, for each of the R requests:
    # over the host link the m missed records (m x 1152 bytes); in HBM the selection in and the
    # slots out, the slot map and LRU order read and written, the k - m hit records read, the m
    # missed records and their two page-table entries written, the queries in and the output
    # out.  The staging of the misses and the chunk partials are implementation choices and
    # are not counted.  At 32 requests the link carries the binding share.
    kern_us = head["kern_us"]
    t_us = statistics.fmean(kern_us)
    m_req = head["misses_timed"] / (K * L * R)  # misses per (request, layer) launch share
    link_bytes = R * m_req * REC
    hbm_bytes = R * (k * 4 + B * 4 * 2 + B * 2 * 2 + k * 4 + (k - m_req) * REC + m_req * (REC + 8 + 8)
                     + w.heads * 576 * 2 + w.heads * 512 * 4)
    link_gbs = link_bytes / (t_us * 1e-6) / 1e9
    hbm_gbs = hbm_bytes / (t_us * 1e-6) / 1e9
    kname = "resolve_kernel<4,2,true>"
    hbm = {"achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": hbm_gbs / HBM_PEAK_GBS,
           "algorithmic_bytes_per_launch": hbm_bytes, "traffic": profile_traffic("resolve_attn_kernel", "batched")}
    roof = {"kernel": kname, "bound": "link", "achieved": link_gbs, "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
            "frac": link_gbs / HOST_LINK_PEAK_GBS, "traffic": hbm["traffic"],
            "algorithmic_bytes_per_launch": link_bytes,
            "frac_of_measured_link_ceiling": link_gbs / link["ceiling_GBps"],
            "measured_link_ceiling_GBps": link["ceiling_GBps"],
            "avg_launch_us_kernel_events": t_us, "avg_launch_us_rocprof": profile_avg_us(kname, "batched"),
            "hbm": hbm}
    if hbm["frac"] > roof["frac"]:  # (not at this shape: reported for completeness)
        roof["bound"] = "hbm"

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_batched(synth, w, head, W, K, args.cpu_seconds)
        progress("oracle %.2f M selections/s on %d threads" % (cpu["value"] / 1e6, cpu["cores"]))
        if not args.quick:
            detail["configs"] = cpu_baseline_configs(torch, hk, synth, dev)
            for row in detail["configs"]:
                row["gpu_miss_frac_of_link"] = row["gpu_miss_GBps"] / link["ceiling_GBps"]
    head["cache"].close()

    value = head["value"]
    line = {
        "metric": "resolved selections/s",
        "value": value,
        "unit": "selections/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": head["elapsed"] / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32 index + bf16 records (fp32 attention accumulate)",
        "data": "synthetic (seeded selection traces; counter-based N(0,1) bf16 records and queries)",
        "config": {"workload": "batched decode: 32 requests x 16 layers, ctx 32768, k 2048, B 4096; per layer one "
                               "launch for all requests of RESOLVE + sparse decode attention (16 heads) over "
                               "the published slots",
                   "requests": R, "layers": L, "ctx": w.ctx, "top_k": k, "buffer_slots": B,
                   "record_bytes": REC, "heads": w.heads, "parallelism": "single GPU"},
        "metric_parts": {
            "resolved_selections_per_s": value,
            "miss_fetch_GBps_fused_kernel": link_gbs,
            "miss_fetch_frac_of_link_ceiling": link_gbs / link["ceiling_GBps"],
            "miss_fetch_GBps_whole_step": detail["steady_link_GBps"],
            "link_ceiling_GBps": link["ceiling_GBps"],
            "all_hit_resolve_us_per_layer_r1": detail["all_hit_us_per_layer_r1"],
            "all_hit_resolve_us_per_layer_r32": detail["all_hit_us_per_layer_r32"],
            "launch_latency_bound_us": detail.get("launch_latency_us"),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": detail,
        "bench_wall_s": round(time.time() - t_start, 1),
    }
    print(json.dumps(line))


def batched_decode(torch, hk, synth, dev, w, W, K, args, passes=("timing", "separate")):
    """The headline: the batched decode step (32 requests x 16 layers, ctx 32768, k 2048,
    B 4096, 16 heads).  A step resolves every layer for all requests in one launch and attends
    over the published slots (hs_resolve_attn: the fused kernel, then the finish kernel).
    Inputs (selection traces, queries) are resident in HBM and every step's buffer addresses
    are computed before the timed region.  W warmup steps, then K timed steps with nothing
    between kernels.  Further passes from the same empty start (hs_reset_request): every fused
    kernel stamped by its own start and end, and the separate calls (hs_resolve +
    hs_sparse_attn), which must resolve identically."""
    R, L, k, B, heads = w.R, w.L, w.k, w.B, w.heads
    n = W + K
    lmax = w.max_positions(n)
    scale = 576 ** -0.5
    t_in = time.time()
    cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B))
    fill_pools(synth, cache, w, lmax)
    t_fill = time.time() - t_in
    progress("batched: host pool %.1f GB filled in %.1f s" % (w.host_bytes(n) / 1e9, t_fill))
    trace = np.stack([np.stack([synth.selection_trace(w, r, l, n) for r in range(R)], axis=1)
                      for l in range(L)], axis=1)  # [n][L][R][k]
    d_trace = torch.from_numpy(trace).to(dev)
    d_q = torch.empty((n, L, R, heads, 576), dtype=torch.int16, device=dev)
    for t in range(n):  # [R][L][H][576] per step, stored [L][R][H][576]
        d_q[t].copy_(torch.from_numpy(synth.queries(R, L, t, heads=heads).view(np.int16)).permute(1, 0, 2, 3))
    d_ctx = torch.full((R,), w.ctx, dtype=torch.int32, device=dev)
    d_slots = torch.empty((L, R, k), dtype=torch.int32, device=dev)
    d_stats = torch.zeros((n, L, R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    d_out = torch.empty((L, R, heads, 512), dtype=torch.float32, device=dev)
    compute = torch.cuda.current_stream()
    cs = compute.cuda_stream
    a_sel = [[addr(d_trace, t, l) for l in range(L)] for t in range(n)]
    a_q = [[addr(d_q, t, l) for l in range(L)] for t in range(n)]
    a_stats = [[addr(d_stats, t, l) for l in range(L)] for t in range(n)]
    a_slots = [addr(d_slots, l) for l in range(L)]
    a_out = [addr(d_out, l) for l in range(L)]
    a_ctx = d_ctx.data_ptr()
    torch.cuda.synchronize()
    input_s = time.time() - t_in
    progress("batched: inputs resident in HBM after %.1f s" % input_s)
    h = cache.h

    def step(t, fused=True):
        sel, q, st = a_sel[t], a_q[t], a_stats[t]
        for l in range(L):
            if fused:
                hk.hs_resolve_attn(h, l, sel[l], a_ctx, a_slots[l], st[l], 0, 0, q[l], heads, 512, a_out[l],
                                   scale, cs)
            else:
                hk.hs_resolve(h, l, sel[l], a_ctx, a_slots[l], st[l], 0, 0, cs)
                hk.hs_sparse_attn(h, l, q[l], heads, 512, a_slots[l], a_out[l], scale, 0, cs)

    def reset():
        for r in range(R):
            hk.hs_reset_request(h, r, cs)
        d_stats.zero_()
        torch.cuda.synchronize()

    def value_pass(fused=True):
        for t in range(W):
            step(t, fused)
        sync_barrier(torch)
        t0 = time.perf_counter()
        for i in range(K):
            step(W + i, fused)
        t_enq = time.perf_counter() - t0
        sync_barrier(torch)
        return time.perf_counter() - t0, t_enq

    fused = hk.hs_resolve_attn_wgs(h) > 0
    elapsed, enqueue = value_pass()
    progress("batched: %.1f M selections/s, %.3f ms per step" % (K * L * R * k / elapsed / 1e6, elapsed / K * 1e3))
    stats = d_stats.cpu().numpy()
    out_fused = d_out.clone()
    kern_us, elapsed_sep, att_dev = [elapsed / (K * L) * 1e6], float("nan"), float("nan")
    if "timing" in passes:  # kernel durations of the fused kernel, the same steps from the same empty start
        reset()
        for t in range(W):
            step(t)
        hk.hs_timing_start(h, K * L)
        for i in range(K):
            step(W + i)
        sync_barrier(torch)
        kern_us = [float(x) for x in hk.hs_timing_read(h, K * L)]
        assert len(kern_us) == K * L
        assert np.array_equal(d_stats.cpu().numpy(), stats), "the timing pass resolved differently"
        assert torch.equal(d_out, out_fused), "the timing pass attended differently"
    if "separate" in passes:  # the separate calls (hs_resolve + hs_sparse_attn), the same steps
        reset()
        elapsed_sep, _ = value_pass(fused=False)
        assert np.array_equal(d_stats.cpu().numpy(), stats), "the separate calls resolved differently"
        att_dev = float((d_out - out_fused).abs().max() / out_fused.abs().max())
    assert not stats[..., 2].any(), "error bits set"
    misses_timed = int(stats[W:, :, :, 1].sum())
    hits_timed = int(stats[W:, :, :, 0].sum())
    fetched = stats[W:, :, :, 4].astype(np.uint32).astype(np.int64) + \
        (stats[W:, :, :, 5].astype(np.uint32).astype(np.int64) << 32)
    assert int(fetched.sum()) == misses_timed * REC, "bytes_fetched disagrees with misses"
    selections = K * L * R * k
    # occupied slots evicted in the timed steps (empty slots are taken first)
    occ = np.minimum(B, np.cumsum(stats[:, :, :, 1], axis=0))
    before = np.concatenate([np.zeros_like(occ[:1]), occ[:-1]])
    evicted = np.maximum(0, stats[:, :, :, 1] - (B - before))
    detail = {
        "path": "hs_resolve_attn (fused RESOLVE + attention kernel, then the finish kernel)" if fused
                else "hs_resolve_attn (two calls: no fused kernel for this configuration)",
        "fused_wgs_per_request": hk.hs_resolve_attn_wgs(h),
        "host_enqueue_us_per_step": enqueue / K * 1e6,
        "fused_kernel_us_per_layer_mean": statistics.fmean(kern_us),
        "fused_kernel_us_per_layer_median": statistics.median(kern_us),
        "fused_kernel_us_p90": float(np.percentile(kern_us, 90)),
        "separate_selections_per_s": selections / elapsed_sep,
        "separate_ms_per_step": elapsed_sep / K * 1e3,
        "fused_vs_separate_attention_max_rel_diff": att_dev,
        "miss_rate": misses_timed / max(1, misses_timed + hits_timed),
        "misses_per_launch": misses_timed / (K * L),
        "steady_link_GBps": misses_timed * REC / elapsed / 1e9,
        "occupied_slots_evicted_timed": int(evicted[W:].sum()),
        "first_step_evicting": int(np.argmax(evicted.sum(axis=(1, 2)) > 0)) + 1,
        "cold_step_misses": int(stats[0, :, :, 1].sum()),
        "host_pool_GB": w.host_bytes(n) / 1e9,
        "host_pool_fill_s": round(t_fill, 1),
        "input_setup_s": round(input_s, 1),
    }
    return {"value": selections / elapsed, "elapsed": elapsed, "kern_us": kern_us, "stats": stats,
            "trace": trace, "misses_timed": misses_timed, "detail": detail, "cache": cache, "lmax": lmax}


def measure_headline(torch, hk, synth, dev, W=8, K=24):
    """The headline's decode steps (batched, hs_resolve_attn) alone: W warmup + K steps, no
    timing or separate-call pass (for the profiler's counter passes)."""
    import types
    w = synth.WORKLOADS["batched"].scaled(B=4096)
    head = batched_decode(torch, hk, synth, dev, w, W, K, types.SimpleNamespace(), passes=())
    head["cache"].close()
    return {"headline_selections_per_s": head["value"], "headline_ms_per_step": head["elapsed"] / K * 1e3,
            "steps": K, "warmup": W}


def measure_long_decode(torch, hk, synth, dev, W=8, K=64):
    """The long-request decode step (1 request x 8 layers, ctx 131072, k 2048, B 4096): the
    write-through of the new token, then per layer hs_resolve_attn.  The write-through as one
    kernel on the compute stream, and on a backup stream with its event pair (the pages'
    layout); fused kernels stamped by their own start and end; the separate calls."""
    w = synth.WORKLOADS["long"]
    R, L, k, B = w.R, w.L, w.k, w.B
    n = W + K
    lmax = w.max_positions(n)
    heads, scale = w.heads, 576 ** -0.5
    cfg = hk.make_config(R, L, lmax, k, B, newest_slot=True)
    trace = np.stack([np.stack([synth.selection_trace(w, r, l, n) for r in range(R)], axis=1)
                      for l in range(L)], axis=1)  # [n][L][R][k]
    d_trace = torch.from_numpy(trace).to(dev)
    new_pos = w.ctx + np.arange(n)
    d_new_kv = torch.from_numpy(np.stack([synth.records_at(R, L, [p] * R) for p in new_pos])).to(dev)
    d_new_pos = torch.from_numpy(np.repeat(new_pos[:, None], R, axis=1).astype(np.int32)).to(dev)
    d_ctx = torch.from_numpy((new_pos[:, None] + 1).repeat(R, axis=1).astype(np.int32)).to(dev)
    d_q = torch.from_numpy(np.stack([synth.queries(R, L, t, heads=heads) for t in range(n)])
                           .view(np.int16)).to(dev).permute(0, 2, 1, 3, 4).contiguous()
    d_slots = torch.empty((L, R, k), dtype=torch.int32, device=dev)
    d_stats = torch.zeros((n, L, R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    d_out = torch.empty((L, R, heads, 512), dtype=torch.float32, device=dev)
    compute = torch.cuda.current_stream()
    backup = torch.cuda.Stream()
    cs, bs = compute.cuda_stream, backup.cuda_stream
    a_sel = [[addr(d_trace, t, l) for l in range(L)] for t in range(n)]
    a_q = [[addr(d_q, t, l) for l in range(L)] for t in range(n)]
    a_stats = [[addr(d_stats, t, l) for l in range(L)] for t in range(n)]
    a_ctx = [addr(d_ctx, t) for t in range(n)]
    a_kv = [addr(d_new_kv, t) for t in range(n)]
    a_pos = [addr(d_new_pos, t) for t in range(n)]
    a_slots = [addr(d_slots, l) for l in range(L)]
    a_out = [addr(d_out, l) for l in range(L)]

    def fresh():
        c = hk.HiSparse(cfg)
        for r in range(R):
            synth.fill_request(c.host_pool_address(r), r, L, lmax, w.ctx)
        return c

    def step(c, t, fused=True, backup_stream=False):
        hk.hs_writeback(c.h, a_kv[t], a_pos[t], cs, bs if backup_stream else cs)
        for l in range(L):
            if fused:
                hk.hs_resolve_attn(c.h, l, a_sel[t][l], a_ctx[t], a_slots[l], a_stats[t][l], 0, 0, a_q[t][l], heads,
                                   512, a_out[l], scale, cs)
            else:
                hk.hs_resolve(c.h, l, a_sel[t][l], a_ctx[t], a_slots[l], a_stats[t][l], 0, 0, cs)
                hk.hs_sparse_attn(c.h, l, a_q[t][l], heads, 512, a_slots[l], a_out[l], scale, 0, cs)

    def run(fused=True, backup_stream=False, timed=False):
        c = fresh()
        d_stats.zero_()
        for t in range(W):
            step(c, t, fused, backup_stream)
        sync_barrier(torch)
        if timed:
            hk.hs_timing_start(c.h, K * L)
        t0 = time.perf_counter()
        for i in range(K):
            step(c, W + i, fused, backup_stream)
        sync_barrier(torch)
        el = time.perf_counter() - t0
        backup.synchronize()
        kern = [float(x) for x in hk.hs_timing_read(c.h, K * L)] if timed else None
        c.close()
        return el, kern, d_stats.cpu().numpy()

    el, _, st = run()
    out_fused = d_out.clone()
    el_bs, _, st_bs = run(backup_stream=True)
    assert np.array_equal(st, st_bs) and torch.equal(d_out, out_fused), "backup-stream pass differs"
    _, kern, st_t = run(timed=True)
    assert np.array_equal(st, st_t)
    el_sep, _, st_sep = run(fused=False)
    assert np.array_equal(st, st_sep)
    sel = K * L * R * k
    m = int(st[W:, ..., 1].sum())
    return {"workload": "long request: 1 req x 8 layers, ctx 131072, k 2048, B 4096, write-through + sparse "
                        "attention (16 heads)",
            "selections_per_s": sel / el, "ms_per_step": el / K * 1e3,
            "write_through_backup_stream_selections_per_s": sel / el_bs,
            "write_through_backup_stream_ms_per_step": el_bs / K * 1e3,
            "fused_kernel_us_per_layer_mean": statistics.fmean(kern),
            "fused_kernel_us_per_layer_median": statistics.median(kern),
            "separate_selections_per_s": sel / el_sep,
            "miss_rate": m / (K * L * R * k), "misses_per_layer_step": m / (K * L * R),
            "steps": K, "warmup": W}


def cpu_baseline_batched(synth, w, head, W, K, budget_s):
    """The oracle as it stands, on this host's cores, over the headline's trace: one oracle
    cache per (request, layer), the same empty start, the W warmup steps resolved untimed
    (RESOLVE only: they only build the state), then the timed steps that fit the budget, each
    a RESOLVE and a float64 attention over the selected records per (request, layer).  The
    oracle reads the records from the library's pinned pool (RESOLVE never writes it).  Its
    miss counts must equal the GPU's for every (step, layer, request) it ran.  One thread per
    cache up to the host's cores (at most 16), then one thread."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    import oracle

    R, L, k, B = w.R, w.L, w.k, w.B
    trace, stats, cache, lmax = head["trace"], head["stats"], head["cache"], head["lmax"]
    pools = [cache.host_pool(r) for r in range(R)]

    def leg(threads, budget):
        caches = {(r, l): oracle.Cache(B, lmax, REC) for r in range(R) for l in range(L)}
        pool = ThreadPoolExecutor(max_workers=threads)

        def layer_step(args):
            t, r, l, q, attend = args
            c = caches[(r, l)]
            out, _, m, _, _ = c.resolve(trace[t, l, r], w.ctx, pools[r][l])
            if attend:
                oracle.attention.sparse_decode_attention(q[r, l], c.hot, out, 576 ** -0.5)
            return m

        def run_step(t, attend):
            q = synth.queries(R, L, t, heads=w.heads) if attend else None
            jobs = [(t, r, l, q, attend) for l in range(L) for r in range(R)]
            return np.array(list(pool.map(layer_step, jobs))).reshape(L, R)

        for t in range(W):
            run_step(t, False)
        done = 0
        t0 = time.perf_counter()
        while done < K and time.perf_counter() - t0 < budget:
            m = run_step(W + done, True)
            assert np.array_equal(m, stats[W + done, :, :, 1]), "oracle and GPU misses differ"
            done += 1
        el = time.perf_counter() - t0
        pool.shutdown()
        for c in caches.values():
            c.close()
        return done * L * R * k / el, done

    threads = min(L * R, os.cpu_count() or 1, 16)
    with threadpool_limits(limits=1):
        value, done = leg(threads, budget_s)
        value1, done1 = leg(1, budget_s / 2)
    return {"value": value, "unit": "selections/s", "cores": threads, "kind": "oracle",
            "sample": "%d of the %d timed decode steps (after the same %d warmup steps, resolved untimed), all "
                      "%d layers x %d requests; RESOLVE + float64 attention per (request, layer); misses "
                      "checked equal to the GPU's" % (done, K, W, L, R),
            "single_thread_value": value1,
            "single_thread_sample": "the first %d timed steps, same start, one thread" % done1,
            "host_cpu": host_cpu(), "nproc": os.cpu_count()}


def calibration_copy(torch, hk, dev):
    """One plain copy of known size (64 MiB): the calibration kernel of the HBM-traffic counters."""
    a = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    hk.hs_probe_copy(a.data_ptr(), b.data_ptr(), a.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    del a, b


def measure_link(torch, hk, dev):
    """Host-link ceiling: max of a DMA copy and a zero-copy streaming read, 1 GiB pinned."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    sink = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream()
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    e1.record(s)
    torch.cuda.synchronize()
    dma = 3 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    hk.hs_probe_host_read(src.data_ptr(), n, sink.data_ptr(), 256, s.cuda_stream)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(3):
        hk.hs_probe_host_read(src.data_ptr(), n, sink.data_ptr(), 256, s.cuda_stream)
    e1.record(s)
    torch.cuda.synchronize()
    zc = 3 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # scattered 1152-byte records: 65536 distinct records at random places in the same buffer
    nrec = 65536
    idx = np.random.Generator(np.random.PCG64(7)).choice(n // REC, size=nrec, replace=False).astype(np.int32)
    d_idx = torch.from_numpy(idx).to(dev)
    d_rec = torch.empty((nrec, REC), dtype=torch.uint8, device=dev)
    hk.hs_probe_host_records(src.data_ptr(), n // REC, REC, d_idx.data_ptr(), nrec, d_rec.data_ptr(), 1024,
                             s.cuda_stream)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(3):
        hk.hs_probe_host_records(src.data_ptr(), n // REC, REC, d_idx.data_ptr(), nrec, d_rec.data_ptr(), 1024,
                                 s.cuda_stream)
    e1.record(s)
    torch.cuda.synchronize()
    rec = 3 * nrec * REC / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return {"dma_GBps": dma, "zero_copy_GBps": zc, "ceiling_GBps": max(dma, zc), "random_records_GBps": rec}


def run_resolve_only(torch, hk, synth, w, dev, trace, lmax, steps, flags, resident=None, cache=None):
    """RESOLVE alone over `steps` steps of a trace on a fresh cache; per-launch µs per step.
    With `resident` (a ResidentSpec) a resident tier is bound and its block table follows
    the spec's per-step layout (table rewrites are outside the timed launches).  `cache`: a
    fresh, filled handle to use (and leave open) instead of a new one."""
    R, L, k, B = w.R, w.L, w.k, w.B
    own = cache is None
    if own:
        cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B, block_tokens=w.block_tokens, newest_slot=w.append))
        for r in range(R):
            synth.fill_request(cache.host_pool_address(r), r, L, lmax, w.ctx)
    if resident is not None:
        from synth.resident import resident_layout
        P = resident.page_tokens
        phys, masks, total = resident_layout(w, steps, resident, max_positions=lmax)
        rows = max(1, total) * P
        d_pool = torch.empty((L, rows, REC), dtype=torch.uint8, device=dev)  # never read by RESOLVE
        d_tables = torch.from_numpy(np.where(masks, phys[None], -1).astype(np.int32)).to(dev)
        d_table = torch.empty_like(d_tables[0])
        hk.hs_bind_resident(cache.h, d_table.data_ptr(), phys.shape[1], P, d_pool.data_ptr(), rows)
    d_trace = torch.from_numpy(np.ascontiguousarray(trace[:steps])).to(dev)
    d_slots = torch.empty((R, k), dtype=torch.int32, device=dev)
    d_stats = torch.zeros((steps, L, R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    ctx = torch.from_numpy((w.ctx + 1 + np.arange(steps))[:, None].repeat(R, 1).astype(np.int32)).to(dev) \
        if w.append else torch.full((steps, R), w.ctx, dtype=torch.int32, device=dev)
    if w.append:
        pos = w.ctx + np.arange(steps)
        new_kv = torch.from_numpy(np.stack([synth.records_at(R, L, [p] * R) for p in pos])).to(dev)
        new_pos = torch.from_numpy(pos[:, None].repeat(R, 1).astype(np.int32)).to(dev)
    torch.cuda.synchronize()
    hk.hs_timing_start(cache.h, steps * L)  # every launch stamped by its own start and end
    for t in range(steps):
        if resident is not None:
            d_table.copy_(d_tables[t])
        if w.append:
            hk.hs_writeback(cache.h, new_kv[t].data_ptr(), new_pos[t].data_ptr(), s.cuda_stream, s.cuda_stream)
        for l in range(L):
            hk.hs_resolve(cache.h, l, d_trace[t, l].data_ptr(), ctx[t].data_ptr(), d_slots.data_ptr(),
                          d_stats[t, l].data_ptr(), 0, flags, s.cuda_stream)
    torch.cuda.synchronize()
    us = hk.hs_timing_read(cache.h, steps * L).astype(np.float64).reshape(steps, L)
    st = d_stats.cpu().numpy()
    if own:
        cache.close()
    return us, st


def long_trace(synth, steps):
    """The long request's workload (one token appended per step), its trace [steps][L][R][k]
    and its pool size in positions."""
    w = synth.WORKLOADS["long"]
    trace = np.stack([np.stack([synth.selection_trace(w, r, l, steps) for r in range(w.R)], axis=1)
                      for l in range(w.L)], axis=1)
    return w, trace, w.max_positions(steps)


def measure_fetch(torch, hk, synth, dev):
    """IO cost inside RESOLVE on identical metadata states (the same trace from the same empty
    start, run once normally and once with SKIP_IO), for the long workload.  The cold step's
    fetch rate is its miss bytes over the whole RESOLVE kernel (a lower bound on the link rate
    reached: the metadata stages count as transfer time); the difference to the SKIP_IO
    kernel only says how much of the kernel the IO adds, since the fetch overlaps stages 1-3."""
    steps = 64
    w, trace, lmax = long_trace(synth, steps)
    us_io, st = run_resolve_only(torch, hk, synth, w, dev, trace, lmax, steps, 0)
    us_skip, st2 = run_resolve_only(torch, hk, synth, w, dev, trace, lmax, steps, hk.HS_SKIP_IO)
    # the same counts (bytes_fetched differs: the no-IO pass moves no bytes)
    assert np.array_equal(st[..., :4], st2[..., :4]) and not st2[..., 4:].any()
    miss_bytes = st[..., 1].sum(axis=2) * REC  # [steps][L]
    return {"long_cold_resolve_us_per_layer": float(us_io[0].mean()),
            "long_cold_resolve_skip_io_us_per_layer": float(us_skip[0].mean()),
            "long_cold_fetch_GBps": float(miss_bytes[0].sum() / (us_io[0].sum() * 1e-6) / 1e9),
            "long_cold_io_added_us_per_layer": float((us_io[0] - us_skip[0]).mean()),
            "long_steady_resolve_us_per_layer": float(us_io[8:].mean()),
            "long_steady_resolve_skip_io_us_per_layer": float(us_skip[8:].mean()),
            "long_steady_miss_bytes_per_layer": float(miss_bytes[8:].mean())}


def measure_fetch_heavy(torch, hk, synth, dev):
    """The fetch-heavy launch: 32 requests, cold (every one of the 32 x 2048 entries misses),
    75.5 MB through the host link in one RESOLVE launch."""
    wl = synth.WORKLOADS["batched"].scaled(L=1)
    tr = np.stack([np.stack([synth.selection_trace(wl, r, 0, 2) for r in range(wl.R)], axis=1)], axis=1)
    us_io, st = run_resolve_only(torch, hk, synth, wl, dev, tr, wl.max_positions(2), 2, 0)
    us_skip, _ = run_resolve_only(torch, hk, synth, wl, dev, tr, wl.max_positions(2), 2, hk.HS_SKIP_IO)
    b = float(st[0, :, :, 1].sum() * REC)
    return {"batched_cold_launch_bytes": b,
            "batched_cold_resolve_us": float(us_io[0, 0]),
            "batched_cold_resolve_skip_io_us": float(us_skip[0, 0]),
            "batched_cold_fetch_GBps": b / (us_io[0, 0] * 1e-6) / 1e9,
            "batched_cold_io_added_us": float(us_io[0, 0] - us_skip[0, 0])}


def measure_capacity(torch, hk, synth, dev, steps=24):
    """Block selections (32 blocks of 64 tokens, 4 requests, 1,048,576-token context, B = 4096),
    one layer: the cold launch (every token misses) and the steady state, miss bytes over the
    whole RESOLVE kernel."""
    wl = synth.WORKLOADS["capacity"].scaled(L=1)
    tr = np.stack([np.stack([synth.selection_trace(wl, r, 0, steps) for r in range(wl.R)], axis=1)], axis=1)
    us, st = run_resolve_only(torch, hk, synth, wl, dev, tr, wl.max_positions(steps), steps, 0)
    miss_bytes = st[:, 0, :, 1].sum(axis=1) * REC  # [steps]
    return {"capacity_cold_launch_bytes": float(miss_bytes[0]),
            "capacity_cold_resolve_us": float(us[0, 0]),
            "capacity_cold_fetch_GBps": float(miss_bytes[0] / (us[0, 0] * 1e-6) / 1e9),
            "capacity_steady_resolve_us": float(np.median(us[2:, 0])),
            "capacity_steady_miss_rate": float(st[2:, 0, :, 1].sum() / (st[2:, 0, :, :2].sum())),
            "capacity_steady_fetch_GBps": float(miss_bytes[2:].sum() / (us[2:, 0].sum() * 1e-6) / 1e9)}


def measure_replay(torch, hk, synth, dev, steps=12):
    """Shared-layer replay: 16 requests, one anchor and its three shared layers, 131072-token
    context, k = 2048, B = 4096.  Each step resolves the anchor with the miss plan recorded,
    then times hs_prefetch_shared (three copy-only replay launches on the prefetch stream)
    with events on that stream, and each replay kernel by its own start and end: plan bytes
    (3 x misses x 1152) per second of the call and of the three kernels, cold and steady."""
    wl = synth.WORKLOADS["shared"].scaled(L=4)
    R, k, B = wl.R, wl.k, wl.B
    lmax = wl.max_positions(steps)
    cache = hk.HiSparse(hk.make_config(R, wl.L, lmax, k, B, layer_group=wl.group))
    for r in range(R):
        synth.fill_request(cache.host_pool_address(r), r, wl.L, lmax, wl.ctx)
    tr = np.stack([synth.selection_trace(wl, r, 0, steps) for r in range(R)], axis=1)  # [steps][R][k]
    d_tr = torch.from_numpy(tr).to(dev)
    d_ctx = torch.full((R,), wl.ctx, dtype=torch.int32, device=dev)
    d_slots = torch.empty((R, k), dtype=torch.int32, device=dev)
    d_stats = torch.zeros((steps, R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    cs = torch.cuda.current_stream()
    ps = torch.cuda.Stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    hk.hs_timing_start(cache.h, steps * 4)  # per step: the anchor's RESOLVE, then three replays
    for t in range(steps):
        hk.hs_resolve(cache.h, 0, d_tr[t].data_ptr(), d_ctx.data_ptr(), d_slots.data_ptr(), d_stats[t].data_ptr(),
                      0, hk.HS_RECORD_PLAN, cs.cuda_stream)
        torch.cuda.synchronize()
        ev[t][0].record(ps)
        hk.hs_prefetch_shared(cache.h, 0, cs.cuda_stream, ps.cuda_stream)
        ev[t][1].record(ps)
        torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    kern = hk.hs_timing_read(cache.h, steps * 4).astype(np.float64).reshape(steps, 4)[:, 1:].sum(axis=1)
    st = d_stats.cpu().numpy()
    cache.close()
    assert not st[..., 2].any()
    plan_bytes = 3 * st[:, :, 1].sum(axis=1) * REC  # [steps]
    return {"replay_cold_bytes": float(plan_bytes[0]),
            "replay_cold_us": float(us[0]),
            "replay_cold_GBps": float(plan_bytes[0] / (us[0] * 1e-6) / 1e9),
            "replay_cold_kernels_GBps": float(plan_bytes[0] / (kern[0] * 1e-6) / 1e9),
            "replay_steady_us": float(np.median(us[2:])),
            "replay_steady_bytes": float(plan_bytes[2:].mean()),
            "replay_steady_GBps": float(plan_bytes[2:].sum() / (us[2:].sum() * 1e-6) / 1e9),
            "replay_steady_kernel_us": float(np.median(kern[2:]) / 3),
            "replay_steady_kernels_GBps": float(plan_bytes[2:].sum() / (kern[2:].sum() * 1e-6) / 1e9)}


def measure_all_hit(torch, hk, synth, dev):
    """All-hit RESOLVE µs per layer at k = 2048, B = 4096: after one warm step every step
    repeats the selection.  Single request (long shape) and 32 requests (batched shape)."""
    out = {}
    for name, wl in (("r1", synth.WORKLOADS["long"].scaled(append=False, force_newest=False, L=4)),
                     ("r32", synth.WORKLOADS["batched"].scaled(L=1))):
        steps = 128
        tr = np.stack([np.stack([synth.selection_trace(wl, r, l, steps, all_hit=True) for r in range(wl.R)],
                                axis=1) for l in range(wl.L)], axis=1)
        us, st = run_resolve_only(torch, hk, synth, wl, dev, tr, wl.max_positions(steps), steps, 0)
        assert st[1:, :, :, 1].sum() == 0
        out["all_hit_us_per_layer_%s" % name] = float(np.median(us[2:]))
        # algorithmic HBM bytes of an all-hit launch: selection, slot map + LRU read and written, slots
        b = wl.R * (wl.k * 4 * 2 + wl.B * (4 + 2) * 2)
        out["all_hit_hbm_bound_us_%s" % name] = b / (HBM_PEAK_GBS * 1e9) * 1e6
    return out


def measure_resident(torch, hk, synth, dev):
    """Resident tier in front of the hot slots.  All resident (a short request that fits the
    device pool): the kernel returns after the block-table lookup, at 1 and 32 requests.
    Long workload with the last 16384 prefill tokens and 5 % of older pages resident:
    steady-state µs per layer and the share of entries the resident tier serves."""
    from synth.resident import ResidentSpec
    out = {}
    for name, wl in (("r1", synth.WORKLOADS["long"].scaled(append=False, force_newest=False, L=4,
                                                           ctx=32768)),
                     ("r32", synth.WORKLOADS["batched"].scaled(L=1))):
        steps = 64
        tr = np.stack([np.stack([synth.selection_trace(wl, r, l, steps) for r in range(wl.R)], axis=1)
                       for l in range(wl.L)], axis=1)
        us, st = run_resolve_only(torch, hk, synth, wl, dev, tr, wl.max_positions(steps), steps, 0,
                                  resident=ResidentSpec(all_resident=True))
        assert (st[..., 3] == wl.k).all() and st[..., 1].sum() == 0
        out["all_resident_us_per_layer_%s" % name] = float(np.median(us[1:]))
    steps = 64
    w, trace, lmax = long_trace(synth, steps)
    us, st = run_resolve_only(torch, hk, synth, w, dev, trace, lmax, steps, 0,
                              resident=ResidentSpec(window_tokens=16384, old_frac=0.05))
    out["long_resident_steady_us_per_layer"] = float(us[8:].mean())
    out["long_resident_share"] = float(st[8:, ..., 3].sum() / (st[8:].shape[0] * w.L * w.R * w.k))
    out["long_resident_miss_rate"] = float(st[8:, ..., 1].sum() / (st[8:].shape[0] * w.L * w.R * w.k))
    return out


def measure_fp8(torch, hk, synth, dev, steps=40, warmup=8):
    """The long-request step (write-through, RESOLVE, attention over 8 layers) with FP8 latent-KV
    records (656 bytes: E4M3 codes, block scales, bf16 rope): whole-step throughput through
    hs_resolve_attn (the fused kernel over FP8 tiles), and through hs_resolve + hs_sparse_attn
    from the same empty start."""
    w = synth.WORKLOADS["long"]
    R, L, k, B = w.R, w.L, w.k, w.B
    n = steps + warmup
    lmax = w.max_positions(n)
    rec = synth.FP8_RECORD_BYTES
    cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B, newest_slot=True, fp8=True))
    for r in range(R):
        synth.fill_request(cache.host_pool_address(r), r, L, lmax, w.ctx, rec_bytes=rec)
    trace = np.stack([np.stack([synth.selection_trace(w, r, l, n) for r in range(R)], axis=1)
                      for l in range(L)], axis=1)
    d_trace = torch.from_numpy(trace).to(dev)
    pos = w.ctx + np.arange(n)
    d_new = torch.from_numpy(np.stack([synth.records_at(R, L, [p] * R, rec_bytes=rec) for p in pos])).to(dev)
    d_pos = torch.from_numpy(np.repeat(pos[:, None], R, axis=1).astype(np.int32)).to(dev)
    d_ctx = torch.from_numpy((pos[:, None] + 1).repeat(R, axis=1).astype(np.int32)).to(dev)
    d_q = torch.from_numpy(np.stack([synth.queries(R, L, t, heads=w.heads) for t in range(n)])
                           .view(np.int16)).to(dev).permute(0, 2, 1, 3, 4).contiguous()
    d_slots = torch.empty((L, R, k), dtype=torch.int32, device=dev)
    d_stats = torch.zeros((n, L, R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    d_out = torch.empty((L, R, w.heads, 512), dtype=torch.float32, device=dev)
    cs = torch.cuda.current_stream().cuda_stream

    def step(c, t, fused):
        hk.hs_writeback(c.h, d_new[t].data_ptr(), d_pos[t].data_ptr(), cs, cs)
        for l in range(L):
            if fused:
                hk.hs_resolve_attn(c.h, l, d_trace[t, l].data_ptr(), d_ctx[t].data_ptr(), d_slots[l].data_ptr(),
                                   d_stats[t, l].data_ptr(), 0, 0, d_q[t, l].data_ptr(), w.heads, 512,
                                   d_out[l].data_ptr(), 576 ** -0.5, cs)
            else:
                hk.hs_resolve(c.h, l, d_trace[t, l].data_ptr(), d_ctx[t].data_ptr(), d_slots[l].data_ptr(),
                              d_stats[t, l].data_ptr(), 0, 0, cs)
                hk.hs_sparse_attn(c.h, l, d_q[t, l].data_ptr(), w.heads, 512, d_slots[l].data_ptr(),
                                  d_out[l].data_ptr(), 576 ** -0.5, 0, cs)

    def run(c, fused):
        for t in range(warmup):
            step(c, t, fused)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(warmup, n):
            step(c, t, fused)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        return el

    fused = hk.hs_resolve_attn_wgs(cache.h) > 0
    el = run(cache, True)
    st = d_stats.cpu().numpy()
    cache.close()
    cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B, newest_slot=True, fp8=True))
    for r in range(R):
        synth.fill_request(cache.host_pool_address(r), r, L, lmax, w.ctx, rec_bytes=rec)
    d_stats.zero_()
    el_sep = run(cache, False)
    assert np.array_equal(d_stats.cpu().numpy(), st) and not st[..., 2].any()
    cache.close()
    return {"fp8_long_selections_per_s": steps * L * R * k / el, "fp8_long_ms_per_step": el / steps * 1e3,
            "fp8_long_fused": fused,
            "fp8_long_separate_selections_per_s": steps * L * R * k / el_sep,
            "fp8_record_bytes": rec}


def measure_rows(torch, hk, synth, dev, rows=4, steps=24):
    """Speculative decoding with three draft tokens: each call resolves 4 verification rows of
    k = 2048 (their union, first reference order) into B = 5 k slots, long-request shape
    (1 request, 8 layers, write-through).  Median µs per call (union + RESOLVE + scatter)."""
    from synth.traces import verify_rows
    w = synth.WORKLOADS["long"].scaled(B=5 * 2048)
    R, L, k, B = w.R, w.L, w.k, w.B
    lmax = w.max_positions(steps)
    cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B, newest_slot=True, verify_rows=rows))
    for r in range(R):
        synth.fill_request(cache.host_pool_address(r), r, L, lmax, w.ctx)
    tr = np.stack([np.stack([verify_rows(w, r, l, steps, rows) for r in range(R)], axis=1) for l in range(L)], axis=1)
    d_tr = torch.from_numpy(tr).to(dev)  # [steps][L][R][rows][k]
    pos = w.ctx + np.arange(steps)
    d_new = torch.from_numpy(np.stack([synth.records_at(R, L, [p] * R) for p in pos])).to(dev)
    d_pos = torch.from_numpy(np.repeat(pos[:, None], R, axis=1).astype(np.int32)).to(dev)
    d_ctx = torch.from_numpy((pos[:, None] + 1).repeat(R, axis=1).astype(np.int32)).to(dev)
    d_out = torch.empty((R, rows, k), dtype=torch.int32, device=dev)
    d_stats = torch.zeros((steps, L, R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
           for _ in range(steps)]
    for t in range(steps):
        hk.hs_writeback(cache.h, d_new[t].data_ptr(), d_pos[t].data_ptr(), s.cuda_stream, s.cuda_stream)
        for l in range(L):
            evs[t][l][0].record(s)
            hk.hs_resolve_rows(cache.h, l, rows, d_tr[t, l].data_ptr(), d_ctx[t].data_ptr(), d_out.data_ptr(),
                               d_stats[t, l].data_ptr(), 0, 0, s.cuda_stream)
            evs[t][l][1].record(s)
    torch.cuda.synchronize()
    us = np.array([[evs[t][l][0].elapsed_time(evs[t][l][1]) * 1e3 for l in range(L)] for t in range(steps)])
    st = d_stats.cpu().numpy()
    assert not st[..., 2].any()
    union = (st[4:, ..., 0] + st[4:, ..., 1]).mean()
    cache.close()
    return {"spec4_resolve_rows_us_per_layer": float(np.median(us[4:])),
            "spec4_union_entries": float(union),
            "spec4_miss_rate_of_union": float(st[4:, ..., 1].sum() / max(1, (st[4:, ..., 0] + st[4:, ..., 1]).sum()))}


def measure_short(torch, hk, synth, dev, steps=64):
    """Short-sequence fast path: a request admitted short (2048 tokens in slot order, B = 4096,
    k = 2048) resolves each layer to its own positions with no hash, LRU or IO.  Median µs per
    layer call, 1 request x 8 layers (events)."""
    R, L, k, B, ctx = 1, 8, 2048, 4096, 3072
    w = synth.WORKLOADS["long"].scaled(append=False, force_newest=False, ctx=ctx)
    lmax = ctx
    cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B))
    for r in range(R):
        synth.fill_request(cache.host_pool_address(r), r, L, lmax, ctx)
        hk.hs_admit_short(cache.h, r, ctx, 0)
    tr = np.stack([np.stack([synth.selection_trace(w, r, l, steps) for r in range(R)], axis=1) for l in range(L)], axis=1)
    d_tr = torch.from_numpy(tr).to(dev)
    d_ctx = torch.full((R,), ctx, dtype=torch.int32, device=dev)
    d_out = torch.empty((R, k), dtype=torch.int32, device=dev)
    d_st = torch.zeros((steps, L, R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
           for _ in range(steps)]
    for t in range(steps):
        for l in range(L):
            evs[t][l][0].record(s)
            hk.hs_resolve(cache.h, l, d_tr[t, l].data_ptr(), d_ctx.data_ptr(), d_out.data_ptr(), d_st[t, l].data_ptr(),
                          0, 0, s.cuda_stream)
            evs[t][l][1].record(s)
    torch.cuda.synchronize()
    st = d_st.cpu().numpy()
    assert (st[..., 0] == k).all() and not st[..., 1:3].any()
    us = np.array([[evs[t][l][0].elapsed_time(evs[t][l][1]) * 1e3 for l in range(L)] for t in range(steps)])
    cache.close()
    return {"short_fast_path_us_per_layer": float(np.median(us[2:]))}


def measure_batched(torch, hk, synth, dev, layers=4, steps=16, warmup=4):
    """The batched decode step: 32 requests, ctx 32768, k 2048, B 4096, every layer through
    hs_resolve_attn (the fused kernel: per request one resolving workgroup and 7 fetch
    workgroups of 5 tiles each, then the finish kernel).  Four of the sixteen layers (the host
    pool of all sixteen is 19.3 GB; every layer is independent and costs the same).  Steady
    state after the cold step: selections/s, and the miss bytes per second over the host link,
    which bounds this step."""
    w = synth.WORKLOADS["batched"].scaled(L=layers, B=4096)
    R, L, k, B = w.R, w.L, w.k, w.B
    n = warmup + steps
    lmax = w.max_positions(n)
    cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B))
    for r in range(R):
        synth.fill_request(cache.host_pool_address(r), r, L, lmax, w.ctx)
    tr = np.stack([np.stack([synth.selection_trace(w, r, l, n) for r in range(R)], axis=1) for l in range(L)],
                  axis=1)
    d_tr = torch.from_numpy(tr).to(dev)
    d_q = torch.from_numpy(np.stack([synth.queries(R, L, t) for t in range(n)]).view(np.int16)).to(dev)
    d_q = d_q.permute(0, 2, 1, 3, 4).contiguous()  # [steps][L][R][16][576]
    d_ctx = torch.full((R,), w.ctx, dtype=torch.int32, device=dev)
    d_slots = torch.empty((L, R, k), dtype=torch.int32, device=dev)
    d_stats = torch.zeros((n, L, R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    d_out = torch.empty((L, R, 16, 512), dtype=torch.float32, device=dev)
    cs = torch.cuda.current_stream().cuda_stream

    def step(t):
        for l in range(L):
            hk.hs_resolve_attn(cache.h, l, d_tr[t, l].data_ptr(), d_ctx.data_ptr(), d_slots[l].data_ptr(),
                               d_stats[t, l].data_ptr(), 0, 0, d_q[t, l].data_ptr(), 16, 512, d_out[l].data_ptr(),
                               576 ** -0.5, cs)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(warmup, n):
        step(t)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    st = d_stats.cpu().numpy()
    assert st[..., 2].sum() == 0
    miss_bytes = float(st[warmup:, :, :, 1].sum()) * REC
    wgs = hk.hs_resolve_attn_wgs(cache.h)
    cache.close()
    return {"batched_fused_wgs_per_request": wgs,
            "batched_step_ms_4_layers": el / steps * 1e3,
            "batched_us_per_layer": el / (steps * L) * 1e6,
            "batched_selections_per_s": steps * L * R * k / el,
            "batched_miss_rate": float(st[warmup:, ..., 1].sum() / (steps * L * R * k)),
            "batched_steady_link_GBps": miss_bytes / el / 1e9}


def measure_shared_step(torch, hk, synth, dev, steps=12, warmup=4):
    """A decode step of the shared-index workload, one anchor group: 16 requests, the anchor
    and its three shared layers, ctx 131072, k 2048, B 4096, 16 heads.  Per step the anchor
    goes through hs_resolve_attn with its miss plan recorded; hs_prefetch_shared replays the
    plan into the three shared layers on the prefetch stream; each shared layer's attention
    (hs_sparse_attn over the anchor's slots) waits for its own layer's replay only.
    Selections/s count the k selected tokens of every request in all four layers.  The anchor's
    fused kernel and the replay kernels are stamped by their own start and end."""
    w = synth.WORKLOADS["shared"].scaled(L=4)
    R, L, k, B = w.R, w.L, w.k, w.B
    n = warmup + steps
    lmax = w.max_positions(n)
    cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B, layer_group=w.group))
    for r in range(R):
        synth.fill_request(cache.host_pool_address(r), r, L, lmax, w.ctx)
    tr = np.stack([synth.selection_trace(w, r, 0, n) for r in range(R)], axis=1)  # [n][R][k]
    d_tr = torch.from_numpy(tr).to(dev)
    d_q = torch.from_numpy(np.stack([synth.queries(R, L, t) for t in range(n)]).view(np.int16)).to(dev)
    d_q = d_q.permute(0, 2, 1, 3, 4).contiguous()  # [n][L][R][16][576]
    d_ctx = torch.full((R,), w.ctx, dtype=torch.int32, device=dev)
    d_slots = torch.empty((R, k), dtype=torch.int32, device=dev)
    d_stats = torch.zeros((n, R, hk.HS_STATS_WORDS), dtype=torch.int32, device=dev)
    d_out = torch.empty((L, R, 16, 512), dtype=torch.float32, device=dev)
    cs = torch.cuda.current_stream()
    ps = torch.cuda.Stream()
    scale = 576 ** -0.5

    def step(t):
        hk.hs_resolve_attn(cache.h, 0, d_tr[t].data_ptr(), d_ctx.data_ptr(), d_slots.data_ptr(),
                           d_stats[t].data_ptr(), 0, hk.HS_RECORD_PLAN, d_q[t, 0].data_ptr(), 16, 512,
                           d_out[0].data_ptr(), scale, cs.cuda_stream)
        hk.hs_prefetch_shared(cache.h, 0, cs.cuda_stream, ps.cuda_stream)
        for l in range(1, L):
            hk.hs_wait_layer(cache.h, l, cs.cuda_stream)
            hk.hs_sparse_attn(cache.h, l, d_q[t, l].data_ptr(), 16, 512, d_slots.data_ptr(), d_out[l].data_ptr(),
                              scale, 0, cs.cuda_stream)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(warmup, n):
        step(t)
    torch.cuda.synchronize()
    ps.synchronize()
    el = time.perf_counter() - t0
    # the same steps again from an empty start, with the kernels stamped (fused, then 3 replays)
    wgs = hk.hs_resolve_attn_wgs(cache.h)
    st = d_stats.cpu().numpy()
    cache.close()
    cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B, layer_group=w.group))
    for r in range(R):
        synth.fill_request(cache.host_pool_address(r), r, L, lmax, w.ctx)
    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    hk.hs_timing_start(cache.h, steps * 4)
    for t in range(warmup, n):
        step(t)
    torch.cuda.synchronize()
    ps.synchronize()
    us = hk.hs_timing_read(cache.h, steps * 4).astype(np.float64).reshape(steps, 4)
    cache.close()
    assert not st[..., 2].any()
    plan_bytes = 3 * st[warmup:, :, 1].sum(axis=1) * REC
    return {"shared_step_us": el / steps * 1e6,
            "shared_selections_per_s": steps * L * R * k / el,
            "shared_fused_wgs_per_request": wgs,
            "shared_anchor_fused_kernel_us": float(np.median(us[:, 0])),
            "shared_replay_kernels_us_per_step": float(np.median(us[:, 1:].sum(axis=1))),
            "shared_replay_GBps": float(plan_bytes.sum() / (us[:, 1:].sum() * 1e-6) / 1e9),
            "shared_miss_rate": float(st[warmup:, :, 1].sum() / (steps * R * k))}


def measure_attention(torch, hk, synth, dev, steps=12, warmup=2):
    """The attention consumer alone (hs_sparse_attn: attention kernel, then the chunk merge) at
    the batched shape: 32 requests, k 2048, B 4096, 16 heads, one layer.  Each step resolves
    (untimed), then the attention call runs between events on the launch stream.  Bytes per
    call: the k records of every request, the queries and the outputs."""
    w = synth.WORKLOADS["batched"].scaled(L=1, B=4096)
    R, L, k, B = w.R, w.L, w.k, w.B
    n = warmup + steps
    lmax = w.max_positions(n)
    cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B))
    for r in range(R):
        synth.fill_request(cache.host_pool_address(r), r, L, lmax, w.ctx)
    tr = np.stack([synth.selection_trace(w, r, 0, n) for r in range(R)], axis=1)  # [n][R][k]
    d_tr = torch.from_numpy(tr).to(dev)
    d_q = torch.from_numpy(np.stack([synth.queries(R, L, t)[:, 0] for t in range(n)]).view(np.int16)).to(dev)
    d_ctx = torch.full((R,), w.ctx, dtype=torch.int32, device=dev)
    d_slots = torch.empty((R, k), dtype=torch.int32, device=dev)
    d_out = torch.empty((R, 16, 512), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for t in range(n):
        hk.hs_resolve(cache.h, 0, d_tr[t].data_ptr(), d_ctx.data_ptr(), d_slots.data_ptr(), 0, 0, 0, s.cuda_stream)
        ev[t][0].record(s)
        hk.hs_sparse_attn(cache.h, 0, d_q[t].data_ptr(), 16, 512, d_slots.data_ptr(), d_out.data_ptr(),
                          576 ** -0.5, 0, s.cuda_stream)
        ev[t][1].record(s)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev[warmup:]])
    cache.close()
    nbytes = R * (k * REC + 16 * 576 * 2 + 16 * 512 * 4)
    t_us = float(np.median(us))
    return {"attention_r32_call_us": t_us, "attention_r32_bytes": nbytes,
            "attention_r32_GBps": nbytes / (t_us * 1e-6) / 1e9,
            "attention_r32_frac_of_hbm_peak": nbytes / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def measure_empty(torch, hk):
    s = torch.cuda.current_stream()
    hk.hs_probe_empty(100, s.cuda_stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    hk.hs_probe_empty(2000, s.cuda_stream)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / 2000


def measure_hbm(torch, hk, dev):
    """HBM rates: a 1 GiB copy (bytes read + written), a streaming read of it (256 workgroups
    of 16-byte loads, 8 per thread in flight), and 65536 scattered 1152-byte records gathered
    from it into a dense buffer (the access pattern of the attention's hot-slot reads; bytes
    read)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    copy = 2 * n / timed(lambda: hk.hs_probe_copy(a.data_ptr(), b.data_ptr(), n, s.cuda_stream)) / 1e9
    sink = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    read = n / timed(lambda: hk.hs_probe_host_read(a.data_ptr(), n, sink.data_ptr(), 256, s.cuda_stream)) / 1e9
    nrec = 65536
    idx = np.random.Generator(np.random.PCG64(7)).choice(n // REC, size=nrec, replace=False).astype(np.int32)
    d_idx = torch.from_numpy(idx).to(dev)
    gather = nrec * REC / timed(lambda: hk.hs_probe_host_records(a.data_ptr(), n // REC, REC, d_idx.data_ptr(), nrec,
                                                                 b.data_ptr(), 4096, s.cuda_stream)) / 1e9
    del a, b
    return {"hbm_copy_GBps": copy, "hbm_stream_read_GBps": read, "hbm_scattered_records_read_GBps": gather}


def cpu_baseline_configs(torch, hk, synth, dev, budget_s=3.0):
    """Each workload side by side: GPU RESOLVE (hs_resolve, every launch stamped by its own
    start and end) and the oracle on this host's cores, the same seeded trace from the same
    empty start, steady-state steps (the cold step and the next excluded).  The oracle reads
    the records from the library's pinned pool (filled by the same generator; nothing writes
    it here) and runs one thread per (request, layer) cache; it times the steady steps that
    fit its budget.  Long runs without the appended token here (RESOLVE only; the decode step
    with write-through and attention is the headline).  The shared-index workload's row is its
    anchor layer (the replay is measured on its own).  Selections/s count every selected
    token; miss GB/s are missed record bytes over the same time."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    W = synth.WORKLOADS
    cases = [("tiny", W["tiny"], 32),
             ("long (no append)", W["long"].scaled(append=False, force_newest=False), 24),
             ("batched B=2048", W["batched"].scaled(L=2, B=2048), 16),
             ("batched B=4096", W["batched"].scaled(L=2, B=4096), 16),
             ("batched B=8192", W["batched"].scaled(L=2, B=8192), 16),
             ("shared (anchor)", W["shared"].scaled(L=1, group=1), 16),
             ("capacity (blocks)", W["capacity"].scaled(L=1), 24)]
    link = None
    out = []
    threads_max = min(16, os.cpu_count() or 1)
    for name, w, steps in cases:
        R, L, k, B = w.R, w.L, w.k, w.B
        lmax = w.max_positions(steps)
        trace = np.stack([np.stack([synth.selection_trace(w, r, l, steps) for r in range(R)], axis=1)
                          for l in range(L)], axis=1)  # [steps][L][R][kb]
        cache = hk.HiSparse(hk.make_config(R, L, lmax, k, B, block_tokens=w.block_tokens))
        for r in range(R):
            synth.fill_request(cache.host_pool_address(r), r, L, lmax, w.ctx)
        # GPU; then the oracle reads the same pool (RESOLVE does not write it)
        us, st = run_resolve_only(torch, hk, synth, w, dev, trace, lmax, steps, 0, cache=cache)
        gpu_t = float(us[2:].sum()) * 1e-6
        gpu_sel = (steps - 2) * L * R * k / gpu_t
        gpu_miss = float(st[2:, :, :, 1].sum()) * REC / gpu_t / 1e9
        # oracle
        caches = {(r, l): oracle.Cache(B, lmax, REC) for r in range(R) for l in range(L)}
        base = {r: cache.host_pool_address(r) for r in range(R)}
        threads = min(R * L, threads_max)
        pool = ThreadPoolExecutor(max_workers=threads)

        def one(args):
            t, r, l = args
            sel = trace[t, l, r]
            if w.block_tokens > 1:
                sel = oracle.expand_blocks(sel, w.block_tokens)
            _, _, m, _, _ = caches[(r, l)].resolve(sel, w.ctx, base[r] + l * lmax * REC)
            return m

        def step(t):
            return sum(pool.map(one, [(t, r, l) for r in range(R) for l in range(L)]))

        step(0)
        step(1)
        done, misses = 0, 0
        t0 = time.perf_counter()
        while 2 + done < steps and time.perf_counter() - t0 < budget_s:
            misses += step(2 + done)
            done += 1
        el = time.perf_counter() - t0
        pool.shutdown()
        exp = int(st[2:2 + done, :, :, 1].sum())
        assert misses == exp, (name, misses, exp)  # the same trace, the same misses
        for c in caches.values():
            c.close()
        cache.close()
        row = {"workload": name, "requests": R, "layers": L, "top_k": k, "buffer_slots": B,
               "miss_rate": float(st[2:, :, :, 1].sum() / ((steps - 2) * L * R * k)),
               "gpu_selections_per_s": gpu_sel, "gpu_miss_GBps": gpu_miss,
               "gpu_resolve_us_per_launch": float(us[2:].mean()),
               "oracle_selections_per_s": done * L * R * k / el if done else None,
               "oracle_miss_GBps": misses * REC / el / 1e9 if done else None,
               "oracle_threads": threads, "oracle_steps": done}
        out.append(row)
    return out


def host_cpu():
    """Model name of this host's processor (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# secondary measurements that --measure can run on their own (name -> f(torch, hk, synth, dev))
SECONDARY = {
    "replay": measure_replay,
    "capacity": measure_capacity,
    "batched": measure_batched,
    "long_decode": measure_long_decode,
    "headline": measure_headline,
    "fetch_heavy": measure_fetch_heavy,
    "all_hit": measure_all_hit,
    "rows": measure_rows,
    "attention": measure_attention,
    "shared_step": measure_shared_step,
    "fp8": measure_fp8,
    "short": measure_short,
}

if __name__ == "__main__":
    main()
