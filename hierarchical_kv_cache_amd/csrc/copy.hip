// Byte-moving kernels around RESOLVE: write-through of the newest token,
// copy-only replay of an anchor's miss plan, metadata init/export, and the
// link/latency probes used for measurement.
#include <hip/hip_ext.h>

#include "hs_internal.h"

namespace hs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCopyThreads = 256;

// Division of a flattened chunk index by the chunks per record (C <= 1024,
// indices < 2^24): float estimate, then one correction step.
__device__ __forceinline__ void split_index(int f, int C, float invC, int& j, int& c) {
  j = (int)((float)f * invC);
  c = f - j * C;
  if (c < 0) { --j; c += C; }
  if (c >= C) { ++j; c -= C; }
}

// New token -> slot B of every (request, layer); the newest position is set
// ("HiSparse 深度解析" (gentlecold.top) §3.4: written into the GPU's reserved
// slot first).  Flattened over (request, layer, 16-byte chunk).
// WT: the write-through in the same pass (each 16-byte chunk also stored into the host pool at
// the new position, then the system-scope fence of backup_kernel), for callers that order it on
// their own stream instead of a backup stream.
template <bool WT>
__global__ void __launch_bounds__(kCopyThreads) append_kernel(AppendParams p) {
  const int C = p.rec_bytes >> 4;
  const int per_req = p.L * C;
  const int total = p.R * per_req;
  const float invC = 1.0f / (float)per_req;
  for (int f = blockIdx.x * blockDim.x + threadIdx.x; f < total; f += gridDim.x * blockDim.x) {
    int r, rest;
    split_index(f, per_req, invC, r, rest);
    const int32_t pos = p.new_pos[r];
    if (pos < 0 || pos >= p.max_positions) continue;  // rejected: this request is left as it was
    const int l = rest / C, c = rest - l * C;
    const u32x4* src = (const u32x4*)(p.new_kv + ((size_t)r * p.L + l) * p.rec_bytes) + c;
    u32x4* dst = (u32x4*)(p.hot + (((size_t)r * p.L + l) * (p.B + 1) + p.B) * p.rec_bytes) + c;
    const u32x4 v = *src;
    *dst = v;
    if constexpr (WT) {
      uint8_t* row = const_cast<uint8_t*>(p.host_base[r]) + ((size_t)l * p.max_positions + pos) * p.rec_bytes;
      store_host16(v, row + 16 * (size_t)c);
    }
    // a short request keeps its tokens in slot order while they fit ("HiSparse 深度解析" §5.4)
    // (on an on-demand hot buffer, only into a backed slot: the caller grows the request first)
    const bool in_order = p.ctrl[r * 4 + 3] != 0 && pos < p.B && (!p.cap || pos < p.cap[r]);
    if (in_order) *((u32x4*)(p.hot + (((size_t)r * p.L + l) * (p.B + 1) + pos) * p.rec_bytes) + c) = v;
    if (rest == 0) {
      p.newest[r] = pos;
      if (in_order) {
        for (int a = 0; a < p.A; ++a) {  // every anchor's slot map and page table
          const uint32_t* ca = p.ctrl + (size_t)a * p.R * 4;
          const int cur = (int)(launch_number(*(const uint64_t*)&ca[r * 4]) & 1u);
          p.slot_pos[((size_t)a * p.R + r) * 2 * p.B + (size_t)cur * p.B + pos] = pos;
          p.page_table[((size_t)a * p.R + r) * (size_t)p.max_positions + pos] = pt_entry(pos, 0u);
        }
      }
    }
  }
  if constexpr (WT) __threadfence_system();
}

// Slot B -> host pool at the newest position (write-through on the backup
// stream, gentlecold.top §3.4 and §5.4).  Non-temporal stores into the
// coherent pinned pool, then a system-scope fence.
__global__ void __launch_bounds__(kCopyThreads) backup_kernel(AppendParams p) {
  const int C = p.rec_bytes >> 4;
  const int per_req = p.L * C;
  const int total = p.R * per_req;
  const float invC = 1.0f / (float)per_req;
  for (int f = blockIdx.x * blockDim.x + threadIdx.x; f < total; f += gridDim.x * blockDim.x) {
    int r, rest;
    split_index(f, per_req, invC, r, rest);
    const int32_t pos = p.new_pos[r];
    if (pos < 0 || pos >= p.max_positions) continue;
    const int l = rest / C, c = rest - l * C;
    const u32x4* src =
        (const u32x4*)(p.hot + (((size_t)r * p.L + l) * (p.B + 1) + p.B) * p.rec_bytes) + c;
    // the pool table is shared with the readers (const); the write-through owns this row
    uint8_t* row = const_cast<uint8_t*>(p.host_base[r]) + ((size_t)l * p.max_positions + pos) * p.rec_bytes;
    store_host16(*src, row + 16 * (size_t)c);
  }
  __threadfence_system();
}

// Copy-only replay of an anchor's miss plan into one shared layer
// (gentlecold.top §3.6 and §5.6): the same (position, slot) pairs, this
// layer's own records.  A small fixed number of workgroups does it, so the
// copy leaves most of the GPU to the compute stream.  Up to kReplayFlatR
// requests, every workgroup builds the prefix of the per-request miss counts
// in LDS and the grid strides over the flattened (request, miss, 16-byte
// chunk) space, so the launch stays balanced however the misses fall over
// the requests.  Beyond that, ceil(grid / R) workgroups take each request's
// own chunk space (a workgroup takes every grid-th request when R > grid).
constexpr int kReplayFlatR = 1024;
constexpr int kReplayU = 8;  // loads in flight per thread
static_assert(4 * kCopyThreads >= kReplayFlatR, "each thread sums four requests' counts");

__device__ __forceinline__ void replay_flat(const ReplayParams& p, int* pre, int* scan) {
  const int t = threadIdx.x;
  const int C = p.rec_bytes >> 4;
  // pre[r] = misses of requests before r, pre[R] = all (R <= 4 * kCopyThreads)
  int mv[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * t + i;
    mv[i] = r < p.R ? (int)p.ctrl[r * 4 + 2] : 0;
    sum += mv[i];
  }
  scan[t] = sum;
  __syncthreads();
  for (int off = 1; off < kCopyThreads; off <<= 1) {
    const int add = t >= off ? scan[t - off] : 0;
    __syncthreads();
    scan[t] += add;
    __syncthreads();
  }
  int run = scan[t] - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * t + i;
    if (r < p.R) pre[r] = run;
    run += mv[i];
  }
  if (t == kCopyThreads - 1) pre[p.R] = scan[t];
  __syncthreads();
  const int64_t total = (int64_t)pre[p.R] * C;
  const int64_t stride = (int64_t)gridDim.x * kCopyThreads;
  for (int64_t f0 = (int64_t)blockIdx.x * kCopyThreads + t; f0 < total; f0 += stride * kReplayU) {
    u32x4 v[kReplayU];
    int rr[kReplayU], jj[kReplayU], cc[kReplayU];
#pragma unroll
    for (int u = 0; u < kReplayU; ++u) {
      const int64_t f = f0 + u * stride;
      if (f < total) {
        const int j = (int)(f / C);
        cc[u] = (int)(f - (int64_t)j * C);
        int lo = 0, hi = p.R - 1;  // the request r with pre[r] <= j < pre[r + 1]
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pre[mid] <= j) lo = mid; else hi = mid - 1;
        }
        rr[u] = lo;
        jj[u] = j - pre[lo];
        const int32_t* ppos = p.plan + (size_t)lo * 2 * p.plan_k;
        v[u] = load_host16(p.host_base[lo] + p.host_layer_off + (size_t)ppos[jj[u]] * p.rec_bytes +
                           16 * (size_t)cc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kReplayU; ++u)
      if (f0 + u * stride < total) {
        const int32_t* pslot = p.plan + (size_t)rr[u] * 2 * p.plan_k + p.plan_k;
        uint8_t* dbase = p.hot + (size_t)rr[u] * p.hot_req_stride + p.hot_layer_off;
        *((u32x4*)(dbase + (size_t)pslot[jj[u]] * p.rec_bytes) + cc[u]) = v[u];
      }
  }
}

__global__ void __launch_bounds__(kCopyThreads) replay_kernel(ReplayParams p) {
  __shared__ int pre[kReplayFlatR + 1];
  __shared__ int scan[kCopyThreads];
  if (p.R <= kReplayFlatR) {
    replay_flat(p, pre, scan);
    return;
  }
  const int C = p.rec_bytes >> 4;
  const float invC = 1.0f / (float)C;
  const int P = ((int)gridDim.x + p.R - 1) / p.R;  // workgroups per request
  const int stride = P * (int)blockDim.x;
  for (int pair = blockIdx.x; pair < p.R * P; pair += gridDim.x) {
    const int r = pair / P;
    const int t0 = (pair - r * P) * (int)blockDim.x + (int)threadIdx.x;
    const int m = (int)p.ctrl[r * 4 + 2];
    const int total = m * C;
    const int32_t* ppos = p.plan + (size_t)r * 2 * p.plan_k;
    const int32_t* pslot = ppos + p.plan_k;
    const uint8_t* hbase = p.host_base[r] + p.host_layer_off;
    uint8_t* dbase = p.hot + (size_t)r * p.hot_req_stride + p.hot_layer_off;
    for (int f0 = t0; f0 < total; f0 += stride * kReplayU) {
      u32x4 v[kReplayU];
      int jj[kReplayU], cc[kReplayU];
#pragma unroll
      for (int u = 0; u < kReplayU; ++u) {
        const int f = f0 + u * stride;
        if (f < total) {
          split_index(f, C, invC, jj[u], cc[u]);
          v[u] = load_host16(hbase + (size_t)ppos[jj[u]] * p.rec_bytes + 16 * (size_t)cc[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kReplayU; ++u)
        if (f0 + u * stride < total)
          *((u32x4*)(dbase + (size_t)pslot[jj[u]] * p.rec_bytes) + cc[u]) = v[u];
    }
  }
}

// Admission state ("HiSparse 深度解析" (gentlecold.top) §5.3, §5.4 release):
// every slot empty, every position host-only, LRU in slot order, no newest.
// grid.y = anchor, grid.z = request (or the one request being reset).
__global__ void __launch_bounds__(kCopyThreads) init_kernel(InitParams p) {
  const int a = blockIdx.y;
  const int r = p.request >= 0 ? p.request : (int)blockIdx.z;
  const size_t ar = (size_t)a * p.R + r;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int nt = gridDim.x * blockDim.x;
  for (int s = t; s < p.B; s += nt) {
    p.slot_pos[(ar * 2 + 0) * p.B + s] = -1;
    p.slot_pos[(ar * 2 + 1) * p.B + s] = -1;
    p.lru[(ar * 2 + 0) * p.Bpad + s] = (int16_t)s;
    p.lru[(ar * 2 + 1) * p.Bpad + s] = (int16_t)s;
  }
  uint64_t* pt = p.page_table + ar * (size_t)p.max_positions;
  for (int64_t q = t; q < p.max_positions; q += nt) pt[q] = kPtHostOnly;
  if (t == 0) {
    p.ctrl[ar * 4 + 0] = 0;
    p.ctrl[ar * 4 + 1] = 0;
    p.ctrl[ar * 4 + 2] = 0;
    p.ctrl[ar * 4 + 3] = 0;
    if (a == 0) p.newest[r] = -1;
  }
}

// Admission of a short request ("HiSparse 深度解析" (gentlecold.top) §5.3, §5.4): its first
// ctx tokens of every layer are staged from host into slots 0 .. ctx-1 in order, every
// anchor's slot map and page table record them, and the request is marked short.
// Flattened over (layer, position, 16-byte chunk); the metadata by the first ctx threads.
__global__ void __launch_bounds__(kCopyThreads) admit_kernel(AdmitParams p) {
  const int r = p.request;
  const int C = p.rec_bytes >> 4;
  const int64_t total = (int64_t)p.L * p.ctx * C;
  const int64_t nt = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t f = t0; f < total; f += nt) {
    const int64_t lp = f / C;
    const int c = (int)(f - lp * C);
    const int l = (int)(lp / p.ctx), pos = (int)(lp - (int64_t)l * p.ctx);
    const uint8_t* src = p.host_base[r] + ((size_t)l * p.max_positions + pos) * p.rec_bytes + 16 * (size_t)c;
    uint8_t* dst = p.hot + (size_t)r * p.hot_req_stride + ((size_t)l * (p.B + 1) + pos) * p.rec_bytes + 16 * (size_t)c;
    *(u32x4*)dst = load_host16(src);
  }
  for (int64_t s = t0; s < p.ctx; s += nt) {
    for (int a = 0; a < p.A; ++a) {
      const uint32_t* ca = p.ctrl + (size_t)a * p.R * 4;
      const int cur = (int)(launch_number(*(const uint64_t*)&ca[r * 4]) & 1u);
      p.slot_pos[((size_t)a * p.R + r) * 2 * p.B + (size_t)cur * p.B + s] = (int32_t)s;
      p.page_table[((size_t)a * p.R + r) * (size_t)p.max_positions + s] = pt_entry((int32_t)s, 0u);
    }
  }
  if (t0 == 0)
    for (int a = 0; a < p.A; ++a) p.ctrl[((size_t)a * p.R + r) * 4 + 3] = 1u;
}

__global__ void __launch_bounds__(kCopyThreads) export_kernel(ExportParams p) {
  const int r = blockIdx.y;
  const int cur = (int)(launch_number(*(const uint64_t*)&p.ctrl[r * 4]) & 1u);
  for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < p.B; s += gridDim.x * blockDim.x) {
    if (p.out_slot_pos) p.out_slot_pos[(size_t)r * p.B + s] = p.slot_pos[((size_t)r * 2 + cur) * p.B + s];
    if (p.out_lru) p.out_lru[(size_t)r * p.B + s] = p.lru[((size_t)r * 2 + cur) * p.Bpad + s];
  }
  // the page table's slots (the low half of each entry; the generation tag is bookkeeping)
  if (p.out_page_table) {
    const uint64_t* pt = p.page_table + (size_t)r * p.max_positions;
    int32_t* o = p.out_page_table + (size_t)r * p.max_positions;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < p.max_positions;
         q += (int64_t)gridDim.x * blockDim.x)
      o[q] = (int32_t)(uint32_t)pt[q];
  }
  if (p.out_newest && blockIdx.x == 0 && threadIdx.x == 0) p.out_newest[r] = p.newest ? p.newest[r] : -1;
}

template <int U>
__global__ void __launch_bounds__(kCopyThreads) probe_host_read_kernel(const u32x4* __restrict__ src,
                                                                       size_t n16, u32x4* sink) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t base = tid; base < n16; base += stride * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t idx = base + (size_t)u * stride;
      v[u] = idx < n16 ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  // keep the loads: a store that is (almost) never taken
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[tid & 1023] = acc;
}

__global__ void __launch_bounds__(kCopyThreads) probe_copy_kernel(const u32x4* __restrict__ src,
                                                                  u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Gathers n records at random indices of a pinned host array into a dense
// device array, flattened over (record, 16-byte chunk): the link rate a fetch of
// scattered 1152-byte records can reach.  Indices outside [0, src_records) are
// skipped.
__global__ void __launch_bounds__(kCopyThreads) probe_host_records_kernel(const unsigned char* __restrict__ src,
                                                                          const int32_t* __restrict__ index,
                                                                          int n, int C, int64_t src_records,
                                                                          unsigned char* __restrict__ dst) {
  const int total = n * C;
  const float invC = 1.0f / (float)C;
  for (int f = blockIdx.x * blockDim.x + threadIdx.x; f < total; f += gridDim.x * blockDim.x) {
    int j, c;
    split_index(f, C, invC, j, c);
    const int32_t i = index[j];
    if (i < 0 || (int64_t)i >= src_records) continue;
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(src + (size_t)i * C * 16) + c);
    *((u32x4*)(dst + (size_t)j * C * 16) + c) = v;
  }
}

__global__ void probe_empty_kernel() {}

__global__ void set_capacity_kernel(int32_t* cap, int r, int slots) { cap[r] = slots; }

int grid_for(size_t work, int per_block, int cap) {
  size_t b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > (size_t)cap) b = cap;
  return (int)b;
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t s, bool write_through) {
  const size_t work = (size_t)p.R * p.L * (p.rec_bytes >> 4);
  if (write_through)
    hipLaunchKernelGGL(append_kernel<true>, dim3(grid_for(work, kCopyThreads, 1024)), dim3(kCopyThreads), 0, s, p);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3(grid_for(work, kCopyThreads, 1024)), dim3(kCopyThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_backup(const AppendParams& p, hipStream_t s) {
  const size_t work = (size_t)p.R * p.L * (p.rec_bytes >> 4);
  hipLaunchKernelGGL(backup_kernel, dim3(grid_for(work, kCopyThreads, 256)), dim3(kCopyThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_replay(const ReplayParams& p, int wgs, hipStream_t s, const KernelTiming* tm) {
  if (tm && tm->start) {
    hipExtLaunchKernelGGL(replay_kernel, dim3(wgs), dim3(kCopyThreads), 0, s, tm->start, tm->stop, 0u, p);
  } else {
    hipLaunchKernelGGL(replay_kernel, dim3(wgs), dim3(kCopyThreads), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_init(const InitParams& p, hipStream_t s) {
  const int bx = grid_for((size_t)(p.max_positions > p.B ? p.max_positions : p.B), kCopyThreads * 8, 256);
  dim3 grid(bx, p.A, p.request >= 0 ? 1 : p.R);
  hipLaunchKernelGGL(init_kernel, grid, dim3(kCopyThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_admit(const AdmitParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.L * p.ctx * (p.rec_bytes >> 4);
  const int bx = grid_for((size_t)(n > p.ctx ? n : p.ctx), kCopyThreads * 4, 1024);
  hipLaunchKernelGGL(admit_kernel, dim3(bx), dim3(kCopyThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_export(const ExportParams& p, hipStream_t s) {
  dim3 grid(grid_for((size_t)p.B, kCopyThreads, 64), p.R);
  hipLaunchKernelGGL(export_kernel, grid, dim3(kCopyThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_probe_host_read(const void* src, size_t bytes, void* sink, int wgs, hipStream_t s) {
  hipLaunchKernelGGL(probe_host_read_kernel<8>, dim3(wgs), dim3(kCopyThreads), 0, s,
                     (const u32x4*)src, bytes / 16, (u32x4*)sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(grid_for(bytes / 16, kCopyThreads, 4096)), dim3(kCopyThreads),
                     0, s, (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return hipGetLastError();
}

hipError_t launch_probe_host_records(const void* src, const int32_t* index, int n, int rec_bytes,
                                     int64_t src_records, void* dst, int wgs, hipStream_t s) {
  hipLaunchKernelGGL(probe_host_records_kernel, dim3(wgs), dim3(kCopyThreads), 0, s, (const unsigned char*)src,
                     index, n, rec_bytes >> 4, src_records, (unsigned char*)dst);
  return hipGetLastError();
}

hipError_t launch_set_capacity(int32_t* cap, int r, int slots, hipStream_t s) {
  hipLaunchKernelGGL(set_capacity_kernel, dim3(1), dim3(1), 0, s, cap, r, slots);
  return hipGetLastError();
}

hipError_t launch_probe_empty(int n, hipStream_t s) {
  for (int i = 0; i < n; ++i) hipLaunchKernelGGL(probe_empty_kernel, dim3(1), dim3(64), 0, s);
  return hipGetLastError();
}

}  // namespace hs
