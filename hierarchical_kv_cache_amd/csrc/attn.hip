// Sparse decode attention over the slots RESOLVE published ("HiSparse 深度解析"
// (gentlecold.top) §5.4 and §6.5: attention reads the physical rows -- hot slots,
// or resident rows when a resident tier is bound -- aligned with the
// top-k order).  Per request, H <= 16 query heads share one latent KV record
// per token: the key is all 576 bf16 of the record, the value its first 512.
//
// Work split (split-k over the top-k entries): workgroup (r, s) owns a chunk
// of request r's entries and walks it in tiles of 64 tokens, keeping a running
// max / sum per head.  A second small kernel merges the per-chunk partials
// (max, sum, unnormalised output) of each (request, head).  With R >= 8 all
// chunks of a request run on one XCD.
// attn_tiles_kernel<F8>: 1024-thread workgroups on the tile functions the
// fused kernel's fetch workgroups use, for bf16 or FP8 records.  The chunk's
// record addresses are found in one pass, each tile is gathered into registers
// (16-byte loads) while the previous tile is attended, and attend_tile keeps
// all 16 waves on v_mfma_f32_16x16x32_bf16 (scores split by key range, P V by
// 32 output channels per wave).
#include <algorithm>
#include <mutex>

#include "hs_internal.h"
#include "hs_attend.h"

namespace hs {
namespace {

// Workgroup (r, s) over chunk s of request r (<= kAttnMaxChunk entries, so at most 16 tiles).
// A slot that names no record (outside [0, B] and the resident rows) makes the chunk's result
// NaN, so the request's output shows it; rows past the chunk's end read a finite filler (for
// bf16 records the request's first query row, for FP8 records a zero record: a query row
// decoded as FP8 could hold NaN codes).  F8: FP8 records (tile_load8 / tile_store8).
template <bool F8>
__global__ void __launch_bounds__(kAT) attn_tiles_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char tile[kTileRows * kTileStride];
  __shared__ __attribute__((aligned(16))) unsigned char qs[16 * kQStride];
  __shared__ __attribute__((aligned(16))) unsigned char att_lds[F8 ? kAttnScratch8 : kAttnScratch];
  __shared__ uint64_t asrc[kAttnMaxChunk];  // record address of each chunk entry
  int r, s;
  if (p.R >= 8) {  // chunks of one request on one XCD (workgroups go round-robin over 8 XCDs)
    const int x = blockIdx.x & 7, loc = blockIdx.x >> 3;
    r = (loc / p.S) * 8 + x;
    s = loc % p.S;
    if (r >= p.R) return;
  } else {
    r = blockIdx.x / p.S;
    s = blockIdx.x % p.S;
  }
  if (p.num_reqs && r >= *p.num_reqs) return;
  const int tid = threadIdx.x;
  const int t_begin = s * p.chunk;
  const int n = min(p.k, t_begin + p.chunk) - t_begin;
  const int nt = (n + kTileRows - 1) / kTileRows;
  const uint8_t* hot_r = p.hot + (size_t)r * p.hot_req_stride + p.hot_layer_off;
  const uint8_t* filler = F8 ? p.zero : (const uint8_t*)(p.q + (size_t)r * p.heads * kAttnDk);
  u32x4 qv[kQU];
  q_load(qv, p.q, r, p.heads);
  int bad = 0;
  // the newest slot and the backed LRU slots (all of them, unless the hot buffer is on demand)
  const int capr = p.cap ? p.cap[r] : p.B;
  if (tid < nt * kTileRows) {
    const uint8_t* src = filler;
    if (tid < n) {
      const int sl = p.slots[(size_t)r * p.k + t_begin + tid];
      const int64_t rr = (int64_t)sl - (p.B + 1);
      if (sl >= 0 && (sl < capr || sl == p.B)) src = hot_r + (size_t)sl * p.rec_bytes;
      else if (rr >= 0 && rr < p.res_rows) src = p.res + (size_t)rr * p.rec_bytes;
      else bad = 1;
    }
    asrc[tid] = (uint64_t)src;
  }
  q_store(qv, qs);
  bad = __syncthreads_or(bad);
  const float sl2 = p.scale * 1.4426950408889634f;  // scores kept in log2 units
  u32x4 tv[F8 ? kTU8 : kTU];
  if constexpr (F8) tile_load8(tv, asrc);
  else tile_load(tv, asrc);
  AttnAcc acc;
  acc_init(acc);
  for (int t = 0; t < nt; ++t) {
    if (t > 0) __syncthreads();  // the previous tile's readers are done with the tile and P
    if constexpr (F8) tile_store8(tv, tile, tile_scales8(att_lds));
    else tile_store(tv, tile);
    if (t + 1 < nt) {  // flies during this tile's math
      if constexpr (F8) tile_load8(tv, asrc + (t + 1) * kTileRows);
      else tile_load(tv, asrc + (t + 1) * kTileRows);
    }
    __syncthreads();
    attend_tile<F8>(tile, qs, att_lds, min(kTileRows, n - t * kTileRows), sl2, acc);
  }
  if (bad) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc.m[i] = nan;
      acc.l[i] = nan;
      acc.o[0][i] = nan;
      acc.o[1][i] = nan;
    }
  }
  attend_write(acc, p.part + ((size_t)r * p.S + s) * kPartStride,
               p.S == 1 ? p.out + (size_t)r * p.heads * kAttnDv : nullptr, p.heads);
}

// Merge of the S chunk partials of one (request, head): o = sum_s 2^(m_s - M) o_s /
// sum_s 2^(m_s - M) l_s.  One wave per (request, head, 128 channels), two channels per
// lane.  Every lane issues its (m, l) pairs and the first kMergeBatch partial rows at once,
// so a merge of up to kMergeBatch chunks costs one memory round trip.
constexpr int kMergeBatch = 32;
constexpr int kMergeQuarters = kAttnDv / 128;

// One wave: channels 128 qt .. 128 qt + 127 of head hh, from the S partials of one request
// (pr); `fac` is this wave's LDS scratch of kAttnMaxChunks floats.  Every wave of the
// workgroup calls it (it holds a workgroup barrier).
__device__ __forceinline__ void merge_quarter(const float* pr, int S, int hh, int qt, int lane, float* fac,
                                              float* orow) {
  const float* base = pr + hh * kAttnDv + qt * 128 + 2 * lane;
  constexpr int NU = kAttnMaxChunks / 64;
  float mv[NU], lv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int q = lane + 64 * u;
    const float* pq = pr + (size_t)q * kPartStride + 16 * kAttnDv;
    mv[u] = q < S ? pq[hh] : -INFINITY;
    lv[u] = q < S ? pq[16 + hh] : 0.0f;
  }
  f32x2 v[kMergeBatch];
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u)
    v[u] = u < S ? *(const f32x2*)(base + (size_t)u * kPartStride) : f32x2{0.0f, 0.0f};
  float M = mv[0];
#pragma unroll
  for (int u = 1; u < NU; ++u) M = fmaxf(M, mv[u]);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) M = fmaxf(M, __shfl_xor(M, d));
  float den = 0.0f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const float f = exp2f(mv[u] - M);  // 0 for the chunks past S (m = -inf)
    fac[lane + 64 * u] = f;
    den += f * lv[u];
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) den += __shfl_xor(den, d);
  __syncthreads();
  f32x2 acc = {0.0f, 0.0f};
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) acc += fac[u] * v[u];
  for (int q0 = kMergeBatch; q0 < S; q0 += kMergeBatch) {  // more than kMergeBatch chunks
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      v[u] = q0 + u < S ? *(const f32x2*)(base + (size_t)(q0 + u) * kPartStride) : f32x2{0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) acc += fac[q0 + u < kAttnMaxChunks ? q0 + u : 0] * v[u];
  }
  *(f32x2*)(orow + qt * 128 + 2 * lane) = acc * (1.0f / den);
}

__global__ void __launch_bounds__(64) attn_merge_kernel(AttnParams p) {
  __shared__ float fac[kAttnMaxChunks];
  const int rh = blockIdx.x / kMergeQuarters, qt = blockIdx.x - rh * kMergeQuarters;
  const int r = rh / p.heads, hh = rh - r * p.heads;
  if (p.num_reqs && r >= *p.num_reqs) return;
  merge_quarter(p.part + (size_t)r * p.S * kPartStride, p.S, hh, qt, threadIdx.x, fac,
                p.out + ((size_t)r * p.heads + hh) * p.value_dim);
}

// The fused call's second kernel.  Workgroups [0, merge_blocks): one per (request, head),
// four waves for the four 128-channel quarters: the chunk merge, or NaN rows when workgroup
// 0 of the fused kernel reported an error for the request (with one chunk the fetch
// workgroup wrote the output itself).  The other workgroups take the misses of every request
// whose resolve succeeded: each builds the prefix of their miss counts in LDS (the fused
// kernel runs at most kFinishThreads requests), then the grid strides over all requests'
// misses at once for the page-table updates (the evicted position host only, the new
// position in its victim slot, tagged with the launch's generation), and over their 16-byte
// chunks to copy the missed records from the staging area into their victim slots.  No two
// misses share a slot or a position, and evicted positions are not selected, so the writes
// are independent.
constexpr int kFinishThreads = 256;
constexpr int kFinishUnroll = 4;
constexpr int kFinishMaxCopyBlocks = 1024;

// the request r with pre[r] <= j < pre[r + 1] (pre non-decreasing, pre[R] > j)
__device__ __forceinline__ int request_of(const int* pre, int R, int j) {
  int lo = 0, hi = R - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void __launch_bounds__(kFinishThreads) attn_finish_kernel(FinishParams p) {
  __shared__ float fac[kFinishThreads / 64][kAttnMaxChunks];
  __shared__ int pre[kFinishThreads + 1];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (b < p.merge_blocks) {
    const int r = b / p.heads, hh = b - r * p.heads;
    if (p.num_reqs && r >= *p.num_reqs) return;
    float* orow = p.out + ((size_t)r * p.heads + hh) * p.value_dim;
    if (p.hdr[r * 4] != 0) {
      for (int c = tid; c < p.value_dim; c += kFinishThreads) orow[c] = __builtin_nanf("");
      return;
    }
    if (p.S == 1) return;
    merge_quarter(p.part + (size_t)r * p.S * kPartStride, p.S, hh, tid >> 6, tid & 63, fac[tid >> 6], orow);
    return;
  }
  // pre[r] = misses of the applying requests before r (p.R <= kFinishThreads): an inclusive
  // scan within each wave (shuffles), then the waves' totals added in through LDS
  const int nr = p.num_reqs ? min(*p.num_reqs, p.R) : p.R;
  const int mine = (tid < nr && p.hdr[tid * 4] == 0) ? (int)p.hdr[tid * 4 + 1] : 0;
  const int lane = tid & 63, wv = tid >> 6;
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  __shared__ int wsum[kFinishThreads / 64];
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  for (int w = 0; w < wv; ++w) incl += wsum[w];
  pre[tid] = incl - mine;
  if (tid == kFinishThreads - 1) pre[kFinishThreads] = incl;
  __syncthreads();
  const int M = pre[kFinishThreads];
  const int C = p.rec_bytes >> 4;
  const int nthreads = (gridDim.x - p.merge_blocks) * kFinishThreads;
  const int t0 = (b - p.merge_blocks) * kFinishThreads + tid;
  for (int j = t0; j < M; j += nthreads) {
    const int r = request_of(pre, p.R, j);
    const int32_t* ml = p.mlist + ((size_t)r * p.k + (j - pre[r])) * 4;
    uint64_t* pt = p.page_table + (size_t)r * p.max_positions;
    const int32_t old = ml[2];
    if (old >= 0) pt[old] = kPtHostOnly;
    pt[ml[3]] = pt_entry(ml[1], p.hdr[r * 4 + 2]);
  }
  const int total = M * C;  // M <= 256 * 4096
  for (int f0 = t0; f0 < total; f0 += nthreads * kFinishUnroll) {
    u32x4 v[kFinishUnroll];
    int slot[kFinishUnroll], cc[kFinishUnroll], rr[kFinishUnroll];
#pragma unroll
    for (int u = 0; u < kFinishUnroll; ++u) {
      const int f = f0 + u * nthreads;
      if (f < total) {
        const int j = f / C;
        cc[u] = f - j * C;
        const int r = request_of(pre, p.R, j);
        rr[u] = r;
        const int32_t* ml = p.mlist + ((size_t)r * p.k + (j - pre[r])) * 4;
        slot[u] = ml[1];
        v[u] = *((const u32x4*)(p.stage + ((size_t)r * p.k + ml[0]) * p.rec_bytes) + cc[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kFinishUnroll; ++u)
      if (f0 + u * nthreads < total)
        *((u32x4*)(p.hot + (size_t)rr[u] * p.hot_req_stride + p.hot_layer_off + (size_t)slot[u] * p.rec_bytes) +
          cc[u]) = v[u];
  }
}

}  // namespace

// ---- allocation-free attention (hs_sparse_attn_static) ------------------------------------
// The chunk partials of hs_sparse_attn_static live in this file-scope device array instead of
// the handle's workspace: kStaticAttnPartials partial records (16.8 MB), one copy per GPU,
// held until the process ends.  Host code never passes the array's name to a kernel (on the
// host it is a stand-in, not a device address): attn_scratch_init takes each device's address
// of it once, with that device current, and the launches use that address.
static __device__ __align__(256) float scratch[(size_t)kStaticAttnPartials * kPartStride];

namespace {
constexpr int kScratchMaxDevices = 64;
float* g_scratch_ptr[kScratchMaxDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

hipError_t attn_scratch_init(int device) {
  if (device < 0 || device >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[device] = (float*)ptr;
  return hipSuccess;
}

float* attn_scratch(int device) {
  if (device < 0 || device >= kScratchMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  const int grid = p.R >= 8 ? 8 * ((p.R + 7) / 8) * p.S : p.R * p.S;
  if (p.fp8) hipLaunchKernelGGL(attn_tiles_kernel<true>, dim3(grid), dim3(kAT), 0, s, p);
  else hipLaunchKernelGGL(attn_tiles_kernel<false>, dim3(grid), dim3(kAT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S == 1) return e;
  return launch_attn_merge(p, s);
}

hipError_t launch_attn_merge(const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL(attn_merge_kernel, dim3(p.R * p.heads * kMergeQuarters), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_finish(const FinishParams& p, hipStream_t s) {
  if (p.R > kFinishThreads) return hipErrorInvalidValue;  // one prefix entry per request
  // enough copy workgroups for every selected entry's chunks in one stride (all misses)
  const int64_t chunks = (int64_t)p.R * p.k * (p.rec_bytes >> 4);
  const int64_t per_block = (int64_t)kFinishThreads * kFinishUnroll;
  const int copy = (int)std::min<int64_t>(kFinishMaxCopyBlocks, (chunks + per_block - 1) / per_block);
  hipLaunchKernelGGL(attn_finish_kernel, dim3(p.merge_blocks + copy), dim3(kFinishThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace hs
