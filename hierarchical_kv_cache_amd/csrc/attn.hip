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
//   - bf16 records (attn_tiles_kernel): 1024-thread workgroups on the tile
//     functions the fused kernel uses.  The chunk's record addresses are found
//     in one pass, each tile is gathered into registers (5 16-byte loads per
//     thread) while the previous tile is attended, 4 waves compute the scores
//     on v_mfma_f32_16x16x32_bf16 and all 16 accumulate P V, 32 channels each.
//   - FP8 records (attn_kernel): 4 waves; a tile's E4M3 codes are turned into
//     bf16 in LDS, the scores keep one MFMA accumulator per 128-dim scale block,
//     and P is scaled per block for P V.
// P is split into bf16 hi + lo parts so the fp32 probabilities survive the
// bf16 operand.
#include <algorithm>

#include "hs_internal.h"
#include "hs_attend.h"

namespace hs {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int AT = 256;                 // 4 waves
constexpr int TT = 64;                  // tokens per tile
constexpr int RS = kTileStride;         // LDS row stride (1168 bytes): conflict-free QK^T and P V
                                        // operand reads
constexpr int KSTEPS = kAttnDk / 32;    // 18
constexpr int CHUNKS = kAttnDk * 2 / 16;  // 72 16-byte chunks per record
constexpr int CT = kAttnDv / 4 / 16;    // 8 channel tiles of 16 per wave
constexpr int QS = kAttnDk * 2 + 16;       // LDS stride of a query row (padded off the bank period)
// FP8 records (the fp8 latent-KV layout, 656 bytes): 512 E4M3 codes in 4 blocks of 128 with
// a float32 scale each, then 64 bf16.  The gather turns them into the same bf16 rows.
constexpr int F8_DATA = 32;                // 16-byte chunks of codes (16 values each)
constexpr int F8_ITEMS = F8_DATA + 8;      // + 8 chunks of bf16 rope values
constexpr int F8_GATHER = TT * F8_ITEMS / AT;  // 10 items per thread per tile

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (finite inputs)
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// FP8 records.
__global__ void __launch_bounds__(AT, 1) attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char rows[TT * RS];
  __shared__ __attribute__((aligned(16))) unsigned char qs[16 * QS];  // q rows, zero past `heads`
  // P (hi and lo bf16 parts) as P V operands: [wave][32-token block][head][k]; each wave gets
  // P times its channel block's per-token scale.
  __shared__ __attribute__((aligned(16))) uint16_t phi[4][2][16][32];
  __shared__ __attribute__((aligned(16))) uint16_t plo[4][2][16][32];
  __shared__ float s_scale[TT][4];  // the block scales of each token of the tile
  __shared__ float smax[4][16];
  __shared__ float ssum[4][16];
  __shared__ int s_slot[kAttnMaxChunk];

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
  const int lane = tid & 63, w = tid >> 6, col = lane & 15, qd = lane >> 4;
  const int t_begin = s * p.chunk;
  const int t_end = min(p.k, t_begin + p.chunk);
  const int n_tok = t_end - t_begin;

  const uint8_t* hot_r = p.hot + (size_t)r * p.hot_req_stride + p.hot_layer_off;
  const int32_t* slots_r = p.slots + (size_t)r * p.k;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const u32x4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};

  // the chunk's slots and the queries, both in LDS, loaded together
  {
    constexpr int QL = (16 * CHUNKS + AT - 1) / AT;  // 5 query chunks per thread
    constexpr int SL = kAttnMaxChunk / AT;           // 4 slots per thread
    u32x4 qv[QL];
    int sv[SL];
#pragma unroll
    for (int u = 0; u < SL; ++u) {
      const int i = tid + u * AT;
      sv[u] = i < n_tok ? slots_r[t_begin + i] : -1;
    }
#pragma unroll
    for (int u = 0; u < QL; ++u) {
      const int f = tid + u * AT;
      const int h = f / CHUNKS, c = f - h * CHUNKS;
      qv[u] = (f < 16 * CHUNKS && h < p.heads)
                  ? *((const u32x4*)(p.q + ((size_t)r * p.heads + h) * kAttnDk) + c) : zero4;
    }
#pragma unroll
    for (int u = 0; u < SL; ++u)
      if (tid + u * AT < n_tok) s_slot[tid + u * AT] = sv[u];
#pragma unroll
    for (int u = 0; u < QL; ++u) {
      const int f = tid + u * AT;
      const int h = f / CHUNKS, c = f - h * CHUNKS;
      if (f < 16 * CHUNKS) *(u32x4*)(qs + h * QS + c * 16) = qv[u];
    }
  }
  __syncthreads();

  // records of the tile starting at token t0: 10 16-byte loads per thread (each data chunk
  // with its block's scale), all in flight
  constexpr int NG = F8_GATHER;
  u32x4 stage[NG];
  float sscale[NG];
  // the record of a published slot: 0..B hot rows, B+1+row resident rows, else none
  auto record_of = [&](int tok) -> const uint8_t* {
    const int sl = s_slot[tok - t_begin];
    const int64_t rr = (int64_t)sl - (p.B + 1);
    return (sl >= 0 && sl <= p.B) ? hot_r + (size_t)sl * p.rec_bytes
           : (rr >= 0 && rr < p.res_rows) ? p.res + (size_t)rr * p.rec_bytes : nullptr;
  };
  auto gather = [&](int t0) {
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int f = tid + u * AT;
      const int row = f / F8_ITEMS, c = f - row * F8_ITEMS;
      const int tok = t0 + row;
      // past the end: exact zeros; no record (a slot outside the published range): NaN, so
      // the output shows it
      if (tok >= t_end) {
        stage[u] = zero4;
        sscale[u] = 0.0f;
      } else {
        const uint8_t* src = record_of(tok);
        const int off = c < F8_DATA ? 16 * c : 528 + 16 * (c - F8_DATA);
        stage[u] = src ? *(const u32x4*)(src + off) : nan4;
        sscale[u] = (src && c < F8_DATA) ? *(const float*)(src + 512 + 4 * (c >> 3)) : __builtin_nanf("");
      }
    }
  };

  const float sl2 = p.scale * 1.4426950408889634f;  // scores kept in log2 units
  float m_run[4], l_lane[4];
  f32x4 o[CT];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_lane[i] = 0.0f; }
#pragma unroll
  for (int c = 0; c < CT; ++c) o[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  gather(t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += TT) {
    __syncthreads();  // the previous tile is no longer read
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int f = tid + u * AT;
      const int row = f / F8_ITEMS, c = f - row * F8_ITEMS;
      if (c < F8_DATA) {
        // 16 codes -> 16 bf16, exactly (an E4M3 value has 4 significant bits); the block
        // scale is applied to the fp32 sums below instead of rounding code * scale
        uint32_t wv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)stage[u][q], false);
          const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)stage[u][q], true);
          wv[2 * q] = (__float_as_uint(a.x) >> 16) | (__float_as_uint(a.y) & 0xFFFF0000u);
          wv[2 * q + 1] = (__float_as_uint(b.x) >> 16) | (__float_as_uint(b.y) & 0xFFFF0000u);
        }
        u32x4* d = (u32x4*)(rows + row * RS + c * 32);
        d[0] = u32x4{wv[0], wv[1], wv[2], wv[3]};
        d[1] = u32x4{wv[4], wv[5], wv[6], wv[7]};
        if ((c & 7) == 0) s_scale[row][c >> 3] = sscale[u];
      } else {
        *(u32x4*)(rows + row * RS + 1024 + (c - F8_DATA) * 16) = stage[u];
      }
    }
    __syncthreads();
    if (t0 + TT < t_end) gather(t0 + TT);  // the next tile's loads fly during this tile's math

    // scores of tokens 16w .. 16w+15: lane gets s[head = 4 qd + i][token = col]
    f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
    const unsigned char* krow = rows + (16 * w + col) * RS + qd * 16;
    const unsigned char* qrow = qs + col * QS + qd * 16;  // A operand: q[head = col][32 ks + 8 qd + j]
    {
      // one accumulator per 128-dim scale block (4 k-steps each) and one for the bf16 part
      f32x4 sb[5];
#pragma unroll
      for (int b = 0; b < 5; ++b) sb[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8 qa = *(const bf16x8*)(qrow + ks * 64);
        const bf16x8 kb = *(const bf16x8*)(krow + ks * 64);
        sb[ks < 16 ? ks >> 2 : 4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kb, sb[ks < 16 ? ks >> 2 : 4], 0, 0, 0);
      }
      const float* scl = s_scale[16 * w + col];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc[i] = sb[0][i] * scl[0] + sb[1][i] * scl[1] + sb[2][i] * scl[2] + sb[3][i] * scl[3] + sb[4][i];
    }
    const bool valid = (t0 + 16 * w + col) < t_end;
    float sv[4], mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = valid ? sacc[i] * sl2 : -INFINITY;
      mx[i] = row16_max(sv[i]);
    }
    if (col == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) smax[w][qd * 4 + i] = mx[i];
    __syncthreads();

    float alpha[4];
    const int tl = 16 * w + col;  // token within the tile
    const int bk = tl >> 5, t32 = tl & 31;
    const int kk = (t32 & 3) * 8 + (t32 >> 2);  // P V operands pair k index 8 qd + j with token 4 j + qd
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = qd * 4 + i;
      float mn = fmaxf(fmaxf(smax[0][hh], smax[1][hh]), fmaxf(smax[2][hh], smax[3][hh]));
      mn = fmaxf(mn, m_run[i]);
      alpha[i] = exp2f(m_run[i] - mn);
      m_run[i] = mn;
      const float pv = exp2f(sv[i] - mn);
      l_lane[i] = l_lane[i] * alpha[i] + pv;
      const float* scl = s_scale[tl];
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const float pw = pv * scl[w2];
        const uint16_t hi = f32_to_bf16_bits(pw);
        phi[w2][bk][hh][kk] = hi;
        plo[w2][bk][hh][kk] = f32_to_bf16_bits(pw - bf16_bits_to_f32(hi));
      }
    }
    __syncthreads();

    // o[head][channel] += p v over this tile; wave w owns channels 128 w .. 128 w + 127
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[c][i] *= alpha[i];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const bf16x8 ahi = *(const bf16x8*)&phi[w][b][col][qd * 8];
      const bf16x8 alo = *(const bf16x8*)&plo[w][b][col][qd * 8];
      const unsigned char* vb = rows + (b * 32 + qd) * RS + (w * 128 + col) * 2;
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        bf16x8 vv;
#pragma unroll
        for (int j = 0; j < 8; ++j) vv[j] = *(const __bf16*)(vb + 4 * j * RS + c * 32);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, vv, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, vv, o[c], 0, 0, 0);
      }
    }
  }

  // per-head sums: over the 16 token columns of a quarter-wave, then over waves
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    l_lane[i] = row16_sum(l_lane[i]);
  }
  __syncthreads();
  if (col == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) ssum[w][qd * 4 + i] = l_lane[i];
  __syncthreads();

  if (p.S == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = qd * 4 + i;
      if (hh >= p.heads) continue;
      const float inv = 1.0f / (ssum[0][hh] + ssum[1][hh] + ssum[2][hh] + ssum[3][hh]);
      float* orow = p.out + ((size_t)r * p.heads + hh) * p.value_dim + w * 128 + col;
#pragma unroll
      for (int c = 0; c < CT; ++c) orow[c * 16] = o[c][i] * inv;
    }
    return;
  }

  float* part = p.part + ((size_t)r * p.S + s) * kPartStride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = qd * 4 + i;
#pragma unroll
    for (int c = 0; c < CT; ++c) part[hh * kAttnDv + w * 128 + c * 16 + col] = o[c][i];
  }
  if (w == 0 && col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = qd * 4 + i;
      part[16 * kAttnDv + hh] = m_run[i];
      part[16 * kAttnDv + 16 + hh] = ssum[0][hh] + ssum[1][hh] + ssum[2][hh] + ssum[3][hh];
    }
  }
}

// bf16 records: workgroup (r, s) over chunk s of request r (<= kAttnMaxChunk entries, so at
// most 16 tiles).  A slot that names no record (outside [0, B] and the resident rows) makes
// the chunk's result NaN, so the request's output shows it.
__global__ void __launch_bounds__(kAT) attn_tiles_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char tile[kTileRows * kTileStride];
  __shared__ __attribute__((aligned(16))) unsigned char qs[16 * kQStride];
  __shared__ __attribute__((aligned(16))) unsigned char scratch[kAttnScratch];
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
  const uint8_t* filler = (const uint8_t*)(p.q + (size_t)r * p.heads * kAttnDk);  // finite rows
  u32x4 qv[kQU];
  q_load(qv, p.q, r, p.heads);
  int bad = 0;
  if (tid < nt * kTileRows) {
    const uint8_t* src = filler;
    if (tid < n) {
      const int sl = p.slots[(size_t)r * p.k + t_begin + tid];
      const int64_t rr = (int64_t)sl - (p.B + 1);
      if (sl >= 0 && sl <= p.B) src = hot_r + (size_t)sl * p.rec_bytes;
      else if (rr >= 0 && rr < p.res_rows) src = p.res + (size_t)rr * p.rec_bytes;
      else bad = 1;
    }
    asrc[tid] = (uint64_t)src;
  }
  q_store(qv, qs);
  bad = __syncthreads_or(bad);
  const float sl2 = p.scale * 1.4426950408889634f;  // scores kept in log2 units
  u32x4 tv[kTU];
  tile_load(tv, asrc);
  AttnAcc acc;
  acc_init(acc);
  for (int t = 0; t < nt; ++t) {
    if (t > 0) __syncthreads();  // the previous tile's readers are done with the tile and P
    tile_store(tv, tile);
    if (t + 1 < nt) tile_load(tv, asrc + (t + 1) * kTileRows);  // flies during this tile's math
    __syncthreads();
    attend_tile<false>(tile, qs, scratch, min(kTileRows, n - t * kTileRows), sl2, acc);
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
  // pre[r] = misses of the applying requests before r (p.R <= kFinishThreads)
  const int nr = p.num_reqs ? min(*p.num_reqs, p.R) : p.R;
  const int mine = (tid < nr && p.hdr[tid * 4] == 0) ? (int)p.hdr[tid * 4 + 1] : 0;
  pre[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kFinishThreads; off <<= 1) {
    const int add = tid >= off ? pre[tid - off] : 0;
    __syncthreads();
    pre[tid] += add;
    __syncthreads();
  }
  const int incl = pre[tid];
  __syncthreads();
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

hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  const int grid = p.R >= 8 ? 8 * ((p.R + 7) / 8) * p.S : p.R * p.S;
  if (p.fp8) hipLaunchKernelGGL(attn_kernel, dim3(grid), dim3(AT), 0, s, p);
  else hipLaunchKernelGGL(attn_tiles_kernel, dim3(grid), dim3(kAT), 0, s, p);
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
