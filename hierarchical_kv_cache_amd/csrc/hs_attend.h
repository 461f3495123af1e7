// Device functions of the record tile and the attention over it, shared by the fused
// RESOLVE + attention kernel (resolve.hip) and the attention kernel (attn.hip): a 64-row tile
// of 1152-byte bf16 records gathered into registers and written to LDS, the 16 query rows,
// and the attention of 16 heads over one tile folded into a running maximum, sum and output
// (online softmax), on 1024-thread workgroups.
#pragma once

#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kAT = kResolveThreads;  // threads of a tile workgroup (16 waves)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The record tile: 64 rows of 72 16-byte chunks.  Thread t holds chunks t, t + kAT, ...
// (row f / 72, chunk f % 72) in registers from their loads until the tile is written to LDS,
// so the loads fly meanwhile (in the fused kernel while workgroup 0 runs stages 1-3; in both
// kernels during the previous tile's attention).  Loads straight into LDS made the fused
// kernel's LDS waits wait for them as well.  Non-temporal: every record is read once per
// launch.
constexpr int kRowChunks = kAttnDk / 8;               // 16-byte chunks per 1152-byte record
constexpr int kTileChunks = kTileRows * kRowChunks;   // 4608
constexpr int kTU = (kTileChunks + kAT - 1) / kAT;      // chunks per thread
constexpr int kQChunks = 16 * kRowChunks;             // query rows of 16 heads
constexpr int kQU = (kQChunks + kAT - 1) / kAT;

// row addresses in LDS (asrc[row]) -> this thread's chunks of the tile
__device__ __forceinline__ void tile_load(u32x4 (&tv)[kTU], const uint64_t* asrc) {
#pragma unroll
  for (int u = 0; u < kTU; ++u) {
    const int f = threadIdx.x + u * kAT;
    if (f < kTileChunks) {
      const int row = f / kRowChunks, c = f - row * kRowChunks;
      tv[u] = load_host16((const uint8_t*)asrc[row] + 16 * c);
    }
  }
}
__device__ __forceinline__ void tile_store(const u32x4 (&tv)[kTU], unsigned char* tile) {
#pragma unroll
  for (int u = 0; u < kTU; ++u) {
    const int f = threadIdx.x + u * kAT;
    if (f < kTileChunks) {
      const int row = f / kRowChunks, c = f - row * kRowChunks;
      *(u32x4*)(tile + (size_t)row * kTileStride + 16 * c) = tv[u];
    }
  }
}
// the query rows of request r (rows past `heads`: zeros)
__device__ __forceinline__ void q_load(u32x4 (&qv)[kQU], const uint16_t* q, int r, int heads) {
#pragma unroll
  for (int u = 0; u < kQU; ++u) {
    const int f = threadIdx.x + u * kAT;
    const int h = f / kRowChunks, c = f - h * kRowChunks;
    qv[u] = (f < kQChunks && h < heads) ? load_host16((const uint8_t*)(q + ((size_t)r * heads + h) * kAttnDk) + 16 * c)
                                        : u32x4{0u, 0u, 0u, 0u};
  }
}
__device__ __forceinline__ void q_store(const u32x4 (&qv)[kQU], unsigned char* qs) {
#pragma unroll
  for (int u = 0; u < kQU; ++u) {
    const int f = threadIdx.x + u * kAT;
    const int h = f / kRowChunks, c = f - h * kRowChunks;
    if (f < kQChunks) *(u32x4*)(qs + (size_t)h * kQStride + 16 * c) = qv[u];
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// FP8 records (656 bytes: 32 16-byte chunks of E4M3 codes, one chunk of the 4 float32 block
// scales, 8 chunks of bf16 values) in the same 64-row tile: the codes become bf16 exactly (an
// E4M3 value has 4 significant bits) in the first 1024 bytes of the row, the bf16 values follow,
// and the scales go to a [64][4] array apart; the scores and P V apply them in fp32.
constexpr int kF8RowChunks = kF8RecordBytes / 16;         // 41
constexpr int kF8TileChunks = kTileRows * kF8RowChunks;   // 2624
constexpr int kTU8 = (kF8TileChunks + kAT - 1) / kAT;     // chunks per thread

__device__ __forceinline__ void tile_load8(u32x4 (&tv)[kTU8], const uint64_t* asrc) {
#pragma unroll
  for (int u = 0; u < kTU8; ++u) {
    const int f = threadIdx.x + u * kAT;
    if (f < kF8TileChunks) {
      const int row = f / kF8RowChunks, c = f - row * kF8RowChunks;
      tv[u] = load_host16((const uint8_t*)asrc[row] + 16 * c);
    }
  }
}
// chunk c of FP8 record `row` into the tile (codes as bf16, scales apart, bf16 values after)
__device__ __forceinline__ void store8_chunk(const u32x4& v, unsigned char* tile, float* scales, int row, int c) {
  if (c < 32) {
    uint32_t wv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[q], false);
      const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[q], true);
      wv[2 * q] = (__float_as_uint(a.x) >> 16) | (__float_as_uint(a.y) & 0xFFFF0000u);
      wv[2 * q + 1] = (__float_as_uint(b.x) >> 16) | (__float_as_uint(b.y) & 0xFFFF0000u);
    }
    u32x4* d = (u32x4*)(tile + (size_t)row * kTileStride + 32 * c);
    d[0] = u32x4{wv[0], wv[1], wv[2], wv[3]};
    d[1] = u32x4{wv[4], wv[5], wv[6], wv[7]};
  } else if (c == 32) {
    *(u32x4*)(scales + 4 * row) = v;
  } else {
    *(u32x4*)(tile + (size_t)row * kTileStride + 1024 + 16 * (c - 33)) = v;
  }
}
__device__ __forceinline__ void tile_store8(const u32x4 (&tv)[kTU8], unsigned char* tile, float* scales) {
#pragma unroll
  for (int u = 0; u < kTU8; ++u) {
    const int f = threadIdx.x + u * kAT;
    if (f < kF8TileChunks) {
      const int row = f / kF8RowChunks, c = f - row * kF8RowChunks;
      store8_chunk(tv[u], tile, scales, row, c);
    }
  }
}

// A wave's own rows of a tile, for callers whose lanes l0 .. l0 + 3 of wave w resolved the
// tile's rows 16 i + w (i = 0..3): each lane holds the record address of its row (rsrc),
// the wave reads those four into scalar registers, and lane l takes chunks q = l + 64 u of
// the four rows (row i = q / RC).  No workgroup barrier stands between a wave's address
// lookups and its loads.  RC: 16-byte chunks per record.
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
template <typename T>
__device__ __forceinline__ T pick4(const T (&x)[4], int i) {
  return i == 0 ? x[0] : i == 1 ? x[1] : i == 2 ? x[2] : x[3];
}
template <int RC, int U>
__device__ __forceinline__ void wave_rows_load(u32x4 (&tv)[U], uint64_t rsrc, int l0) {
  static_assert(4 * RC <= 64 * U, "a wave's four rows fit its lanes' chunks");
  const int lane = threadIdx.x & 63;
  uint64_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = readlane64(rsrc, l0 + i);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int q = lane + 64 * u;
    if (q < 4 * RC) {
      const int i = q / RC, c = q - i * RC;
      tv[u] = load_host16((const uint8_t*)pick4(b, i) + 16 * c);
    }
  }
}
// the wave's loaded chunks into the LDS tile (F8: FP8 records, as tile_store8)
template <int RC, int U, bool F8>
__device__ __forceinline__ void wave_rows_store(const u32x4 (&tv)[U], unsigned char* tile, float* scales) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int q = lane + 64 * u;
    if (q < 4 * RC) {
      const int i = q / RC, c = q - i * RC;
      const int row = 16 * i + w;
      if constexpr (F8) store8_chunk(tv[u], tile, scales, row, c);
      else *(u32x4*)(tile + (size_t)row * kTileStride + 16 * c) = tv[u];
    }
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even (finite inputs)
  return (uint16_t)(u >> 16);
}

// Running attention of one fetch workgroup over its tiles (online softmax).  Lane (wave w,
// quarter qd, column col) holds, for heads 4 qd + i, the running maximum m and sum l of the
// scores (log2 units) and the unnormalised output o of channels 32 w + 16 c + col.
struct AttnAcc {
  float m[4], l[4];
  f32x4 o[2];
};

__device__ __forceinline__ void acc_init(AttnAcc& a) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a.m[i] = -INFINITY;
    a.l[i] = 0.0f;
  }
  a.o[0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  a.o[1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// The [64][4] block scales of an FP8 tile in the attention scratch.
__device__ __forceinline__ float* tile_scales8(unsigned char* scratch) {
  return (float*)(scratch + kAttnScales8Off);
}

// V operand of v_mfma_f32_16x16x32_bf16 by two transposed LDS reads (ds_read_b64_tr_b16).
// Within each 16-lane group the instruction hands output lane L, element j, element L % 4 of
// the 8 bytes that lane 4 j + L / 4 addressed.  So lane s of group g addresses token row
// v_row(g, s / 4) (second read: v_row(g, 4 + s / 4)) at channel c0 + 4 (s % 4), and lane L ends
// up with channel c0 + L of rows v_row(g, 0..7): k index 8 g + j is token v_row(g, j) of the
// 32-token block.  v_row gives each group's read the rows 2 a + p (one parity p, a step of 2),
// whose 32-byte pieces start on distinct 8-bank blocks at the 1168-byte row stride, also for
// the two groups an access serves together.
__device__ __forceinline__ int v_row(int g, int j) {
  return 2 * (4 * (g & 1) + (j & 3)) + 16 * (j >> 2) + (g >> 1);
}
// its inverse: the k index of token t (0..31) of a block
__device__ __forceinline__ int v_k(int t) {
  const int a = t >> 1;
  return 8 * (((t & 1) << 1) | ((a >> 2) & 1)) + (((a >> 3) << 2) | (a & 3));
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 v_operand(const unsigned char* tile, int row0, int c0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const unsigned char* a = tile + (row0 + v_row(g, s >> 2)) * kTileStride + 2 * (c0 + 4 * (s & 3));
  typedef s16x4 __attribute__((address_space(3))) * lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(a));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(a + 16 * kTileStride));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Attention of the 16 query heads over one tile of n_tok records held in LDS (sparse decode
// attention, "HiSparse 深度解析" (gentlecold.top) §5.4: the records of the published slots;
// key = the record's 576 values, value = its first 512), folded into the running state, on
// v_mfma_f32_16x16x32_bf16 with all 16 waves busy in every step:
//   1. scores: wave w computes the 16 heads x 16 tokens block of tokens 16 (w % 4) .. + 15 over
//      key range w / 4 (its 4 k-steps of 32 channels, 128 (w / 4) .. + 127, and for w / 4 < 2
//      the rope k-step 16 + w / 4), all its operand reads issued at once, into LDS;
//   2. wave w then takes head w over the 64 tokens (lane = token): the four partial sums added
//      in key-range order, scaled and masked; the tile maximum (16-token blocks, then across
//      them) and the new running maximum, the larger of the two; the probabilities against it,
//      their sum (16-token block sums added in block order), and P split into bf16 hi + lo parts
//      (so the fp32 probabilities survive the bf16 operand) in the operand layout of step 3;
//   3. every wave rescales its running sum and output by 2^(old max - new max) and
//      accumulates P V for 32 output channels, the V operands read transposed (v_operand).
// F8: FP8 records (tile_store8).  Key range kp is scale block kp: its partial takes the token's
// block scale on the fp32 sum before the rope part is added; wave w's 32 output channels lie
// in scale block w / 4, so it takes P times that block's per-token scale (the sums keep the
// unscaled P).
template <bool F8>
__device__ __forceinline__ void attend_tile(const unsigned char* tile, const unsigned char* qs,
                                            unsigned char* scratch, int n_tok, float sl2, AttnAcc& acc) {
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, qd = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int NB = F8 ? 4 : 1;      // P variants (one per scale block)
  float* smax = (float*)scratch;      // [16 heads]: the new running maximum
  float* ssum = smax + 16;            // [16 heads]: the tile's probability sum
  float* spart = ssum + 16;           // step 1 -> 2: [4 key ranges][4 token blocks (kSpartTB)][16 heads][kSpartRow]
  uint16_t* phi = (uint16_t*)(scratch + kAttnPOff);  // step 2 -> 3: [NB][2 token blocks][16 heads][kPRow]
  uint16_t* plo = phi + NB * 2 * 16 * kPRow;
  const float* scl8 = F8 ? tile_scales8(scratch) : nullptr;  // [64][4]
  {
    // lane: partial s[head = 4 qd + i][token = 16 tb + col]
    const int tb = w & 3, kp = w >> 2;  // token block and key range
    const int tl = 16 * tb + col;
    const unsigned char* krow = tile + tl * kTileStride + qd * 16;
    const unsigned char* qrow = qs + col * kQStride + qd * 16;
    bf16x8 qa[4], ka[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qa[j] = *(const bf16x8*)(qrow + (4 * kp + j) * 64);
      ka[j] = *(const bf16x8*)(krow + (4 * kp + j) * 64);
    }
    f32x4 sr = {0.0f, 0.0f, 0.0f, 0.0f};
    if (kp < 2) {
      const bf16x8 qr = *(const bf16x8*)(qrow + (16 + kp) * 64);
      const bf16x8 kr = *(const bf16x8*)(krow + (16 + kp) * 64);
      sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qr, kr, sr, 0, 0, 0);
    }
    f32x4 sa = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[j], ka[j], sa, 0, 0, 0);
    const float sc = F8 ? scl8[4 * tl + kp] : 1.0f;
    float* sp = spart + (kp * 4 + tb) * kSpartTB + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) sp[(4 * qd + i) * kSpartRow] = F8 ? sa[i] * sc + sr[i] : sa[i] + sr[i];
  }
  __syncthreads();
  {
    const int h = w, t = lane;  // head h, token t
    constexpr int KR = 4 * kSpartTB;  // one key range's partials
    const float* sp = spart + (t >> 4) * kSpartTB + h * kSpartRow + (t & 15);
    const float s = sp[0] + sp[KR] + sp[2 * KR] + sp[3 * KR];
    const float sv = t < n_tok ? s * sl2 : -INFINITY;
    const float bm = row16_max(sv);  // each 16-token block's maximum, in every lane of the block
    const float mt = fmaxf(fmaxf(readlane_f(bm, 0), readlane_f(bm, 16)), fmaxf(readlane_f(bm, 32), readlane_f(bm, 48)));
    // the running maximum of head h: element h % 4 of the lanes of quarter h / 4
    const float mnew = fmaxf(readlane_f(pick4(acc.m, h & 3), 16 * (h >> 2)), mt);  // finite: every tile has a valid row
    const float pv = exp2f(sv - mnew);
    const float bs = row16_sum(pv);
    // (read outside the store's branch: inside it only lane 0 would finish its block's sum)
    const float lt = ((readlane_f(bs, 0) + readlane_f(bs, 16)) + readlane_f(bs, 32)) + readlane_f(bs, 48);
    if (t == 0) {
      smax[h] = mnew;
      ssum[h] = lt;
    }
    const int bk = t >> 5, kk = v_k(t & 31);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // a masked row (p = 0) takes no scale: a filler's scale must not turn 0 into NaN
      const float pw = F8 ? (pv != 0.0f ? pv * scl8[4 * t + b] : 0.0f) : pv;
      const uint16_t hi = f32_to_bf16_rne(pw);
      phi[((b * 2 + bk) * 16 + h) * kPRow + kk] = hi;
      plo[((b * 2 + bk) * 16 + h) * kPRow + kk] = f32_to_bf16_rne(pw - __uint_as_float((uint32_t)hi << 16));
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = qd * 4 + i;
    const float mnew = smax[hh];
    const float alpha = exp2f(acc.m[i] - mnew);  // 0 on the first tile
    acc.l[i] = acc.l[i] * alpha + ssum[hh];
    acc.m[i] = mnew;
#pragma unroll
    for (int c = 0; c < 2; ++c) acc.o[c][i] *= alpha;
  }
  // o[head][channel] += p v over the tile; wave w owns channels 32 w .. 32 w + 31
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int pb = F8 ? (w >> 2) * 2 + b : b;  // wave w's channels lie in scale block w / 4
    const bf16x8 ahi = *(const bf16x8*)&phi[(pb * 16 + col) * kPRow + qd * 8];
    const bf16x8 alo = *(const bf16x8*)&plo[(pb * 16 + col) * kPRow + qd * 8];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 vv = v_operand(tile, 32 * b, 32 * w + 16 * c, lane);
      acc.o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, vv, acc.o[c], 0, 0, 0);
      acc.o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, vv, acc.o[c], 0, 0, 0);
    }
  }
}

// The share's result: its partial (unnormalised o, maximum and sum in log2 units) for the
// merge, or the normalised output rows of the heads asked for when the request has one share.
__device__ __forceinline__ void attend_write(const AttnAcc& acc, float* part, float* out, int heads) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, qd = lane >> 4;
  // o[c][i]: head 4 qd + i, channel 32 w + 16 c + col
  if (out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = qd * 4 + i;
      if (hh >= heads) continue;
      const float inv = 1.0f / acc.l[i];
#pragma unroll
      for (int c = 0; c < 2; ++c) out[hh * kAttnDv + 32 * w + 16 * c + col] = acc.o[c][i] * inv;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c) part[(qd * 4 + i) * kAttnDv + 32 * w + 16 * c + col] = acc.o[c][i];
  if (w == 0 && col == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      part[16 * kAttnDv + qd * 4 + i] = acc.m[i];
      part[16 * kAttnDv + 16 + qd * 4 + i] = acc.l[i];
    }
  }
}

}  // namespace
}  // namespace hs
