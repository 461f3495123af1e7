// Internal declarations shared by the host API and the kernels of libhisparse.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/hisparse.h"

namespace hs {

constexpr int kResolveThreads = 1024;  // 16 wave64s: one workgroup resolves one request
constexpr int kMaxSlots = 16384;
constexpr int kMaxTopK = 16384;
constexpr int kMaxRecordBytes = 16384;
constexpr uint32_t kHasNewest = 1u << 8;  // internal resolve flag: slot B holds the newest token
// list entries per thread of the RESOLVE body for speculative unions of <= kUnionShortKE *
// kResolveThreads entries
constexpr int kUnionShortKE = 4;

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Launch counter of an anchor (ctrl[0..1] per request, 64 bits).  The G workgroups of a
// resolve launch that changes the metadata add 2^kLaunchShift to it in total: workgroup 0
// adds 2^kLaunchShift - (G - 1), every other workgroup adds 1, each once it has read the
// metadata.  A workgroup reads the counter before adding its own share, so it sees a strict
// subset of its launch's additions (less than 2^kLaunchShift) and count >> kLaunchShift
// numbers the earlier launches whatever G each launch used.
constexpr int kLaunchShift = 16;
__host__ __device__ inline uint64_t launch_number(uint64_t count) { return count >> kLaunchShift; }

// Page-table entry (64 bits): the slot holding the position in the low half (-1: host only),
// in the high half the generation of the launch that wrote it (launch number + 1; 0 for
// admission and appends).  Workgroup 0 of a launch writes the entries of that launch's
// misses while its sibling workgroups may still be reading the table; a reader that finds
// an entry of its own launch's generation knows the entry was not there before the launch,
// and treats the position as host only, exactly as a sibling that read earlier.
constexpr uint64_t kPtHostOnly = ~0ull;
__host__ __device__ inline uint64_t pt_entry(int32_t slot, uint32_t gen) {
  return ((uint64_t)gen << 32) | (uint32_t)slot;
}
// The slot an entry names for a reader of launch generation `gen` (-1: host only).
__host__ __device__ inline int32_t pt_slot_for(uint64_t e, uint32_t gen) {
  const int32_t slot = (int32_t)(uint32_t)e;
  return (slot >= 0 && (uint32_t)(e >> 32) != gen) ? slot : -1;
}

// Max and sum over the 16 lanes of each DPP row of a wave (lanes 16q .. 16q+15), every lane
// getting the result: lane ^ 1, lane ^ 2 (quad permutations), then the half-row and row
// mirrors (lane i with 7 - i, then with 15 - i) combine quads and half-rows.  DPP moves
// operands between lanes inside the ALU, without the LDS round trip of a shuffle.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  return v + dpp_mov<0x140>(v);
}

// 16-byte non-temporal access to the pinned host pool through global (not flat)
// addresses.  The pool's device addresses come from a table in memory, so the compiler
// cannot prove their address space and would emit flat instructions, which also count
// against the LDS wait counter: every barrier's wait for LDS would then wait for the PCIe
// round trip as well.
typedef uint32_t hs_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ hs_u32x4 load_host16(const uint8_t* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) hs_u32x4*)p);
}
__device__ __forceinline__ void store_host16(hs_u32x4 v, uint8_t* p) {
  __builtin_nontemporal_store(v, (__attribute__((address_space(1))) hs_u32x4*)p);
}

// LDS carve-up of the resolve kernel (shared by host sizing and device code).  The hash
// table is dead once stage 1 has checked for duplicates, so stage 3's per-miss arrays
// (victim, missidx, mrank) reuse its bytes (H >= 2k entries of 4 bytes >= 3 arrays of 2k).
// The per-wave early-fetch lists hold one fetch workgroup's share of the selection.
struct ResolveLds {
  size_t htab, selp, victim, missidx, mrank, sown, wpos, widx, wcap, scratch, total;
};
__host__ __device__ inline ResolveLds resolve_lds(int k, int B, int hash_bits, int G) {
  ResolveLds L;
  const size_t H = size_t(1) << hash_bits;
  const int NWv = kResolveThreads / 64;
  const int nf = G > 1 ? G - 1 : 1;
  const size_t share = (size_t(k) + nf - 1) / nf;  // the largest fetch share
  L.wcap = 64 * ((share + kResolveThreads - 1) / kResolveThreads);  // misses one wave can own
  L.htab = 0;
  L.victim = 0;
  L.missidx = align_up(L.victim + 2 * size_t(k), 16);
  L.mrank = align_up(L.missidx + 2 * size_t(k), 16);
  size_t o = align_up(L.mrank + 2 * size_t(k), 16);
  if (o < 4 * H) o = 4 * H;
  L.selp = o;    o = align_up(o + 4 * size_t(k), 16);
  L.sown = o;    o = align_up(o + 2 * size_t(B), 16);
  L.wpos = o;    o = align_up(o + 4 * NWv * L.wcap, 16);
  L.widx = o;    o = align_up(o + 2 * NWv * L.wcap, 16);
  L.scratch = o; o = align_up(o + 4 * size_t(5 * NWv + 8), 16);
  L.total = o;
  return L;
}
int resolve_elems_per_thread(int k, int B);

// Fused RESOLVE + attention.  Workgroup 0 uses the resolve carve-up; each fetch workgroup
// (a share of <= 64 T selected records, attended one 64-row tile at a time) the record tile,
// the query rows and the attention scratch (scores' maxima and sums, partial scores, P); each
// share entry's record address and miss index stay in the register of the lane that resolved
// it.  The dynamic LDS of the launch is the larger of the two.
constexpr int kTileRows = 64;        // records per tile
constexpr int kFusedMaxTiles = 16;   // tiles per fetch workgroup (share entries <= 1024 threads)
constexpr int kTileStride = 1168;    // LDS row stride of a 1152-byte record (292 words, 8-byte
                                     // aligned for the transposed V reads): consecutive rows start
                                     // 36 banks apart modulo 64, so the 16 rows of a QK^T operand
                                     // read, and the 4 rows of a 16-lane group of a V read, spread
constexpr int kQStride = 1168;       // LDS stride of a query row (16-byte aligned, off the bank period)
// the heads' new maxima and tile sums, the partial scores (4 key ranges x 4 token blocks x 16
// heads, rows of 16 tokens padded to kSpartRow fp32, token blocks kSpartTB apart), then P hi
// and lo (per P variant: 2 token halves x 16 heads, rows of 32 tokens padded to kPRow bf16);
// the padding puts the four lane quarters of an access on distinct banks (writers' quarters
// are 4 heads apart, readers' quarters one token block).  P has space of its own: the step
// that writes it also reads the partial scores of other waves.
constexpr int kSpartRow = 20, kPRow = 40;
constexpr int kSpartTB = 16 * kSpartRow + 16;
constexpr int kAttnSpart = 4 * 4 * kSpartTB * 4;
constexpr int kAttnPOff = 2 * 16 * 4 + kAttnSpart;        // P hi, then P lo
constexpr int kAttnPVariant = 2 * 2 * 16 * kPRow * 2;      // hi + lo bytes of one P variant
constexpr int kAttnScratch = kAttnPOff + kAttnPVariant;
// FP8 records: P per 128-channel scale block (4 variants), then the tile's block scales
constexpr int kAttnScales8Off = kAttnPOff + 4 * kAttnPVariant;
constexpr int kAttnScratch8 = kAttnScales8Off + kTileRows * 4 * 4;
constexpr int kF8RecordBytes = 656;  // 512 E4M3 codes, 4 float32 block scales, 64 bf16
struct FusedLds {
  size_t tile, qs, scratch, total;
};
__host__ __device__ inline FusedLds fused_lds(int k, int B, int hash_bits, int G, int T, bool f8 = false) {
  FusedLds F;
  F.tile = 0;
  F.qs = F.tile + size_t(kTileRows) * kTileStride;
  F.scratch = F.qs + 16 * size_t(kQStride);
  (void)T;  // the tiles of a share no longer add LDS
  const size_t fetch = align_up(F.scratch + (f8 ? kAttnScratch8 : kAttnScratch), 16);
  const size_t resolve = resolve_lds(k, B, hash_bits, G).total;
  F.total = fetch > resolve ? fetch : resolve;
  return F;
}

// Per-anchor metadata in the caller's workspace.  ctrl per request (uint32 x 4):
// [0..1] 64-bit launch counter (launch_number() of it numbers the launches that changed
// the metadata; its parity names the ping-pong half holding the current slot map and LRU
// order), [2] miss-plan count, [3] 1 when the request was admitted short (tokens in slot
// order while the context fits B).
struct ResolveParams {
  const int32_t* sel;        // [R][kb]
  const int32_t* ctx_len;    // [R]
  int32_t* out;              // [R][k]
  hs_stats* stats;           // [R] or null
  const int32_t* num_reqs;   // scalar or null
  uint32_t* ctrl;            // [R][4]
  int32_t* slot_pos;         // [R][2][B]
  int16_t* lru;              // [R][2][Bpad]
  int32_t* plan;             // [R][2][k]
  uint64_t* page_table;      // [R][max_positions] pt_entry values
  const int32_t* newest;     // [R]
  const uint8_t* const* host_base;  // [R] device-usable addresses of each request's host region
  uint8_t* hot;              // hot buffer base [R][L][B+1][rec]
  int64_t host_layer_off;    // layer offset inside a request's host region (bytes)
  int64_t hot_req_stride;    // bytes per request in the hot buffer
  int64_t hot_layer_off;     // layer offset inside a request's hot buffer (bytes)
  int64_t max_positions;
  const int32_t* kvar;       // [R] entries of each request's list (null: k for every request)
  const uint32_t* kerr;      // [R] error bits found before the launch (null: none)
  int32_t plan_k;            // plan row length (entries per request in plan)
  const int32_t* rtable;     // [R][rt_stride] resident page of each logical page (-1 none), or null
  int64_t rt_stride;         // logical pages per request
  int64_t res_rows;          // rows of the resident pool (0 without a resident tier)
  int32_t page_shift;        // log2 tokens per resident page
  int32_t R, B, Bpad, k, kb, bt_shift, rec_bytes, G, hash_bits;
  uint32_t flags;            // HS_RECORD_PLAN | HS_SKIP_IO | kHasNewest
  // fused attention (resolve_kernel<.., true>): G - 1 fetch workgroups per request, each
  // attends over its share of the selection (<= 64 att_tiles entries, a tile at a time)
  const uint16_t* q;         // [R][heads][576] bf16
  float* part;               // [R][G-1][kPartStride] chunk partials (G > 2)
  float* att_out;            // [R][heads][512] (written directly when G == 2)
  const uint8_t* att_res;    // this layer's resident pool [res_rows][rec] (null without one)
  uint32_t* att_hdr;         // [R][4] workgroup 0's report: error bits, misses, page-table generation
  int32_t* att_mlist;        // [R][k][4] per miss: list index, victim slot, evicted position, position
  uint8_t* att_stage;        // [R][k][rec] missed records by list index
  int32_t heads, att_tiles;
  float att_scale;
  const uint8_t* att_zero;   // a zero record: the finite filler row of FP8 tiles
  const int32_t* cap;        // [R] LRU slots backed by device memory (on-demand hot buffer), or
                             // null: every slot is backed
  // a speculative union (hs_resolve_rows): the rows' slots [R][rows_n] from the union's, entry
  // f of a request taking the slot of union entry rows_map[r][f] (-1: none); null otherwise
  int32_t* rows_out;
  const int32_t* rows_map;   // [R][k]
  int32_t rows_n;
};

// The finish kernel of the fused call: chunk merge (or NaN rows on error), the missed records
// from the staging area into their victim slots, the page-table updates of the misses.
struct FinishParams {
  float* out;                // [R][heads][value_dim]
  const float* part;         // [R][S][kPartStride]
  const int32_t* num_reqs;
  const uint32_t* hdr;       // [R][4]
  const int32_t* mlist;      // [R][k][4]
  const uint8_t* stage;      // [R][k][rec]
  uint8_t* hot;
  int64_t hot_req_stride, hot_layer_off;
  uint64_t* page_table;      // the anchor's [R][max_positions]
  int64_t max_positions;
  int32_t R, heads, value_dim, S, k, rec_bytes, merge_blocks;
};

struct AppendParams {
  const uint8_t* new_kv;     // [R][L][rec]
  const int32_t* new_pos;    // [R]
  int32_t* newest;           // [R]
  uint8_t* hot;
  const uint8_t* const* host_base;
  int64_t max_positions;
  int32_t R, L, B, rec_bytes;
  // short requests: their new tokens also go to the slot of their position
  const uint32_t* ctrl;      // anchor 0's [R][4]; anchor a at + a * R * 4
  int32_t* slot_pos;         // anchor 0's [R][2][B]; anchor a at + a * R * 2 * B
  uint64_t* page_table;      // anchor 0's [R][max_positions]
  int32_t A, group;          // anchors, layers per anchor
  const int32_t* cap;        // [R] backed LRU slots (on-demand hot buffer) or null (all)
};

// Admission of a short request: positions [0, ctx) of every layer staged into slots [0, ctx).
struct AdmitParams {
  const uint8_t* const* host_base;
  uint8_t* hot;
  uint32_t* ctrl;            // anchor 0's [R][4]
  int32_t* slot_pos;         // anchor 0's [R][2][B]
  uint64_t* page_table;      // anchor 0's [R][max_positions]
  int64_t max_positions, hot_req_stride;
  int32_t R, L, B, A, rec_bytes, request, ctx;
};

struct ReplayParams {
  const int32_t* plan;       // anchor's [R][2][plan_k]
  const uint32_t* ctrl;      // anchor's [R][4]
  const uint8_t* const* host_base;
  uint8_t* hot;
  int64_t host_layer_off, hot_req_stride, hot_layer_off;
  int32_t R, plan_k, rec_bytes;
};

// Union of the verification rows of one speculative step (first reference order).
struct UnionParams {
  const int32_t* sel;        // [R][rows][kb]
  const int32_t* ctx_len;    // [R]
  const int32_t* num_reqs;   // scalar or null
  int32_t* uni;              // [R][kmax] union, first-reference order
  int32_t* map;              // [R][kmax] union index of each entry (row-major)
  int32_t* cnt;              // [R] union size (0 on error)
  uint32_t* err;             // [R] error bits
  int64_t max_positions;
  int32_t R, rows, k, kb, bt_shift, kmax, hash_bits;
};

struct ScatterParams {
  const int32_t* uout;       // [R][kmax] slot of each union entry
  const int32_t* map;        // [R][kmax]
  const uint32_t* err;       // [R]
  const int32_t* num_reqs;
  int32_t* out;              // [R][rows][k]
  int32_t R, n, kmax;        // n = rows * k entries per request
};

struct AttnParams {
  const uint16_t* q;         // [R][heads][576] bf16
  const int32_t* slots;      // [R][k]
  float* out;                // [R][heads][value_dim]
  float* part;               // [R][S][kPartStride] partial results of the S chunks
  const int32_t* num_reqs;
  const uint8_t* hot;        // layer 0 base
  int64_t hot_req_stride, hot_layer_off;
  const uint8_t* res;        // this layer's resident pool [res_rows][rec] (null without one)
  int64_t res_rows;
  int32_t R, k, B, heads, value_dim, S, chunk, rec_bytes;
  float scale;
  int32_t fp8;               // records in the FP8 layout (HS_CFG_RECORD_FP8)
  const uint8_t* zero;       // a zero record (the FP8 tiles' filler)
  const int32_t* cap;        // [R] backed LRU slots (on-demand hot buffer) or null (all)
};

struct ExportParams {
  const uint32_t* ctrl;
  const int32_t* slot_pos;
  const int16_t* lru;
  const int32_t* newest;
  const uint64_t* page_table;  // [R][max_positions]
  int32_t* out_slot_pos;
  int32_t* out_lru;
  int32_t* out_page_table;
  int32_t* out_newest;
  int64_t max_positions;
  int32_t R, B, Bpad;
};

struct InitParams {
  uint32_t* ctrl;
  int32_t* slot_pos;
  int16_t* lru;
  uint64_t* page_table;
  int32_t* newest;
  int64_t max_positions;
  int32_t R, B, Bpad, A, request;  // request < 0: all
};

// Optional kernel timing of one launch: events stamped by the kernel's own start and end
// (hipExtLaunchKernel), for the measurement aid hs_timing_start / hs_timing_read.
struct KernelTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
hipError_t launch_resolve(const ResolveParams& p, size_t lds_bytes, hipStream_t s, const KernelTiming* tm = nullptr);
// the fused variant; false when no instantiation covers (k, B) (top_k <= 4096, B <= 8192)
bool fused_supported(int k, int B);
hipError_t launch_resolve_attn(const ResolveParams& p, size_t lds_bytes, hipStream_t s,
                               const KernelTiming* tm = nullptr);
hipError_t launch_union(const UnionParams& p, hipStream_t s);
hipError_t launch_scatter(const ScatterParams& p, hipStream_t s);
hipError_t set_union_lds_limit(size_t lds_bytes);
constexpr int kUnionMaxEntries = 8192;  // rows * top_k of one speculative resolve
// the union kernel's LDS: per bucket the position and the row mask / union index, then the
// rank counts (one per wave and entry slot: kUnionMaxEntries / 64) and shared words
inline size_t union_lds_bytes(int hash_bits) {
  return (size_t(8) << hash_bits) + 4 * (kUnionMaxEntries / 64 + 8);
}
// The one-launch speculative rows kernel (resolve_rows_kernel): the union's table first; once
// the union is built its list stays in the table's first 4 kmax bytes (the position array's,
// 4 H >= 8 kmax bytes) and RESOLVE's carve-up takes the bytes from rows_ulist_bytes(kmax) on.
__host__ __device__ inline size_t rows_ulist_bytes(int kmax) { return align_up(size_t(4) * kmax, 16); }
inline size_t rows_lds(int kmax, int B, int resolve_hash_bits, int G, int union_hash_bits) {
  const size_t u = union_lds_bytes(union_hash_bits);
  const size_t r = rows_ulist_bytes(kmax) + resolve_lds(kmax, B, resolve_hash_bits, G).total;
  return u > r ? u : r;
}
// one launch for a union whose capacity needs more than kUnionShortKE entries per thread
hipError_t launch_resolve_rows(const ResolveParams& p, const UnionParams& u, size_t lds_bytes, hipStream_t s,
                               const KernelTiming* tm = nullptr);
hipError_t set_resolve_lds_limit(size_t lds_bytes);
hipError_t launch_append(const AppendParams& p, hipStream_t s, bool write_through);
hipError_t launch_backup(const AppendParams& p, hipStream_t s);
hipError_t launch_replay(const ReplayParams& p, int wgs, hipStream_t s, const KernelTiming* tm = nullptr);
hipError_t launch_attn(const AttnParams& p, hipStream_t s);
hipError_t launch_attn_merge(const AttnParams& p, hipStream_t s);  // the S chunk partials -> out
hipError_t launch_attn_finish(const FinishParams& p, hipStream_t s);
hipError_t launch_export(const ExportParams& p, hipStream_t s);
hipError_t launch_init(const InitParams& p, hipStream_t s);
hipError_t launch_admit(const AdmitParams& p, hipStream_t s);
hipError_t launch_probe_host_read(const void* src, size_t bytes, void* sink, int wgs, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_probe_host_records(const void* src, const int32_t* index, int n, int rec_bytes,
                                     int64_t src_records, void* dst, int wgs, hipStream_t s);
hipError_t launch_probe_empty(int n, hipStream_t s);
// cap[r] = slots, ordered on s (the on-demand hot buffer's capacity of request r)
hipError_t launch_set_capacity(int32_t* cap, int r, int slots, hipStream_t s);
constexpr size_t kHotChunk = size_t(1) << 16;  // mapping unit of the on-demand hot buffer

// attention partial record: [16][512] output accumulators, then [16] max, [16] sum
constexpr int kAttnMaxHeads = 16;
constexpr int kAttnDk = 576;
constexpr int kAttnDv = 512;
constexpr int kPartStride = kAttnMaxHeads * kAttnDv + 2 * kAttnMaxHeads;
constexpr int kAttnMaxChunks = 256;  // top_k <= 16384 in chunks of >= 64 entries
constexpr int kAttnMaxChunk = 1024;  // entries per chunk (their slots are staged in LDS)
// allocation-free attention: partial records in a file-scope device array of attn.hip
constexpr int kStaticAttnPartials = 512;
hipError_t attn_scratch_init(int device);  // with `device` current; once per device
float* attn_scratch(int device);           // that device's address of the array (null before init)

}  // namespace hs
