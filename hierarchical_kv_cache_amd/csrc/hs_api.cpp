// Host side of the C ABI: argument validation, workspace layout, the pinned
// host pool, stream/event ordering, kernel launches.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "hs_internal.h"

using namespace hs;

namespace {

thread_local std::string g_last_error;

hs_status fail(hs_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

hs_status hip_fail(hipError_t e, const char* what) {
  return fail(HS_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HS_HIP(call)                              \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hip_fail(e_, #call); \
  } while (0)

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int64_t x) { int b = 0; while ((int64_t(1) << b) < x) ++b; return b; }

// Offsets (bytes) of every array in the caller's workspace.
struct Layout {
  int A = 0;        // anchor layers
  int Bpad = 0;
  int S = 1;        // attention chunks per request
  int Spart = 1;    // partial records per (layer, request): max(S, fused chunks)
  int kmax = 0;     // longest list one resolve handles: top_k * max(1, verify_rows)
  size_t ctrl = 0, slot_pos = 0, lru = 0, plan = 0, page_table = 0, newest = 0, host_base = 0,
         attn_part = 0, uni = 0, umap = 0, uout = 0, ucnt = 0, uerr = 0, att_zero = 0, att_hdr = 0, att_mlist = 0,
         att_stage = 0, cap = 0, total = 0;
};

int attn_chunks(const hs_config& c) {
  // about one workgroup per CU (256 CUs) over all requests, chunks of >= 64 entries
  int S = (256 + c.num_requests - 1) / c.num_requests;
  const int max_s = (c.top_k + 63) / 64;
  if (S > max_s) S = max_s;
  const int min_s = (c.top_k + kAttnMaxChunk - 1) / kAttnMaxChunk;  // chunks of <= 1024 entries
  if (S < min_s) S = min_s;
  if (S < 1) S = 1;
  return S;
}

// Fused RESOLVE + attention (hs_resolve_attn): per request workgroup 0 and S fetch
// workgroups, all of them resident at once (one workgroup per CU, 256 CUs), bf16 records of
// 576 values or FP8 records.  A fetch workgroup attends T tiles of 64 entries: the smallest T
// for which R (S + 1) <= 256 with S = ceil(k / 64 T).  Returns S (and T), or 0 when the
// configuration does not take the fused kernel (whether LDS suffices is checked per device in
// hs_create).
int fused_chunks(const hs_config& c, int* tiles = nullptr) {
  if (!(c.flags & HS_CFG_RECORD_FP8) && c.record_bytes != kAttnDk * 2) return 0;
  if (!fused_supported(c.top_k, c.buffer_slots)) return 0;
  for (int T = 1; T <= kFusedMaxTiles; ++T) {
    const int S = (c.top_k + kTileRows * T - 1) / (kTileRows * T);
    if (int64_t(c.num_requests) * (S + 1) <= 256) {
      if (tiles) *tiles = T;
      return S;
    }
  }
  return 0;
}

Layout make_layout(const hs_config& c) {
  Layout L;
  const size_t R = c.num_requests, B = c.buffer_slots, k = c.top_k;
  L.A = (c.num_layers + c.layer_group - 1) / c.layer_group;
  L.Bpad = (int)align_up(B, 8);
  L.S = attn_chunks(c);
  const int Sf = fused_chunks(c);
  L.Spart = L.S > Sf ? L.S : Sf;
  L.kmax = c.top_k * (c.verify_rows > 1 ? c.verify_rows : 1);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  L.ctrl = take(size_t(L.A) * R * 4 * sizeof(uint32_t));
  L.slot_pos = take(size_t(L.A) * R * 2 * B * sizeof(int32_t));
  L.lru = take(size_t(L.A) * R * 2 * L.Bpad * sizeof(int16_t));
  L.plan = take(size_t(L.A) * R * 2 * L.kmax * sizeof(int32_t));
  L.page_table = take(size_t(L.A) * R * size_t(c.max_positions) * sizeof(uint64_t));
  L.newest = take(R * sizeof(int32_t));
  L.host_base = take(R * sizeof(void*));
  L.attn_part = take(size_t(c.num_layers) * R * L.Spart * kPartStride * sizeof(float));
  L.att_zero = take(size_t(c.record_bytes));  // a zero record: filler rows of FP8 tiles
  L.cap = take(R * sizeof(int32_t));           // backed slots per request (on-demand hot buffer)
  if (Sf) {  // the fused call's report, miss list and staging area (one set per handle)
    L.att_hdr = take(R * 4 * sizeof(uint32_t));
    L.att_mlist = take(R * k * 4 * sizeof(int32_t));
    L.att_stage = take(R * k * size_t(c.record_bytes));
  }
  if (c.verify_rows > 1) {  // union scratch of hs_resolve_rows (one set per handle)
    L.uni = take(R * L.kmax * sizeof(int32_t));
    L.umap = take(R * L.kmax * sizeof(int32_t));
    L.uout = take(R * L.kmax * sizeof(int32_t));
    L.ucnt = take(R * sizeof(int32_t));
    L.uerr = take(R * sizeof(uint32_t));
  }
  L.total = o;
  return L;
}

hs_status validate(const hs_config* c) {
  if (!c) return fail(HS_EINVAL, "null config");
  if (c->num_requests < 1 || c->num_requests > 65535) return fail(HS_EINVAL, "num_requests must be in [1, 65535]");
  if (c->num_layers < 1 || c->num_layers > 4096) return fail(HS_EINVAL, "num_layers must be in [1, 4096]");
  if (c->record_bytes < 16 || c->record_bytes > kMaxRecordBytes || c->record_bytes % 16)
    return fail(HS_EINVAL, "record_bytes must be a multiple of 16 in [16, %d]", kMaxRecordBytes);
  if (c->top_k < 1 || c->top_k > kMaxTopK) return fail(HS_EINVAL, "top_k must be in [1, %d]", kMaxTopK);
  if (c->buffer_slots < c->top_k || c->buffer_slots > kMaxSlots)
    return fail(HS_EINVAL, "buffer_slots must be in [top_k, %d]", kMaxSlots);
  if (c->block_tokens < 1 || !is_pow2(c->block_tokens) || c->block_tokens > 1024 ||
      c->top_k % c->block_tokens)
    return fail(HS_EINVAL, "block_tokens must be a power of two <= 1024 dividing top_k");
  if (c->max_positions < c->top_k || c->max_positions >= (int64_t(1) << 31))
    return fail(HS_EINVAL, "max_positions must be in [top_k, 2^31)");
  if (c->layer_group < 1 || c->layer_group > c->num_layers)
    return fail(HS_EINVAL, "layer_group must be in [1, num_layers]");
  if (c->wgs_per_request < 0 || c->wgs_per_request > 256)
    return fail(HS_EINVAL, "wgs_per_request must be in [0, 256]");
  if (c->flags & ~(HS_CFG_NEWEST_SLOT | HS_CFG_RECORD_FP8 | HS_CFG_HOT_ON_DEMAND))
    return fail(HS_EINVAL, "unknown config flags");
  if (c->verify_rows < 0 || c->verify_rows > 16) return fail(HS_EINVAL, "verify_rows must be in [0, 16]");
  if (c->verify_rows > 1) {
    if (int64_t(c->verify_rows) * c->top_k > kUnionMaxEntries)
      return fail(HS_EINVAL, "verify_rows * top_k must be <= %d", kUnionMaxEntries);
    if (c->buffer_slots < c->verify_rows * c->top_k)
      return fail(HS_EINVAL, "buffer_slots must hold the selections of all verification rows (>= verify_rows * top_k)");
  }
  if ((c->flags & HS_CFG_RECORD_FP8) && c->record_bytes != 656)
    return fail(HS_EINVAL, "HS_CFG_RECORD_FP8 needs record_bytes = 656");
  // every flattened copy index stays below 2^24 (kernels divide it in float)
  if (int64_t(c->top_k) * (c->record_bytes / 16) >= (int64_t(1) << 24) ||
      int64_t(c->num_requests) * c->num_layers * (c->record_bytes / 16) >= (int64_t(1) << 24))
    return fail(HS_EINVAL, "top_k * record_bytes / 16 and R * L * record_bytes / 16 must be < 2^24");
  return HS_OK;
}

int resolve_hash_bits(int k) {
  // table of >= 4k entries: at most a quarter full, short probe chains
  int bits = ilog2(int64_t(k) * 4);
  if (bits < 6) bits = 6;
  return bits;
}

}  // namespace

struct hs_ctx {
  hs_config cfg;
  Layout lay;
  int G = 1;
  int hash_bits = 0;
  size_t lds_bytes = 0;
  int spec_hash_bits = 0, union_hash_bits = 0;  // RESOLVE of a union, and the union kernel
  size_t spec_lds_bytes = 0;
  size_t rows_lds_bytes = 0;  // one-launch speculative rows (0: the union kernel, then its RESOLVE)
  int att_G = 0, att_T = 1, att_hash_bits = 0;  // fused RESOLVE + attention; att_G 0: not available
  size_t att_lds = 0;
  // measurement aid: kernel-timed RESOLVE launches (hs_timing_start / hs_timing_read)
  std::vector<KernelTiming> tm;
  size_t tm_next = 0;
  const KernelTiming* next_timing() { return tm_next < tm.size() ? &tm[tm_next++] : nullptr; }
  int device = 0;
  uint8_t* hot = nullptr;
  uint8_t* ws = nullptr;
  std::vector<void*> pool;  // per request pinned region
  hipEvent_t ev_appended = nullptr, ev_backup_done = nullptr;
  bool backup_pending = false;  // a backup-stream write-through may still read slot B
  std::vector<hipEvent_t> ev_plan, ev_plan_free, ev_layer;  // per anchor, per anchor, per layer
  std::vector<char> plan_free_pending;
  int replay_wgs = 32;
  // resident tier (hs_bind_resident); rtable null when none is bound
  const int32_t* rtable = nullptr;
  int64_t rt_stride = 0, res_rows = 0;
  int page_shift = 0;
  const uint8_t* res = nullptr;
  // on-demand hot buffer (HS_CFG_HOT_ON_DEMAND): the reserved range, its mapped kHotChunk chunks,
  // and each request's capacity as the host granted it
  bool on_demand = false;
  size_t hot_va_bytes = 0;
  std::vector<hipMemGenericAllocationHandle_t> chunks;
  int64_t mapped_chunks = 0;
  std::vector<int32_t> cap_host;
  int32_t* cap_dev() { return on_demand ? (int32_t*)(ws + lay.cap) : nullptr; }

  uint32_t* ctrl(int a) { return (uint32_t*)(ws + lay.ctrl) + size_t(a) * cfg.num_requests * 4; }
  int32_t* slot_pos(int a) {
    return (int32_t*)(ws + lay.slot_pos) + size_t(a) * cfg.num_requests * 2 * cfg.buffer_slots;
  }
  int16_t* lru(int a) { return (int16_t*)(ws + lay.lru) + size_t(a) * cfg.num_requests * 2 * lay.Bpad; }
  int32_t* plan(int a) { return (int32_t*)(ws + lay.plan) + size_t(a) * cfg.num_requests * 2 * lay.kmax; }
  uint64_t* page_table(int a) {
    return (uint64_t*)(ws + lay.page_table) + size_t(a) * cfg.num_requests * size_t(cfg.max_positions);
  }
  int32_t* newest() { return (int32_t*)(ws + lay.newest); }
  const uint8_t* const* host_base() { return (const uint8_t* const*)(ws + lay.host_base); }
  float* attn_part(int l) {
    return (float*)(ws + lay.attn_part) + size_t(l) * cfg.num_requests * lay.Spart * kPartStride;
  }
  int64_t host_layer_off(int l) const { return int64_t(l) * cfg.max_positions * cfg.record_bytes; }
  int64_t hot_req_stride() const { return int64_t(cfg.num_layers) * (cfg.buffer_slots + 1) * cfg.record_bytes; }
  int64_t hot_layer_off(int l) const { return int64_t(l) * (cfg.buffer_slots + 1) * cfg.record_bytes; }
  bool is_anchor(int l) const { return l % cfg.layer_group == 0; }
};

namespace {

void destroy_events(hs_ctx* h) {
  if (h->ev_appended) (void)hipEventDestroy(h->ev_appended);
  if (h->ev_backup_done) (void)hipEventDestroy(h->ev_backup_done);
  for (auto e : h->ev_plan) if (e) (void)hipEventDestroy(e);
  for (auto e : h->ev_plan_free) if (e) (void)hipEventDestroy(e);
  for (auto e : h->ev_layer) if (e) (void)hipEventDestroy(e);
}

void free_timing(hs_ctx* h) {
  for (auto& t : h->tm) {
    if (t.start) (void)hipEventDestroy(t.start);
    if (t.stop) (void)hipEventDestroy(t.stop);
  }
  h->tm.clear();
  h->tm_next = 0;
}

void free_ctx(hs_ctx* h) {
  if (!h) return;
  destroy_events(h);
  free_timing(h);
  for (void* p : h->pool) if (p) (void)hipHostFree(p);
  if (h->on_demand && h->hot) {
    // no kernel may still use the range: the device finishes its work first
    (void)hipDeviceSynchronize();
    for (size_t c = 0; c < h->chunks.size(); ++c) {
      if (!h->chunks[c]) continue;
      (void)hipMemUnmap(h->hot + c * kHotChunk, kHotChunk);
      (void)hipMemRelease(h->chunks[c]);
    }
    (void)hipMemAddressFree(h->hot, h->hot_va_bytes);
  }
  delete h;
}

// Backs the chunks of the on-demand hot buffer that overlap bytes [lo, hi) with device memory.
hs_status map_hot_range(hs_ctx* h, size_t lo, size_t hi) {
  if (hi <= lo) return HS_OK;
  hipMemAllocationProp prop = {};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = h->device;
  hipMemAccessDesc acc = {};
  acc.location = prop.location;
  acc.flags = hipMemAccessFlagsProtReadWrite;
  for (size_t c = lo / kHotChunk; c <= (hi - 1) / kHotChunk; ++c) {
    if (h->chunks[c]) continue;
    hipMemGenericAllocationHandle_t hnd;
    hipError_t e = hipMemCreate(&hnd, kHotChunk, &prop, 0);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(HS_ENOMEM, "backing the hot buffer: %s", hipGetErrorString(e));
    }
    void* at = h->hot + c * kHotChunk;
    e = hipMemMap(at, kHotChunk, 0, hnd, 0);
    if (e == hipSuccess) e = hipMemSetAccess(at, kHotChunk, &acc, 1);
    if (e != hipSuccess) {
      (void)hipMemUnmap(at, kHotChunk);
      (void)hipMemRelease(hnd);
      return hip_fail(e, "mapping the hot buffer");
    }
    h->chunks[c] = hnd;
    ++h->mapped_chunks;
  }
  return HS_OK;
}

hs_status check_handle(hs_ctx* h) {
  if (!h) return fail(HS_EINVAL, "null handle");
  return HS_OK;
}

hs_status check_layer(hs_ctx* h, int32_t layer) {
  if (layer < 0 || layer >= h->cfg.num_layers) return fail(HS_EINVAL, "layer %d out of range", layer);
  return HS_OK;
}

// The RESOLVE launch of one anchor layer (the fused call overrides G and the hash size).
ResolveParams resolve_params(hs_ctx* h, int32_t layer, const int32_t* d_sel, const int32_t* d_ctx_len,
                             int32_t* d_slots_out, hs_stats* d_stats, const int32_t* d_num_reqs, uint32_t flags) {
  const int a = layer / h->cfg.layer_group;
  ResolveParams p{};
  p.sel = d_sel; p.ctx_len = d_ctx_len; p.out = d_slots_out; p.stats = d_stats; p.num_reqs = d_num_reqs;
  p.ctrl = h->ctrl(a); p.slot_pos = h->slot_pos(a); p.lru = h->lru(a); p.plan = h->plan(a);
  p.page_table = h->page_table(a); p.newest = h->newest(); p.host_base = h->host_base(); p.hot = h->hot;
  p.host_layer_off = h->host_layer_off(layer); p.hot_req_stride = h->hot_req_stride();
  p.hot_layer_off = h->hot_layer_off(layer); p.max_positions = h->cfg.max_positions;
  p.R = h->cfg.num_requests; p.B = h->cfg.buffer_slots; p.Bpad = h->lay.Bpad; p.k = h->cfg.top_k;
  p.kb = h->cfg.top_k / h->cfg.block_tokens; p.bt_shift = ilog2(h->cfg.block_tokens);
  p.rec_bytes = h->cfg.record_bytes; p.G = h->G; p.hash_bits = h->hash_bits;
  p.flags = flags | ((h->cfg.flags & HS_CFG_NEWEST_SLOT) ? kHasNewest : 0u);
  p.rtable = h->rtable; p.rt_stride = h->rt_stride; p.res_rows = h->res_rows; p.page_shift = h->page_shift;
  p.plan_k = h->lay.kmax;
  p.cap = h->cap_dev();
  return p;
}

}  // namespace

extern "C" {

size_t hs_workspace_bytes(const hs_config* cfg) {
  if (validate(cfg) != HS_OK) return 0;
  return make_layout(*cfg).total;
}

hs_status hs_create(const hs_config* cfg, void* d_hot, void* d_workspace, hs_handle* out) {
  if (!out) return fail(HS_EINVAL, "null output handle");
  *out = nullptr;
  hs_status st = validate(cfg);
  if (st != HS_OK) return st;
  const bool on_demand = (cfg->flags & HS_CFG_HOT_ON_DEMAND) != 0;
  if (on_demand && d_hot) return fail(HS_EINVAL, "HS_CFG_HOT_ON_DEMAND: the library reserves the hot buffer (d_hot = NULL)");
  if ((!d_hot && !on_demand) || !d_workspace) return fail(HS_EINVAL, "null hot buffer or workspace");
  if ((uintptr_t)d_hot % 16 || (uintptr_t)d_workspace % 256)
    return fail(HS_EINVAL, "hot buffer must be 16-byte and workspace 256-byte aligned");

  hs_ctx* h = new (std::nothrow) hs_ctx();
  if (!h) return fail(HS_ENOMEM, "handle allocation failed");
  h->cfg = *cfg;
  h->lay = make_layout(*cfg);
  h->hot = (uint8_t*)d_hot;
  h->ws = (uint8_t*)d_workspace;
  h->hash_bits = resolve_hash_bits(cfg->top_k);
  if (cfg->wgs_per_request > 0) {
    h->G = cfg->wgs_per_request;
  } else {
    // enough workgroups per request to keep the host link busy on a miss-heavy step
    int G = 128 / cfg->num_requests;
    h->G = G < 1 ? 1 : (G > 32 ? 32 : G);
  }
  // resolve grid: R * G workgroups of 1024 threads
  if (int64_t(cfg->num_requests) * h->G > (int64_t(1) << 21)) {
    free_ctx(h);
    return fail(HS_EINVAL, "num_requests * wgs_per_request too large for one resolve launch");
  }
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) { free_ctx(h); return hip_fail(e, "hipGetDevice"); }
  // this device's address of the allocation-free attention's partials (once per device)
  e = attn_scratch_init(h->device);
  if (e != hipSuccess) { free_ctx(h); return hip_fail(e, "hipGetSymbolAddress(attention scratch)"); }
  if (on_demand) {  // the hot buffer's address range, backed later by hs_grow_request
    int vmm = 0;
    e = hipDeviceGetAttribute(&vmm, hipDeviceAttributeVirtualMemoryManagementSupported, h->device);
    if (e != hipSuccess || !vmm) {
      free_ctx(h);
      return fail(HS_EINVAL, "HS_CFG_HOT_ON_DEMAND: the device has no virtual memory management");
    }
    hipMemAllocationProp prop = {};
    prop.type = hipMemAllocationTypePinned;
    prop.location.type = hipMemLocationTypeDevice;
    prop.location.id = h->device;
    size_t gran = 0;
    e = hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum);
    if (e != hipSuccess || gran == 0 || kHotChunk % gran) {
      free_ctx(h);
      return fail(HS_EINVAL, "HS_CFG_HOT_ON_DEMAND: allocation granularity %zu does not divide %zu", gran, kHotChunk);
    }
    const size_t bytes = size_t(cfg->num_requests) * cfg->num_layers * (size_t(cfg->buffer_slots) + 1) *
                         size_t(cfg->record_bytes);
    h->hot_va_bytes = align_up(bytes, kHotChunk);
    void* va = nullptr;
    e = hipMemAddressReserve(&va, h->hot_va_bytes, kHotChunk, nullptr, 0);
    if (e != hipSuccess) { free_ctx(h); return hip_fail(e, "hipMemAddressReserve(hot buffer)"); }
    h->on_demand = true;
    h->hot = (uint8_t*)va;
    h->chunks.assign(h->hot_va_bytes / kHotChunk, hipMemGenericAllocationHandle_t{});
    h->cap_host.assign(cfg->num_requests, 0);
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, h->device);
  if (e != hipSuccess) { free_ctx(h); return hip_fail(e, "hipGetDeviceProperties"); }
  // hash table of 4k entries (a quarter full), or 2k (half full) when LDS is short
  auto fit = [&](int k, int& bits, size_t& lds) {
    bits = resolve_hash_bits(k);
    lds = resolve_lds(k, cfg->buffer_slots, bits, h->G).total;
    if (lds > prop.sharedMemPerBlock) {
      bits -= 1;
      lds = resolve_lds(k, cfg->buffer_slots, bits, h->G).total;
    }
    return lds <= prop.sharedMemPerBlock;
  };
  if (!fit(cfg->top_k, h->hash_bits, h->lds_bytes)) {
    size_t need = h->lds_bytes;
    free_ctx(h);
    return fail(HS_EINVAL, "resolve needs %zu bytes of LDS, device allows %zu", need, (size_t)prop.sharedMemPerBlock);
  }
  if (cfg->verify_rows > 1) {
    if (!fit(h->lay.kmax, h->spec_hash_bits, h->spec_lds_bytes)) {
      size_t need = h->spec_lds_bytes;
      free_ctx(h);
      return fail(HS_EINVAL, "resolving %d verification rows needs %zu bytes of LDS, device allows %zu",
                  cfg->verify_rows, need, (size_t)prop.sharedMemPerBlock);
    }
    h->union_hash_bits = ilog2(int64_t(2) * h->lay.kmax);  // at most half full
    if (h->union_hash_bits < 6) h->union_hash_bits = 6;
    if (union_lds_bytes(h->union_hash_bits) > prop.sharedMemPerBlock) {
      free_ctx(h);
      return fail(HS_EINVAL, "the union of %d rows needs too much LDS", cfg->verify_rows);
    }
    // a union whose capacity needs more than kUnionShortKE entries per thread: built and resolved
    // in one launch where the union's table and RESOLVE's carve-up (after the list) fit LDS
    if ((h->lay.kmax + kResolveThreads - 1) / kResolveThreads > kUnionShortKE) {
      const size_t lds = rows_lds(h->lay.kmax, cfg->buffer_slots, h->spec_hash_bits, h->G, h->union_hash_bits);
      if (lds <= prop.sharedMemPerBlock) h->rows_lds_bytes = lds;
    }
  }
  // fused RESOLVE + attention: G = chunks + 1, when its LDS fits (a half-full hash if need be)
  int T = 1;
  if (const int Sf = fused_chunks(*cfg, &T)) {
    const int G = Sf + 1;
    int bits = resolve_hash_bits(cfg->top_k);
    const bool f8 = (cfg->flags & HS_CFG_RECORD_FP8) != 0;
    size_t lds = fused_lds(cfg->top_k, cfg->buffer_slots, bits, G, T, f8).total;
    if (lds > prop.sharedMemPerBlock) {
      bits -= 1;
      lds = fused_lds(cfg->top_k, cfg->buffer_slots, bits, G, T, f8).total;
    }
    if (lds <= prop.sharedMemPerBlock) {
      h->att_G = G;
      h->att_T = T;
      h->att_hash_bits = bits;
      h->att_lds = lds;
    }
  }
  // the limit is per kernel, not per handle: allow the device maximum once
  e = set_resolve_lds_limit(prop.sharedMemPerBlock);
  if (e == hipSuccess) e = set_union_lds_limit(prop.sharedMemPerBlock);
  if (e != hipSuccess) { free_ctx(h); return hip_fail(e, "hipFuncSetAttribute(resolve)"); }

  // pinned host pool: one allocation per request (the driver refuses single pins near 80 GiB)
  const size_t per_req = size_t(cfg->num_layers) * size_t(cfg->max_positions) * size_t(cfg->record_bytes);
  h->pool.assign(cfg->num_requests, nullptr);
  std::vector<const void*> dev_bases(cfg->num_requests);
  for (int r = 0; r < cfg->num_requests; ++r) {
    e = hipHostMalloc(&h->pool[r], per_req, hipHostMallocCoherent | hipHostMallocMapped);
    if (e != hipSuccess) {
      h->pool[r] = nullptr;
      (void)hipGetLastError();
      free_ctx(h);
      return fail(HS_ENOMEM, "pinning %zu bytes for request %d failed: %s", per_req, r, hipGetErrorString(e));
    }
    void* dptr = nullptr;
    e = hipHostGetDevicePointer(&dptr, h->pool[r], 0);
    if (e != hipSuccess) { free_ctx(h); return hip_fail(e, "hipHostGetDevicePointer"); }
    dev_bases[r] = dptr;
  }

  // events (timing disabled: ordering only)
  const int A = h->lay.A;
  h->ev_plan.assign(A, nullptr);
  h->ev_plan_free.assign(A, nullptr);
  h->plan_free_pending.assign(A, 0);
  h->ev_layer.assign(cfg->num_layers, nullptr);
  auto mk = [&](hipEvent_t* ev) { return hipEventCreateWithFlags(ev, hipEventDisableTiming); };
  if ((e = mk(&h->ev_appended)) != hipSuccess || (e = mk(&h->ev_backup_done)) != hipSuccess) {
    free_ctx(h);
    return hip_fail(e, "hipEventCreate");
  }
  for (int a = 0; a < A; ++a)
    if ((e = mk(&h->ev_plan[a])) != hipSuccess || (e = mk(&h->ev_plan_free[a])) != hipSuccess) {
      free_ctx(h);
      return hip_fail(e, "hipEventCreate");
    }
  for (int l = 0; l < cfg->num_layers; ++l)
    if (!h->is_anchor(l) && (e = mk(&h->ev_layer[l])) != hipSuccess) {
      free_ctx(h);
      return hip_fail(e, "hipEventCreate");
    }

  // workspace: zero, then the admission state; host base table
  e = hipMemset(h->ws, 0, h->lay.total);
  if (e == hipSuccess)
    e = hipMemcpy(h->ws + h->lay.host_base, dev_bases.data(), sizeof(void*) * cfg->num_requests,
                  hipMemcpyHostToDevice);
  if (e == hipSuccess) {
    InitParams ip{};
    ip.ctrl = h->ctrl(0); ip.slot_pos = h->slot_pos(0); ip.lru = h->lru(0);
    ip.page_table = h->page_table(0); ip.newest = h->newest();
    ip.max_positions = cfg->max_positions; ip.R = cfg->num_requests; ip.B = cfg->buffer_slots;
    ip.Bpad = h->lay.Bpad; ip.A = A; ip.request = -1;
    e = launch_init(ip, nullptr);
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) { free_ctx(h); return hip_fail(e, "workspace initialisation"); }
  *out = h;
  g_last_error.clear();
  return HS_OK;
}

void* hs_host_pool(hs_handle h, int32_t request) {
  if (!h || request < 0 || request >= h->cfg.num_requests) return nullptr;
  return h->pool[request];
}

void* hs_hot_buffer(hs_handle h) { return h ? (void*)h->hot : nullptr; }

int64_t hs_hot_backed_bytes(hs_handle h) {
  if (!h) return -1;
  if (!h->on_demand) return int64_t(h->cfg.num_requests) * h->hot_req_stride();
  return h->mapped_chunks * int64_t(kHotChunk);
}

hs_status hs_grow_request(hs_handle h, int32_t request, int32_t slots, void* stream) {
  hs_status st;
  if ((st = check_handle(h))) return st;
  if (request < 0 || request >= h->cfg.num_requests) return fail(HS_EINVAL, "request out of range");
  if (slots < 0 || slots > h->cfg.buffer_slots) return fail(HS_EINVAL, "slots must be in [0, buffer_slots]");
  if (!h->on_demand) return HS_OK;  // a caller-owned hot buffer is backed throughout
  // every layer's slots [0, slots) and its newest slot B
  const size_t rec = h->cfg.record_bytes;
  for (int l = 0; l < h->cfg.num_layers; ++l) {
    const size_t base = size_t(request) * h->hot_req_stride() + h->hot_layer_off(l);
    if ((st = map_hot_range(h, base, base + size_t(slots) * rec))) return st;
    const size_t nb = base + size_t(h->cfg.buffer_slots) * rec;
    if ((st = map_hot_range(h, nb, nb + rec))) return st;
  }
  if (slots > h->cap_host[request]) {
    h->cap_host[request] = slots;
    HS_HIP(launch_set_capacity(h->cap_dev(), request, slots, (hipStream_t)stream));
  }
  return HS_OK;
}

int32_t hs_resolve_wgs(hs_handle h) { return h ? h->G : 0; }

int32_t hs_resolve_attn_wgs(hs_handle h) { return h ? h->att_G : 0; }

hs_status hs_resolve(hs_handle h, int32_t layer, const int32_t* d_sel, const int32_t* d_ctx_len,
                     int32_t* d_slots_out, hs_stats* d_stats, const int32_t* d_num_reqs, uint32_t flags,
                     void* stream) {
  hs_status st;
  if ((st = check_handle(h)) || (st = check_layer(h, layer))) return st;
  if (!h->is_anchor(layer))
    return fail(HS_ESTATE, "layer %d shares its anchor's selection: use hs_prefetch_shared", layer);
  if (!d_sel || !d_ctx_len || !d_slots_out) return fail(HS_EINVAL, "null selection, ctx_len or output");
  if (flags & ~(HS_RECORD_PLAN | HS_SKIP_IO)) return fail(HS_EINVAL, "unknown resolve flags");
  hipStream_t s = (hipStream_t)stream;
  const int a = layer / h->cfg.layer_group;
  if ((flags & HS_RECORD_PLAN) && h->plan_free_pending[a]) {
    // the previous plan of this anchor must be replayed before it is overwritten
    HS_HIP(hipStreamWaitEvent(s, h->ev_plan_free[a], 0));
  }
  ResolveParams p = resolve_params(h, layer, d_sel, d_ctx_len, d_slots_out, d_stats, d_num_reqs, flags);
  HS_HIP(launch_resolve(p, h->lds_bytes, s, h->next_timing()));
  return HS_OK;
}

hs_status hs_resolve_attn(hs_handle h, int32_t layer, const int32_t* d_sel, const int32_t* d_ctx_len,
                          int32_t* d_slots_out, hs_stats* d_stats, const int32_t* d_num_reqs, uint32_t flags,
                          const void* d_q, int32_t heads, int32_t value_dim, float* d_out, float scale,
                          void* stream) {
  hs_status st;
  if ((st = check_handle(h)) || (st = check_layer(h, layer))) return st;
  if (flags & HS_SKIP_IO) return fail(HS_EINVAL, "hs_resolve_attn reads the records: HS_SKIP_IO is not allowed");
  if (!h->att_G) {  // no fused kernel for this configuration: the same two calls in sequence
    if ((st = hs_resolve(h, layer, d_sel, d_ctx_len, d_slots_out, d_stats, d_num_reqs, flags, stream))) return st;
    return hs_sparse_attn(h, layer, d_q, heads, value_dim, d_slots_out, d_out, scale, d_num_reqs, stream);
  }
  if (!h->is_anchor(layer))
    return fail(HS_ESTATE, "layer %d shares its anchor's selection: use hs_prefetch_shared", layer);
  if (!d_sel || !d_ctx_len || !d_slots_out) return fail(HS_EINVAL, "null selection, ctx_len or output");
  if (flags & ~(HS_RECORD_PLAN | HS_SKIP_IO)) return fail(HS_EINVAL, "unknown resolve flags");
  if (heads < 1 || heads > kAttnMaxHeads) return fail(HS_EINVAL, "heads must be in [1, %d]", kAttnMaxHeads);
  if (value_dim != kAttnDv) return fail(HS_EINVAL, "value_dim must be %d", kAttnDv);
  if (!d_q || !d_out) return fail(HS_EINVAL, "null q or output");
  if ((uintptr_t)d_q % 16) return fail(HS_EINVAL, "q must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const int a = layer / h->cfg.layer_group;
  if ((flags & HS_RECORD_PLAN) && h->plan_free_pending[a]) HS_HIP(hipStreamWaitEvent(s, h->ev_plan_free[a], 0));
  ResolveParams p = resolve_params(h, layer, d_sel, d_ctx_len, d_slots_out, d_stats, d_num_reqs, flags);
  p.G = h->att_G; p.hash_bits = h->att_hash_bits;
  p.q = (const uint16_t*)d_q; p.part = h->attn_part(layer); p.att_out = d_out;
  p.att_res = h->res ? h->res + size_t(layer) * size_t(h->res_rows) * size_t(h->cfg.record_bytes) : nullptr;
  p.heads = heads; p.att_tiles = h->att_T; p.att_scale = scale; p.att_zero = h->ws + h->lay.att_zero;
  p.att_hdr = (uint32_t*)(h->ws + h->lay.att_hdr); p.att_mlist = (int32_t*)(h->ws + h->lay.att_mlist);
  p.att_stage = h->ws + h->lay.att_stage;
  HS_HIP(launch_resolve_attn(p, h->att_lds, s, h->next_timing()));
  // the chunk merge (or NaN rows), the staged misses into their slots, the page-table updates
  FinishParams f{};
  f.out = d_out; f.part = h->attn_part(layer); f.num_reqs = d_num_reqs; f.hdr = p.att_hdr; f.mlist = p.att_mlist;
  f.stage = p.att_stage; f.hot = h->hot; f.hot_req_stride = h->hot_req_stride(); f.hot_layer_off = h->hot_layer_off(layer);
  f.page_table = h->page_table(a); f.max_positions = h->cfg.max_positions; f.R = h->cfg.num_requests;
  f.heads = heads; f.value_dim = value_dim; f.S = h->att_G - 1; f.k = h->cfg.top_k;
  f.rec_bytes = h->cfg.record_bytes; f.merge_blocks = h->cfg.num_requests * heads;
  HS_HIP(launch_attn_finish(f, s));
  return HS_OK;
}

hs_status hs_resolve_rows(hs_handle h, int32_t layer, int32_t rows, const int32_t* d_sel, const int32_t* d_ctx_len,
                          int32_t* d_slots_out, hs_stats* d_stats, const int32_t* d_num_reqs, uint32_t flags,
                          void* stream) {
  hs_status st;
  if ((st = check_handle(h)) || (st = check_layer(h, layer))) return st;
  if (h->cfg.verify_rows < 2) return fail(HS_ESTATE, "hs_resolve_rows needs verify_rows > 1 in the config");
  if (rows < 1 || rows > h->cfg.verify_rows) return fail(HS_EINVAL, "rows must be in [1, %d]", h->cfg.verify_rows);
  if (!h->is_anchor(layer))
    return fail(HS_ESTATE, "layer %d shares its anchor's selection: use hs_prefetch_shared", layer);
  if (!d_sel || !d_ctx_len || !d_slots_out) return fail(HS_EINVAL, "null selection, ctx_len or output");
  if (flags & ~(HS_RECORD_PLAN | HS_SKIP_IO)) return fail(HS_EINVAL, "unknown resolve flags");
  hipStream_t s = (hipStream_t)stream;
  const int a = layer / h->cfg.layer_group;
  const int R = h->cfg.num_requests, kmax = h->lay.kmax;
  int32_t* uni = (int32_t*)(h->ws + h->lay.uni);
  int32_t* umap = (int32_t*)(h->ws + h->lay.umap);
  int32_t* uout = (int32_t*)(h->ws + h->lay.uout);
  int32_t* ucnt = (int32_t*)(h->ws + h->lay.ucnt);
  uint32_t* uerr = (uint32_t*)(h->ws + h->lay.uerr);
  UnionParams u{};
  u.sel = d_sel; u.ctx_len = d_ctx_len; u.num_reqs = d_num_reqs; u.uni = uni; u.map = umap; u.cnt = ucnt;
  u.err = uerr; u.max_positions = h->cfg.max_positions; u.R = R; u.rows = rows; u.k = h->cfg.top_k;
  u.kb = h->cfg.top_k / h->cfg.block_tokens; u.bt_shift = ilog2(h->cfg.block_tokens); u.kmax = kmax;
  u.hash_bits = h->union_hash_bits;
  const bool one_launch = h->rows_lds_bytes != 0;
  if (!one_launch) HS_HIP(launch_union(u, s));
  if ((flags & HS_RECORD_PLAN) && h->plan_free_pending[a]) HS_HIP(hipStreamWaitEvent(s, h->ev_plan_free[a], 0));
  ResolveParams p{};
  p.sel = uni; p.ctx_len = d_ctx_len; p.out = uout; p.stats = d_stats; p.num_reqs = d_num_reqs;
  p.kvar = ucnt; p.kerr = uerr;
  p.ctrl = h->ctrl(a); p.slot_pos = h->slot_pos(a); p.lru = h->lru(a); p.plan = h->plan(a);
  p.page_table = h->page_table(a); p.newest = h->newest(); p.host_base = h->host_base(); p.hot = h->hot;
  p.host_layer_off = h->host_layer_off(layer); p.hot_req_stride = h->hot_req_stride();
  p.hot_layer_off = h->hot_layer_off(layer); p.max_positions = h->cfg.max_positions;
  p.R = R; p.B = h->cfg.buffer_slots; p.Bpad = h->lay.Bpad; p.k = kmax; p.kb = kmax; p.bt_shift = 0;
  p.rec_bytes = h->cfg.record_bytes; p.G = h->G; p.hash_bits = h->spec_hash_bits;
  p.flags = flags | ((h->cfg.flags & HS_CFG_NEWEST_SLOT) ? kHasNewest : 0u);
  p.rtable = h->rtable; p.rt_stride = h->rt_stride; p.res_rows = h->res_rows; p.page_shift = h->page_shift;
  p.plan_k = kmax;
  p.cap = h->cap_dev();
  // the rows' slots from the union's (by the union's RESOLVE kernel, or a scatter kernel after it)
  p.rows_out = d_slots_out; p.rows_map = umap; p.rows_n = rows * h->cfg.top_k;
  if (one_launch) HS_HIP(launch_resolve_rows(p, u, h->rows_lds_bytes, s, h->next_timing()));
  else HS_HIP(launch_resolve(p, h->spec_lds_bytes, s, h->next_timing()));
  return HS_OK;
}

hs_status hs_bind_resident(hs_handle h, const int32_t* d_block_table, int32_t pages_per_request,
                           int32_t page_tokens, const void* d_resident_kv, int64_t resident_rows) {
  hs_status st;
  if ((st = check_handle(h))) return st;
  if (!d_block_table) {
    h->rtable = nullptr; h->res = nullptr; h->rt_stride = 0; h->res_rows = 0; h->page_shift = 0;
    return HS_OK;
  }
  if (page_tokens < 1 || page_tokens > (1 << 20) || !is_pow2(page_tokens))
    return fail(HS_EINVAL, "page_tokens must be a power of two in [1, 2^20]");
  if (pages_per_request < 1 || int64_t(pages_per_request) * page_tokens < h->cfg.max_positions)
    return fail(HS_EINVAL, "pages_per_request * page_tokens must cover max_positions");
  if (!d_resident_kv || (uintptr_t)d_resident_kv % 16) return fail(HS_EINVAL, "resident pool must be 16-byte aligned");
  if (resident_rows < 1 || resident_rows > (int64_t(1) << 31) - 2 - h->cfg.buffer_slots)
    return fail(HS_EINVAL, "resident_rows must be in [1, 2^31 - 2 - B]");
  h->rtable = d_block_table; h->rt_stride = pages_per_request; h->page_shift = ilog2(page_tokens);
  h->res = (const uint8_t*)d_resident_kv; h->res_rows = resident_rows;
  return HS_OK;
}

hs_status hs_writeback(hs_handle h, const void* d_new_kv, const int32_t* d_new_pos, void* compute, void* backup) {
  hs_status st;
  if ((st = check_handle(h))) return st;
  if (!(h->cfg.flags & HS_CFG_NEWEST_SLOT)) return fail(HS_ESTATE, "hs_writeback needs HS_CFG_NEWEST_SLOT");
  if (!d_new_kv || !d_new_pos) return fail(HS_EINVAL, "null new record or position");
  hipStream_t cs = (hipStream_t)compute, bs = (hipStream_t)backup;
  AppendParams p{};
  p.new_kv = (const uint8_t*)d_new_kv; p.new_pos = d_new_pos; p.newest = h->newest(); p.hot = h->hot;
  p.host_base = h->host_base(); p.max_positions = h->cfg.max_positions; p.R = h->cfg.num_requests;
  p.L = h->cfg.num_layers; p.B = h->cfg.buffer_slots; p.rec_bytes = h->cfg.record_bytes;
  p.ctrl = h->ctrl(0); p.slot_pos = h->slot_pos(0); p.page_table = h->page_table(0); p.A = h->lay.A;
  p.group = h->cfg.layer_group; p.cap = h->cap_dev();
  // Slot B may only be overwritten once the previous write-through has read it (and then every
  // later fetch of the previous newest position finds its bytes on the host).
  if (!backup || backup == compute) {
    // One kernel on `compute` writes slot B and the host pool, ordered with the caller's later
    // work by the stream itself.  A cross-stream event pair costs more GPU time per step than
    // writing a few records to the host, so this is the mode for small appends.
    if (h->backup_pending) HS_HIP(hipStreamWaitEvent(cs, h->ev_backup_done, 0));
    h->backup_pending = false;
    HS_HIP(launch_append(p, cs, true));
    return HS_OK;
  }
  HS_HIP(hipStreamWaitEvent(cs, h->ev_backup_done, 0));
  HS_HIP(launch_append(p, cs, false));
  HS_HIP(hipEventRecord(h->ev_appended, cs));
  HS_HIP(hipStreamWaitEvent(bs, h->ev_appended, 0));
  HS_HIP(launch_backup(p, bs));
  HS_HIP(hipEventRecord(h->ev_backup_done, bs));
  h->backup_pending = true;
  return HS_OK;
}

hs_status hs_prefetch_shared(hs_handle h, int32_t anchor_layer, void* compute, void* prefetch) {
  hs_status st;
  if ((st = check_handle(h)) || (st = check_layer(h, anchor_layer))) return st;
  if (!h->is_anchor(anchor_layer)) return fail(HS_EINVAL, "layer %d is not an anchor", anchor_layer);
  const int a = anchor_layer / h->cfg.layer_group;
  const int last = anchor_layer + h->cfg.layer_group - 1 < h->cfg.num_layers
                       ? anchor_layer + h->cfg.layer_group - 1 : h->cfg.num_layers - 1;
  if (last == anchor_layer) return HS_OK;  // no shared layers
  hipStream_t cs = (hipStream_t)compute, ps = (hipStream_t)prefetch;
  HS_HIP(hipEventRecord(h->ev_plan[a], cs));
  HS_HIP(hipStreamWaitEvent(ps, h->ev_plan[a], 0));
  for (int l = anchor_layer + 1; l <= last; ++l) {
    ReplayParams p{};
    p.plan = h->plan(a); p.ctrl = h->ctrl(a); p.host_base = h->host_base(); p.hot = h->hot;
    p.host_layer_off = h->host_layer_off(l); p.hot_req_stride = h->hot_req_stride();
    p.hot_layer_off = h->hot_layer_off(l); p.R = h->cfg.num_requests; p.plan_k = h->lay.kmax;
    p.rec_bytes = h->cfg.record_bytes;
    HS_HIP(launch_replay(p, h->replay_wgs, ps, h->next_timing()));
    HS_HIP(hipEventRecord(h->ev_layer[l], ps));
  }
  HS_HIP(hipEventRecord(h->ev_plan_free[a], ps));
  h->plan_free_pending[a] = 1;
  return HS_OK;
}

hs_status hs_wait_layer(hs_handle h, int32_t layer, void* stream) {
  hs_status st;
  if ((st = check_handle(h)) || (st = check_layer(h, layer))) return st;
  if (h->is_anchor(layer)) return HS_OK;  // an anchor's bytes are in place when its resolve ends
  HS_HIP(hipStreamWaitEvent((hipStream_t)stream, h->ev_layer[layer], 0));
  return HS_OK;
}

}  // extern "C"

namespace {

// The attention launch of one layer (hs_sparse_attn and hs_sparse_attn_static), after the
// argument checks; partials in the handle's workspace.
hs_status attn_params(hs_ctx* h, int32_t layer, const void* d_q, int32_t heads, int32_t value_dim,
                      const int32_t* d_slots, float* d_out, float scale, const int32_t* d_num_reqs, AttnParams* out) {
  hs_status st;
  if ((st = check_handle(h)) || (st = check_layer(h, layer))) return st;
  const bool fp8 = (h->cfg.flags & HS_CFG_RECORD_FP8) != 0;
  if (!fp8 && h->cfg.record_bytes != kAttnDk * 2)
    return fail(HS_EINVAL, "attention needs 576-element bf16 records (or HS_CFG_RECORD_FP8)");
  if (heads < 1 || heads > kAttnMaxHeads) return fail(HS_EINVAL, "heads must be in [1, %d]", kAttnMaxHeads);
  if (value_dim != kAttnDv) return fail(HS_EINVAL, "value_dim must be %d", kAttnDv);
  if (!d_q || !d_slots || !d_out) return fail(HS_EINVAL, "null q, slots or output");
  if ((uintptr_t)d_q % 16) return fail(HS_EINVAL, "q must be 16-byte aligned");
  AttnParams p{};
  p.q = (const uint16_t*)d_q; p.slots = d_slots; p.out = d_out; p.part = h->attn_part(layer);
  p.num_reqs = d_num_reqs; p.hot = h->hot;
  p.hot_req_stride = h->hot_req_stride(); p.hot_layer_off = h->hot_layer_off(layer);
  p.res = h->res ? h->res + size_t(layer) * size_t(h->res_rows) * size_t(h->cfg.record_bytes) : nullptr;
  p.res_rows = h->res ? h->res_rows : 0;
  p.R = h->cfg.num_requests; p.k = h->cfg.top_k; p.B = h->cfg.buffer_slots; p.heads = heads;
  p.value_dim = value_dim; p.S = h->lay.S;
  p.chunk = (int)align_up((size_t)((h->cfg.top_k + p.S - 1) / p.S), 64);
  p.S = (h->cfg.top_k + p.chunk - 1) / p.chunk;  // no empty chunk
  p.rec_bytes = h->cfg.record_bytes; p.scale = scale; p.fp8 = fp8 ? 1 : 0;
  p.zero = h->ws + h->lay.att_zero;
  p.cap = h->cap_dev();
  *out = p;
  return HS_OK;
}

}  // namespace

extern "C" {

hs_status hs_sparse_attn(hs_handle h, int32_t layer, const void* d_q, int32_t heads, int32_t value_dim,
                         const int32_t* d_slots, float* d_out, float scale, const int32_t* d_num_reqs,
                         void* stream) {
  AttnParams p;
  const hs_status st = attn_params(h, layer, d_q, heads, value_dim, d_slots, d_out, scale, d_num_reqs, &p);
  if (st) return st;
  HS_HIP(launch_attn(p, (hipStream_t)stream));
  return HS_OK;
}

hs_status hs_sparse_attn_static(hs_handle h, int32_t layer, const void* d_q, int32_t heads, int32_t value_dim,
                                const int32_t* d_slots, float* d_out, float scale, const int32_t* d_num_reqs,
                                void* stream) {
  AttnParams p;
  const hs_status st = attn_params(h, layer, d_q, heads, value_dim, d_slots, d_out, scale, d_num_reqs, &p);
  if (st) return st;
  // the partials go to the file-scope device array (the S chunks of every request)
  if (p.S > 1 && int64_t(p.R) * p.S > kStaticAttnPartials)  // (one chunk: the output is written directly)
    return fail(HS_EINVAL, "hs_sparse_attn_static: %d requests x %d chunks need %lld partial records, the "
                "static scratch holds %d", p.R, p.S, (long long)p.R * p.S, kStaticAttnPartials);
  int dev = -1;
  HS_HIP(hipGetDevice(&dev));
  if (dev != h->device) return fail(HS_ESTATE, "hs_sparse_attn_static: device %d is current, the handle's is %d", dev,
                                    h->device);
  p.part = attn_scratch(h->device);
  if (!p.part) return fail(HS_ESTATE, "hs_sparse_attn_static: no scratch address for device %d", h->device);
  HS_HIP(launch_attn(p, (hipStream_t)stream));
  return HS_OK;
}

hs_status hs_export_state(hs_handle h, int32_t layer, int32_t* d_slot_pos, int32_t* d_lru, int32_t* d_page_table,
                          int32_t* d_newest, void* stream) {
  hs_status st;
  if ((st = check_handle(h)) || (st = check_layer(h, layer))) return st;
  if (!h->is_anchor(layer)) return fail(HS_ESTATE, "layer %d has no metadata of its own", layer);
  const int a = layer / h->cfg.layer_group;
  ExportParams p{};
  p.ctrl = h->ctrl(a); p.slot_pos = h->slot_pos(a); p.lru = h->lru(a);
  p.newest = (h->cfg.flags & HS_CFG_NEWEST_SLOT) ? h->newest() : nullptr;
  p.page_table = h->page_table(a); p.max_positions = h->cfg.max_positions;
  p.out_slot_pos = d_slot_pos; p.out_lru = d_lru; p.out_page_table = d_page_table; p.out_newest = d_newest;
  p.R = h->cfg.num_requests; p.B = h->cfg.buffer_slots; p.Bpad = h->lay.Bpad;
  HS_HIP(launch_export(p, (hipStream_t)stream));
  return HS_OK;
}

const uint64_t* hs_page_table(hs_handle h, int32_t layer) {
  if (!h || layer < 0 || layer >= h->cfg.num_layers || !h->is_anchor(layer)) return nullptr;
  return h->page_table(layer / h->cfg.layer_group);
}

hs_status hs_plan(hs_handle h, int32_t layer, const int32_t** d_plan, const uint32_t** d_counts) {
  hs_status st;
  if ((st = check_handle(h)) || (st = check_layer(h, layer))) return st;
  if (!h->is_anchor(layer)) return fail(HS_ESTATE, "layer %d has no plan of its own", layer);
  const int a = layer / h->cfg.layer_group;
  if (d_plan) *d_plan = h->plan(a);
  if (d_counts) *d_counts = h->ctrl(a) + 2;
  return HS_OK;
}

hs_status hs_admit_short(hs_handle h, int32_t request, int32_t ctx_len, void* stream) {
  hs_status st;
  if ((st = check_handle(h))) return st;
  if (request < 0 || request >= h->cfg.num_requests) return fail(HS_EINVAL, "request out of range");
  if (ctx_len < 0 || ctx_len > h->cfg.buffer_slots || ctx_len > h->cfg.max_positions)
    return fail(HS_EINVAL, "a short request holds at most buffer_slots (and max_positions) tokens");
  if (h->on_demand && ctx_len > h->cap_host[request])
    return fail(HS_EINVAL, "request %d has %d backed slots: hs_grow_request before admitting %d tokens", request,
                h->cap_host[request], ctx_len);
  AdmitParams p{};
  p.host_base = h->host_base(); p.hot = h->hot; p.ctrl = h->ctrl(0); p.slot_pos = h->slot_pos(0);
  p.page_table = h->page_table(0); p.max_positions = h->cfg.max_positions; p.hot_req_stride = h->hot_req_stride();
  p.R = h->cfg.num_requests; p.L = h->cfg.num_layers; p.B = h->cfg.buffer_slots; p.A = h->lay.A;
  p.rec_bytes = h->cfg.record_bytes; p.request = request; p.ctx = ctx_len;
  HS_HIP(launch_admit(p, (hipStream_t)stream));
  return HS_OK;
}

hs_status hs_reset_request(hs_handle h, int32_t request, void* stream) {
  hs_status st;
  if ((st = check_handle(h))) return st;
  if (request < 0 || request >= h->cfg.num_requests) return fail(HS_EINVAL, "request out of range");
  InitParams ip{};
  ip.ctrl = h->ctrl(0); ip.slot_pos = h->slot_pos(0); ip.lru = h->lru(0); ip.page_table = h->page_table(0);
  ip.newest = h->newest(); ip.max_positions = h->cfg.max_positions; ip.R = h->cfg.num_requests;
  ip.B = h->cfg.buffer_slots; ip.Bpad = h->lay.Bpad; ip.A = h->lay.A; ip.request = request;
  HS_HIP(launch_init(ip, (hipStream_t)stream));
  return HS_OK;
}

hs_status hs_destroy(hs_handle h) {
  if (!h) return HS_OK;
  // the library's own work (write-through into the pool, replays) must end before the pool goes
  hipError_t e = hipEventSynchronize(h->ev_backup_done);
  for (size_t a = 0; e == hipSuccess && a < h->ev_plan_free.size(); ++a)
    e = hipEventSynchronize(h->ev_plan_free[a]);
  free_ctx(h);
  if (e != hipSuccess) return hip_fail(e, "hs_destroy: waiting for library events");
  return HS_OK;
}

const char* hs_last_error(void) { return g_last_error.c_str(); }

hs_status hs_probe_host_read(const void* host_src, size_t bytes, void* d_sink, int32_t wgs, void* stream) {
  if (!host_src || !d_sink || wgs < 1 || bytes % 16) return fail(HS_EINVAL, "bad probe arguments");
  HS_HIP(launch_probe_host_read(host_src, bytes, d_sink, wgs, (hipStream_t)stream));
  return HS_OK;
}

hs_status hs_probe_copy(const void* d_src, void* d_dst, size_t bytes, void* stream) {
  if (!d_src || !d_dst || bytes % 16) return fail(HS_EINVAL, "bad probe arguments");
  HS_HIP(launch_probe_copy(d_src, d_dst, bytes, (hipStream_t)stream));
  return HS_OK;
}

hs_status hs_probe_host_records(const void* host_src, int64_t src_records, int32_t rec_bytes,
                                const int32_t* d_index, int32_t n, void* d_dst, int32_t wgs, void* stream) {
  if (!host_src || !d_index || !d_dst || wgs < 1 || n < 0 || src_records < 0 || rec_bytes < 16 ||
      rec_bytes % 16 || rec_bytes > 16384 || (int64_t)n * (rec_bytes / 16) > (1ll << 30))
    return fail(HS_EINVAL, "bad probe arguments");
  if (n == 0) return HS_OK;
  HS_HIP(launch_probe_host_records(host_src, d_index, n, rec_bytes, src_records, d_dst, wgs, (hipStream_t)stream));
  return HS_OK;
}

hs_status hs_timing_start(hs_handle h, int32_t n) {
  hs_status st;
  if ((st = check_handle(h))) return st;
  if (n < 0 || n > (1 << 20)) return fail(HS_EINVAL, "n must be in [0, 2^20]");
  free_timing(h);
  h->tm.resize(n);
  for (auto& t : h->tm) {
    hipError_t e = hipEventCreate(&t.start);
    if (e == hipSuccess) e = hipEventCreate(&t.stop);
    if (e != hipSuccess) {
      free_timing(h);
      return hip_fail(e, "hipEventCreate");
    }
  }
  return HS_OK;
}

int32_t hs_timing_read(hs_handle h, float* us_out, int32_t n) {
  if (!h || !us_out || n < 0) return fail(HS_EINVAL, "bad timing read arguments");
  const size_t m = h->tm_next < size_t(n) ? h->tm_next : size_t(n);
  for (size_t i = 0; i < m; ++i) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(h->tm[i].stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, h->tm[i].start, h->tm[i].stop);
    if (e != hipSuccess) return hip_fail(e, "hs_timing_read");
    us_out[i] = ms * 1e3f;
  }
  return (int32_t)m;
}

hs_status hs_probe_empty(int32_t n, void* stream) {
  if (n < 0 || n > (1 << 20)) return fail(HS_EINVAL, "n must be in [0, 2^20]");
  HS_HIP(launch_probe_empty(n, (hipStream_t)stream));
  return HS_OK;
}

}  // extern "C"
