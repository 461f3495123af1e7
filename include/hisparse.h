/*
 * hisparse.h -- C ABI of the hierarchical KV cache for top-k sparse-attention
 * decode on AMD Instinct MI355X (gfx950).
 *
 * What it computes is defined on these pages:
 *   [GC]  "HiSparse 深度解析：论文、SGLang 实现与 vLLM Hybrid HiSparse"
 *         (gentlecold.top)
 *   [VD]  "HiSparse local KV offload architecture" (docs.vllm.ai)
 *   [NJ]  "推理系统基础设施手记（六）：HiSparse" (naphjohn.github.io)
 *   [KJ]  "HiSparse：稀疏注意力的分层 KV Cache 管理" (notes.kuangjux.top)
 *
 * Model ([GC] §3.2, [NJ] §2 and Fig. 3): the full KV history of every
 * (request, layer) lives in pinned host memory and is authoritative.  Each
 * (request, layer) also owns B device slots in HBM (B >= k), a page table
 * position -> slot (or host only) and an LRU order of its slots.  One call per
 * layer (RESOLVE, [GC] §3.5) turns the k selected logical positions into the
 * k physical slots, fetching the records that miss straight from host memory.
 *
 * Conventions
 *   - "device" pointers point to GPU memory (HBM); "host" pointers to host
 *     memory.  Streams are hipStream_t passed as void*; NULL is the null stream.
 *   - Every call that takes a stream is asynchronous on it and performs no
 *     device-to-host readback.  Argument and state errors are detected on the
 *     host and returned synchronously (nothing is enqueued then).  Data errors
 *     (bad positions) are detected on the device and reported in
 *     hs_stats.error; they are never read back by the library.
 *   - The caller owns the hot buffer, the workspace and all streams; the
 *     library owns the pinned host pool and its events.
 *   - Positions and slot indices are int32.  top_k <= B <= 16384 (top_k <= 8192 in
 *     practice: see hs_create), max_positions < 2^31, record_bytes a multiple of 16.
 *   - A handle may be used from one host thread at a time.
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hs_ctx* hs_handle;
typedef int32_t hs_status;

#define HS_OK 0
#define HS_EINVAL (-1) /* bad argument or configuration */
#define HS_ENOMEM (-2) /* pinned host allocation failed */
#define HS_EHIP (-3)   /* a HIP runtime call failed; see hs_last_error() */
#define HS_ESTATE (-4) /* call not valid for this handle or layer */

/* hs_config.flags */
#define HS_CFG_NEWEST_SLOT 1u /* slot B of every (request, layer) holds the newest token ([GC] §3.4, §5.2) */
#define HS_CFG_HOT_ON_DEMAND 4u /* the library reserves the hot buffer's address range and backs it with
                                   device memory as requests grow (hs_grow_request; [GC] §5.4
                                   _grow_device_buffers): hs_create takes d_hot = NULL */
#define HS_CFG_RECORD_FP8 2u  /* records are fp8 latent KV ([GC] §5.5: fp8_e4m3 KV, FlashMLA-style layout):
                                 record_bytes = 656 = 512 OCP E4M3 codes in 4 blocks of 128, a float32
                                 scale per block, then 64 bf16 values; only hs_sparse_attn reads the
                                 layout (RESOLVE moves records as opaque bytes) */

/* hs_resolve flags ([GC] §5.5: compile-time switches of the pages' kernel) */
#define HS_RECORD_PLAN 1u /* anchor layer: record the miss plan for its shared layers ([GC] §3.6, §5.5) */
#define HS_SKIP_IO 2u     /* timing aid ([GC] §4.4, §5.6 no-IO oracle): all metadata as usual, no record
                             bytes move, so the hot buffer is stale afterwards */

/* hs_stats.error bits */
#define HS_ERR_DUP 1u   /* a position (or block) selected twice */
#define HS_ERR_RANGE 2u /* a position outside [0, ctx_len) */
#define HS_ERR_STATE 4u /* internal: page table and slot map disagreed (never expected) */
#define HS_ERR_RESIDENT 8u /* a block-table entry names a row outside the bound resident pool */
#define HS_ERR_CAPACITY 16u /* HS_CFG_HOT_ON_DEMAND: the request needs hot slots that are not backed yet
                               (a short request longer than its grown capacity, or the normal path
                               before all B slots are backed); nothing changes */

typedef struct {
  int32_t num_requests;    /* R: requests resolved together in one launch per layer */
  int32_t num_layers;      /* L */
  int64_t max_positions;   /* positions per (request, layer) in the host pool */
  int32_t record_bytes;    /* bytes of one token's KV record (1152 = 576 bf16) */
  int32_t top_k;           /* k: selected tokens per (request, layer, call) */
  int32_t block_tokens;    /* 1: selections are token positions; n > 1 (power of two): block ids of
                              n tokens, expanded in the kernel ([GC] §5.5) */
  int32_t buffer_slots;    /* B: LRU slots per (request, layer), top_k <= B */
  int32_t layer_group;     /* 1: every layer resolves its own selection.  g > 1: layers g*i are
                              anchors and layers g*i+1 .. g*i+g-1 share the anchor's selection and
                              slot layout ([GC] §3.6 IndexCache / IndexShare) */
  int32_t wgs_per_request; /* workgroups per request in hs_resolve; 0 chooses */
  uint32_t flags;          /* HS_CFG_* */
  int32_t verify_rows;     /* 0 or 1: no speculative decoding.  n > 1: hs_resolve_rows accepts up to n
                              verification rows per call ([GC] §6.5, [VD]); needs
                              n * top_k <= 8192 and buffer_slots >= n * top_k */
} hs_config;

/* Per-request result of one hs_resolve call (device memory, overwritten per call; 24 bytes,
 * 8-byte aligned).  The counts are the pages' hit / miss statistics of the resolve ([GC] §3.3,
 * §3.5: every selected position is a hit or a miss; [GC] §6.5 adds the resident level). */
typedef struct {
  uint32_t hits;          /* selected tokens found in the hot slots (newest slot included) */
  uint32_t misses;        /* selected tokens fetched from host (record_bytes each) */
  uint32_t error;         /* HS_ERR_* bits; when set, nothing of this request changed and its
                             slots_out row is -1 */
  uint32_t resident;      /* selected tokens served by the resident tier (hs_bind_resident);
                             hits + misses + resident = top_k */
  uint64_t bytes_fetched; /* record bytes this call copied from the host pool into the hot
                             slots: misses * record_bytes (0 with HS_SKIP_IO, which moves none) */
} hs_stats;

/*
 * Bytes of device workspace hs_create needs for cfg (0 when cfg is invalid; hs_last_error says
 * why).  The workspace holds what the pages keep resident on the GPU beside the hot buffer
 * ([GC] §3.2: the page table and the LRU metadata of every (request, layer); §5.3: admission
 * reserves each request's slots and metadata before it is scheduled): per anchor layer the slot
 * map and LRU order (two halves each), the page table, the miss plan ([GC] §3.6), and the
 * attention partials and staging of the fused call.  Deterministic in cfg; no allocation.
 */
size_t hs_workspace_bytes(const hs_config* cfg);

/*
 * Creates a cache.
 *   d_hot       device, caller-owned, [R][L][B+1][record_bytes]: the hot buffers
 *               ([GC] §3.2; slot B is the reserved newest slot, [GC] §5.2).  NULL with
 *               HS_CFG_HOT_ON_DEMAND: the library reserves that address range and backs it on
 *               demand (hs_grow_request); no request has device slots until it is grown.
 *   d_workspace device, caller-owned, hs_workspace_bytes(cfg) bytes, 256-byte
 *               aligned: metadata (slot map, LRU order, page table, miss plans,
 *               attention partials).  hs_create initialises it synchronously:
 *               every slot empty, every position host-only ([GC] §5.3).
 * Allocates the pinned host pool, one allocation per request of
 * [L][max_positions][record_bytes] ([NJ] §2.1: contiguous by (request, layer,
 * position)).  The caller fills it with the prefill records (hs_host_pool)
 * before the first hs_resolve.  Returns HS_ENOMEM when pinning fails, HS_EINVAL when a
 * workgroup's LDS cannot hold RESOLVE's tables (the selection's hash of >= 2 top_k buckets,
 * its positions and the slot owners): with MI355X's 160 KB per workgroup that is any
 * top_k above 8192, whatever B.
 */
hs_status hs_create(const hs_config* cfg, void* d_hot, void* d_workspace, hs_handle* out);

/* Host address of request r's pool region [L][max_positions][record_bytes]; NULL if r is out of
 * range.  Valid until hs_destroy. */
void* hs_host_pool(hs_handle h, int32_t request);

/* Device address of the hot buffer [R][L][B+1][record_bytes] (the caller's d_hot, or the range
 * the library reserved with HS_CFG_HOT_ON_DEMAND); NULL for a bad handle. */
void* hs_hot_buffer(hs_handle h);

/*
 * On-demand growth of a request's device buffer ([GC] §5.4: the device buffer grows as needed --
 * _grow_device_buffers -- so a short request does not hold all B slots from the start; §5.3:
 * only a request longer than B gets the full B).  With HS_CFG_HOT_ON_DEMAND, backs slots
 * [0, slots) and the newest slot B of every layer of `request` with device memory (64 KiB
 * chunks of the reserved range, mapped now, on the host), then, ordered on `stream`, raises
 * the request's capacity to `slots` for the kernels.  Capacity only grows (hs_reset_request
 * keeps it; hs_destroy releases everything).  The caller grows a short request before its
 * context outgrows the capacity (hs_admit_short needs ctx_len <= capacity; a hs_writeback of
 * a position >= capacity writes only slot B and the host pool), and grows it to B before its
 * context exceeds B; kernels that would need unbacked slots report HS_ERR_CAPACITY instead.
 *   slots  0 .. B (0: the newest slot only)
 * HS_ENOMEM when device memory runs out (chunks mapped so far stay); without
 * HS_CFG_HOT_ON_DEMAND every slot is backed already and the call does nothing.
 */
hs_status hs_grow_request(hs_handle h, int32_t request, int32_t slots, void* stream);

/* Bytes of device memory behind the hot buffer: all of it for a caller-owned buffer, the mapped
 * chunks with HS_CFG_HOT_ON_DEMAND.  (-1 for a bad handle.) */
int64_t hs_hot_backed_bytes(hs_handle h);

/*
 * RESOLVE of one layer for all requests ([GC] §3.5, [NJ] §3, [KJ] §7.1):
 * stage the selected positions in an LDS hash table, mark hit and evictable
 * slots, assign LRU victims to the misses by wavefront scans, fetch the missed
 * records from pinned host memory, publish the physical slots.
 *   layer        an anchor (or, with layer_group 1, any) layer
 *   d_sel        device [R][top_k / block_tokens] int32 positions (or block ids), distinct
 *   d_ctx_len    device [R] int32: positions of request r must be < d_ctx_len[r]
 *   d_slots_out  device [R][top_k] int32: slot of each selected token, in selection order
 *                (B for the newest token); the layer's KV of entry i is
 *                d_hot[r][layer][d_slots_out[r][i]]
 *   d_stats      device [R] hs_stats, or NULL
 *   d_num_reqs   device int32 scalar, or NULL: requests >= *d_num_reqs are left untouched
 *                (padding of a captured batch, [GC] §5.5)
 *   flags        HS_RECORD_PLAN | HS_SKIP_IO
 * Replacement ([GC] §3.3): empty slots first; this call's hits rank newer than
 * this call's fetched entries; victims are the least recent slots not selected
 * now, ties by lower slot index; misses take victims in selection order.
 * With a resident tier bound (hs_bind_resident) each position is looked up
 * there first ([GC] §6.5): a resident entry gets B + 1 + its resident row and
 * takes no part in the LRU (a slot holding that position counts as not
 * selected); a call whose entries are all resident returns before the hash
 * and LRU stages and changes nothing (duplicates are then not reported).
 * With HS_RECORD_PLAN the stream first waits until the previous plan of this
 * anchor has been replayed.
 */
hs_status hs_resolve(hs_handle h, int32_t layer, const int32_t* d_sel, const int32_t* d_ctx_len,
                     int32_t* d_slots_out, hs_stats* d_stats, const int32_t* d_num_reqs,
                     uint32_t flags, void* stream);

/*
 * RESOLVE of the verification rows of one speculative decode step ([GC] §6.5
 * comparison table: one call resolves the union of all verification rows' top-k,
 * rows selecting the same position share its slot, no row evicts a slot another
 * row reads, misses are assigned in (row, entry) first-reference order; [VD]
 * "Speculative decoding").  The union is resolved exactly as hs_resolve resolves
 * one list; hits, misses and resident counts in d_stats are those of the union.
 *   rows         1 .. cfg.verify_rows
 *   d_sel        device [R][rows][top_k / block_tokens] int32, distinct within each row
 *   d_slots_out  device [R][rows][top_k] int32, the slot of every (row, entry)
 *   other arguments as hs_resolve.  A duplicate inside a row sets HS_ERR_DUP (nothing
 *   changes); repeats across rows are the point and are not errors.
 * Kernel launches on `stream`: when verify_rows x top_k > 4096 and the configuration's LDS
 * allows it, one (every workgroup builds the union in its own LDS, resolves it, and writes
 * every row's slots); otherwise the union, then the RESOLVE of the union, which also writes
 * every row's slots (a third launch writes them when verify_rows x top_k <= 4096).  The union
 * scratch is per handle, so calls on one handle must be ordered on one stream.
 */
hs_status hs_resolve_rows(hs_handle h, int32_t layer, int32_t rows, const int32_t* d_sel,
                          const int32_t* d_ctx_len, int32_t* d_slots_out, hs_stats* d_stats,
                          const int32_t* d_num_reqs, uint32_t flags, void* stream);

/*
 * Binds a resident tier in front of the hot slots ([GC] §6.5; [VD] "Hot lookup
 * and LRU", "Performance invariants"): the caller's regular paged KV cache, of
 * which some pages of each request are on the device.
 *   d_block_table     device, caller-owned [R][pages_per_request] int32: the
 *                     resident page of each logical page (page of position p =
 *                     p / page_tokens), -1 when the page is not resident.  The
 *                     caller may rewrite it between calls (stream-ordered).
 *   pages_per_request pages_per_request * page_tokens >= max_positions
 *   page_tokens       tokens per page, a power of two <= 2^20
 *   d_resident_kv     device, caller-owned [L][resident_rows][record_bytes]; the
 *                     record of position p of layer l is row
 *                     table[r][p / page_tokens] * page_tokens + p % page_tokens
 *   resident_rows     rows per layer, 1 .. 2^31 - 2 - B
 * Afterwards hs_resolve consults the table and hs_sparse_attn reads slots
 * above B from d_resident_kv.  d_block_table = NULL unbinds (other arguments
 * ignored).  Takes effect for calls enqueued after it.
 */
hs_status hs_bind_resident(hs_handle h, const int32_t* d_block_table, int32_t pages_per_request,
                           int32_t page_tokens, const void* d_resident_kv, int64_t resident_rows);

/*
 * Write-through of one new token per request, for every layer ([GC] §3.4, §5.4;
 * [KJ] §7.1): the new token's KV goes into the reserved newest slot, so the newest position is
 * always on the device, and a backup copy goes to the host pool, ordered by events so that a
 * later fetch of that position reads complete bytes.  Needs HS_CFG_NEWEST_SLOT.
 *   d_new_kv   device [R][L][record_bytes]: the new token's records
 *   d_new_pos  device [R] int32: its position (< max_positions)
 * Two streams (backup non-null and distinct from compute), the pages' layout:
 * on `compute` waits for the previous write-through to finish reading slot B,
 * copies d_new_kv into slot B of every layer and makes d_new_pos the newest
 * position; on `backup` waits for that copy, then writes slot B to the host
 * pool at d_new_pos.  A later hs_writeback on `compute` waits for this backup,
 * so any later resolve that fetches that position reads the written bytes.
 * One stream (backup null or equal to compute): a single kernel on `compute`
 * does both copies, so the stream orders it with every later call; it first
 * waits for a two-stream write-through that may still be reading slot B.  On
 * MI355X the cross-stream event pair costs about 18 us of GPU time per step,
 * more than writing R x L records to the host, so small appends take this mode.
 */
hs_status hs_writeback(hs_handle h, const void* d_new_kv, const int32_t* d_new_pos, void* compute,
                       void* backup);

/*
 * Exact layer-wise prefetch ([GC] §3.6, §5.6): `prefetch` waits for the
 * anchor's last hs_resolve (which must have used HS_RECORD_PLAN), then for
 * each shared layer of the anchor's group copies that layer's own records of
 * the plan into the same slots, and records the layer's event.  Shared layers
 * reuse the anchor's d_slots_out.
 */
hs_status hs_prefetch_shared(hs_handle h, int32_t anchor_layer, void* compute, void* prefetch);

/*
 * `stream` waits until the prefetch of shared layer `layer` is done ([GC] §5.6: a shared-index
 * layer waits for its own prefetch event, then reuses the anchor's slot table; [GC] §3.6).
 * The wait is on the event that hs_prefetch_shared recorded for this layer, so a shared layer
 * never waits for the replay of a later one.  An anchor layer (or a layer of a group that has
 * not been prefetched) returns HS_OK with nothing enqueued: an anchor's records are in place
 * when its own resolve ends on the caller's stream.  HS_EINVAL for a bad handle or layer.
 */
hs_status hs_wait_layer(hs_handle h, int32_t layer, void* stream);

/*
 * Sparse decode attention over the published slots ([GC] §5.4: attention reads
 * the slots aligned with the top-k order).  For each request: the key of entry
 * i is the first key_dim bf16 of the record in slot d_slots[r][i] of this
 * layer (a slot B + 1 + row is row `row` of this layer's bound resident pool),
 * its value the first value_dim of them; s = scale * q k^T, softmax over the
 * top_k entries, o = p v.
 *   d_q     device [R][heads][key_dim] bf16, heads 1..16, key_dim = 576 (with HS_CFG_RECORD_FP8 the
 *           key is the 512 dequantised values (code * block scale, rounded to bf16) then the 64
 *           bf16 values; otherwise the record's 576 bf16)
 *   d_slots device [R][top_k] int32 (the layer's, or its anchor's, d_slots_out)
 *   d_out   device [R][heads][value_dim] float32, value_dim = 512
 *   d_num_reqs as for hs_resolve (rows of skipped requests are not written)
 * Slots outside [0, B] and outside the bound resident rows make the request's output rows NaN.
 */
hs_status hs_sparse_attn(hs_handle h, int32_t layer, const void* d_q, int32_t heads,
                         int32_t value_dim, const int32_t* d_slots, float* d_out, float scale,
                         const int32_t* d_num_reqs, void* stream);

/*
 * hs_sparse_attn for callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the same arguments, the same
 * kernels and the same output bit for bit, but the per-chunk attention partials go to a
 * file-scope device array of the library (held on each GPU until the process ends) instead of
 * the handle's workspace.  The call allocates nothing.  Limit: num_requests x chunks per
 * request <= 512 partial records (16.8 MB) when a request has more than one chunk (chunks per
 * request: min(ceil(256 / R), ceil(k / 64)), at least ceil(k / 1024)); otherwise HS_EINVAL.
 * HS_ESTATE unless the handle's device is current.  Every call on one GPU shares that array: calls that overlap on one GPU (different
 * streams, not ordered) race; calls ordered on one stream do not (each call's partials are
 * written before its merge reads them, so nothing needs clearing).
 */
hs_status hs_sparse_attn_static(hs_handle h, int32_t layer, const void* d_q, int32_t heads,
                                int32_t value_dim, const int32_t* d_slots, float* d_out, float scale,
                                const int32_t* d_num_reqs, void* stream);

/*
 * RESOLVE of one anchor layer and the sparse attention over its published slots, in one
 * kernel where the configuration allows ([GC] §3.5 for the resolve, §5.4 for the attention
 * that reads the slots aligned with the top-k order).  Results are those of
 *   hs_resolve(h, layer, d_sel, d_ctx_len, d_slots_out, d_stats, d_num_reqs, flags, stream);
 *   hs_sparse_attn(h, layer, d_q, heads, value_dim, d_slots_out, d_out, scale, d_num_reqs, stream);
 * with the same arguments: the same slots, counts, metadata and hot bytes bit for bit, the
 * same attention up to the order of the fp32 sums.  In the fused kernel one workgroup per
 * request resolves, and S more each take a share of <= 64 T selected entries: they load
 * the share's records (hot slot, resident row or, for a miss, the host record) 64 at a time
 * into LDS while the resolve runs, stage the misses, and attend over the tiles with a
 * running maximum and sum.  A second kernel merges the shares of each (request, head),
 * applies the page-table updates and copies the staged misses into their victim slots.  T is
 * the smallest value in [1, 16] with num_requests * (S + 1) <= 256, S = ceil(top_k / 64 T),
 * so that all workgroups run at once.  It applies to bf16 records of 576 values
 * (record_bytes 1152) and to FP8 records (HS_CFG_RECORD_FP8: the codes are turned into bf16
 * in the tile exactly, the block scales applied in fp32, the misses staged as raw records),
 * with top_k <= 4096, buffer_slots <= 8192 and such a T (so at most 128 requests;
 * hs_resolve_attn_wgs > 0); otherwise this call makes the two calls above.
 * HS_SKIP_IO is not allowed (the attention reads the records).  Errors as for the two calls;
 * a request with error bits gets NaN output rows.
 */
hs_status hs_resolve_attn(hs_handle h, int32_t layer, const int32_t* d_sel, const int32_t* d_ctx_len,
                          int32_t* d_slots_out, hs_stats* d_stats, const int32_t* d_num_reqs, uint32_t flags,
                          const void* d_q, int32_t heads, int32_t value_dim, float* d_out, float scale,
                          void* stream);

/*
 * Copies the current metadata of an anchor layer into caller buffers (device), the state the
 * pages keep resident on the GPU ([GC] §3.2: the page table maps each logical position to a
 * slot or to the host-only sentinel; the LRU metadata orders the slots):
 *   d_slot_pos   [R][B] int32 position held by each slot (-1 empty)
 *   d_lru        [R][B] int32 slots from least to most recent
 *   d_page_table [R][max_positions] int32 slot holding each position (-1: host only; the
 *                newest token's slot B is not entered, [GC] §3.4)
 *   d_newest     [R] int32 newest position (-1 none)
 * Any may be NULL.  Asynchronous on `stream`; HS_ESTATE for a shared layer (it has no
 * metadata of its own).
 */
hs_status hs_export_state(hs_handle h, int32_t layer, int32_t* d_slot_pos, int32_t* d_lru,
                          int32_t* d_page_table, int32_t* d_newest, void* stream);

/* Device address of an anchor layer's page table, uint64 [R][max_positions]: the low 32 bits of
 * an entry are the slot holding the position (int32, -1 = host only), the high 32 bits a
 * generation tag the resolve kernel uses to order its own updates (bookkeeping only). */
const uint64_t* hs_page_table(hs_handle h, int32_t layer);

/* Device address of an anchor layer's miss plan: int32 [R][2][P] (positions, then slots, in miss
 * order), P = top_k * max(1, verify_rows), and uint32 counts (stride 4 per request, count first). */
hs_status hs_plan(hs_handle h, int32_t layer, const int32_t** d_plan, const uint32_t** d_counts);

/*
 * Admission of a short request ([GC] §5.3, §5.4 and §5.5: a request whose tokens fit the device
 * buffer keeps them there in order, and the swap-in kernel's fast path returns their slots
 * directly, with no host IO).  Stages positions [0, ctx_len) of every layer of `request` from the
 * host pool into slots [0, ctx_len) in order, records them in every anchor's slot map and page
 * table (never used, so oldest first), and marks the request short:
 *   - while its context length is <= B, hs_resolve / hs_resolve_rows return slot = position for
 *     every entry and change no LRU state (positions are range-checked only);
 *   - hs_writeback also writes a new token at position p < B into slot p (in order);
 *   - once the context exceeds B (with the B slots full of positions 0 .. B-1) the normal path
 *     takes over from that state.
 * The request must be in the admission state (after hs_create or hs_reset_request) and grow
 * only by hs_writeback.  ctx_len <= buffer_slots (with HS_CFG_HOT_ON_DEMAND, <= the capacity
 * hs_grow_request gave the request).  Asynchronous on `stream`.
 */
hs_status hs_admit_short(hs_handle h, int32_t request, int32_t ctx_len, void* stream);

/* Request release ([GC] §5.4): every layer of request r back to the admission state (all
 * slots empty, all positions host-only, LRU in slot order, no newest token, not short). */
hs_status hs_reset_request(hs_handle h, int32_t request, void* stream);

/*
 * Teardown of the cache, after the pages' release order ([GC] §5.4: a finishing request first
 * waits for the pending backup, then its host and device slots are released): waits for the
 * library's own work still in flight (a backup-stream write-through into the host pool, shared-
 * layer replays reading it), then frees the pinned pool, the events and the handle.  The hot
 * buffer and the workspace are the caller's and stay allocated (with HS_CFG_HOT_ON_DEMAND the
 * device first finishes all its work, then the reserved range is unmapped and released).  NULL
 * is a no-op.  On a HIP error while waiting the handle is still freed and HS_EHIP is returned.
 */
hs_status hs_destroy(hs_handle h);

/* Message of the last failing call on this thread ("" if none). */
const char* hs_last_error(void);

/* Workgroups per request hs_resolve launches for this handle. */
int32_t hs_resolve_wgs(hs_handle h);

/* Workgroups per request of the fused kernel of hs_resolve_attn, S + 1 (0: the call makes
 * two). */
int32_t hs_resolve_attn_wgs(hs_handle h);

/* ---- measurement aids (no part of the cache) ---------------------------------------------- */

/* Streams `bytes` of pinned host memory through the GPU with 16-byte non-temporal loads from
 * `wgs` workgroups (a zero-copy link probe).  d_sink: device, >= 16 KiB. */
hs_status hs_probe_host_read(const void* host_src, size_t bytes, void* d_sink, int32_t wgs,
                             void* stream);
/* Gathers the n records d_index[0..n) (device int32, record numbers) of a pinned host array of
 * src_records records of rec_bytes each (a multiple of 16, at most 16384) into the dense device
 * array d_dst [n][rec_bytes], with 16-byte non-temporal loads from `wgs` workgroups: the link
 * rate of scattered record reads.  Indices outside [0, src_records) are skipped (their d_dst
 * rows are left as they were).  HS_EINVAL for null pointers, bad sizes or n * rec_bytes / 16
 * above 2^30. */
hs_status hs_probe_host_records(const void* host_src, int64_t src_records, int32_t rec_bytes,
                                const int32_t* d_index, int32_t n, void* d_dst, int32_t wgs, void* stream);
/* Plain device-to-device copy kernel (16-byte vectors), for counter calibration. */
hs_status hs_probe_copy(const void* d_src, void* d_dst, size_t bytes, void* stream);
/* n empty kernels back to back on one stream, launched from this call (the launch-latency
 * probe, free of the caller's per-call cost).  HS_EINVAL unless 0 <= n <= 2^20. */
hs_status hs_probe_empty(int32_t n, void* stream);

/* Kernel durations of the next n RESOLVE and replay launches of h, in call order
 * (hs_resolve's kernel, the fused kernel of hs_resolve_attn (not its finish kernel), the
 * RESOLVE kernel of hs_resolve_rows (not its union and scatter kernels), and each shared
 * layer's replay kernel of hs_prefetch_shared), stamped by the kernels' own start and
 * end (hipExtLaunchKernel events), so no event between launches adds to them.
 * hs_timing_start creates n event pairs (dropping earlier ones); launches beyond n are not
 * timed. */
hs_status hs_timing_start(hs_handle h, int32_t n);
/* Waits for the timed launches and writes the first min(n, launched) durations in
 * microseconds, in launch order, to host memory us_out; returns that count (< 0: error). */
int32_t hs_timing_read(hs_handle h, float* us_out, int32_t n);

#ifdef __cplusplus
}
#endif
#endif /* HISPARSE_H */
