/*
 * CPU oracle of the per-(request, layer) hierarchical KV cache.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load, call or link this file; the
 * product path never does.  It shares no code, header or table with the HIP
 * library.
 *
 * It is a plain, slow model written from the pages:
 *   - "HiSparse 深度解析：论文、SGLang 实现与 vLLM Hybrid HiSparse"
 *     (gentlecold.top): §3.2 (host pool is authoritative; each request and
 *     layer owns B device slots, a page table position -> slot or host-only,
 *     and LRU metadata), §3.3 (per-cache LRU in which this step's hits rank
 *     newer than this step's freshly fetched misses), §3.4 (the newest token
 *     lives in a reserved slot and is written through to host), §3.5 (the
 *     RESOLVE steps and the B=8, k=4 worked example), §5.2 (reserved slot at
 *     index B, outside the LRU), §5.3 (a newly admitted long request starts
 *     with every slot empty), §5.5 (miss plan recorded where eviction is
 *     decided; block ids expanded into token positions).
 *   - "推理系统基础设施手记（六）：HiSparse" (naphjohn.github.io) §2 and
 *     Fig. 3 (host pool laid out by (request, layer, position); B >= k).
 *   - "HiSparse：稀疏注意力的分层 KV Cache 管理" (notes.kuangjux.top) §5
 *     (the {1,4,8},{1,5,8},{1,4,8} example).
 *
 * Replacement rule (the pages leave tie-breaks open; this is the reading
 * used throughout): every slot carries a stamp, 0 when never used.  At
 * step t (1-based) the misses, in selection-list order, take the evictable
 * slots (empty, or holding a position not selected this step) in ascending
 * (stamp, slot index) order; each filled slot gets stamp 2t-1; every slot
 * hit this step gets stamp 2t.  The LRU order is the slots sorted by
 * (stamp, slot index).
 *
 * Parity pins: the worked examples of both pages, k=1 against the
 * Mattson stack-distance test, closed forms for B=k and for B >= the
 * number of distinct positions, per-step invariants, and exhaustive
 * comparison with an independently written Python model (oracle/brute.py).
 */
#define _GNU_SOURCE
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { HSO_ERR_DUP = 1, HSO_ERR_RANGE = 2, HSO_ERR_CAPACITY = 4, HSO_ERR_RESIDENT = 8 };

typedef struct {
  int32_t B;
  int32_t rec_bytes;
  int64_t max_positions;
  int32_t newest_slot; /* 1: slot index B holds the newest token (outside the LRU) */
  int32_t short_mode;  /* 1: admitted short: position p sits in slot p while the context fits B */
  int64_t step;        /* resolves completed */
  int64_t newest_pos;  /* -1: no newest token yet */
  int32_t* slot_pos;   /* [B]: position held by the slot, -1 when empty */
  int64_t* stamp;      /* [B]: recency stamp */
  int32_t* page_table; /* [max_positions]: slot holding the position, -1 = host only */
  uint8_t* hot;        /* [(B+1) * rec_bytes]: contents of the device slots */
  uint8_t* selected;   /* [max_positions]: scratch membership flags of the current selection */
  int32_t* scratch;    /* [3 * B + 2]: miss list, evictable list, hit list */
} hso_cache;

void hso_destroy(hso_cache* c) {
  if (!c) return;
  free(c->slot_pos); free(c->stamp); free(c->page_table); free(c->hot); free(c->selected);
  free(c->scratch); free(c);
}

hso_cache* hso_create(int32_t B, int64_t max_positions, int32_t rec_bytes, int32_t newest_slot) {
  if (B <= 0 || max_positions <= 0 || rec_bytes <= 0) return NULL;
  hso_cache* c = (hso_cache*)calloc(1, sizeof(hso_cache));
  if (!c) return NULL;
  c->B = B; c->rec_bytes = rec_bytes; c->max_positions = max_positions;
  c->newest_slot = newest_slot ? 1 : 0; c->step = 0; c->newest_pos = -1;
  c->slot_pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  c->stamp = (int64_t*)calloc((size_t)B, sizeof(int64_t));
  c->page_table = (int32_t*)malloc(sizeof(int32_t) * (size_t)max_positions);
  c->hot = (uint8_t*)calloc((size_t)(B + 1), (size_t)rec_bytes);
  c->selected = (uint8_t*)calloc((size_t)max_positions, 1);
  c->scratch = (int32_t*)malloc(sizeof(int32_t) * (size_t)(3 * B + 2));
  if (!c->slot_pos || !c->stamp || !c->page_table || !c->hot || !c->selected || !c->scratch) {
    hso_destroy(c);
    return NULL;
  }
  for (int32_t s = 0; s < B; ++s) c->slot_pos[s] = -1;                  /* all slots empty */
  for (int64_t p = 0; p < max_positions; ++p) c->page_table[p] = -1;     /* all host only */
  return c;
}

/* (stamp, slot) ascending: the order in which evictable slots are given away. */
static int by_stamp_then_slot(const void* a, const void* b, void* arg) {
  const int64_t* stamp = (const int64_t*)arg;
  int32_t sa = *(const int32_t*)a, sb = *(const int32_t*)b;
  if (stamp[sa] != stamp[sb]) return stamp[sa] < stamp[sb] ? -1 : 1;
  return sa < sb ? -1 : (sa > sb ? 1 : 0);
}

static void sort_evictable(int32_t* ev, int32_t n, const int64_t* stamp) {
  qsort_r(ev, (size_t)n, sizeof(int32_t), by_stamp_then_slot, (void*)stamp);
}

/*
 * Short-sequence fast path ("HiSparse 深度解析" (gentlecold.top) §5.4 and §5.5):
 * while a request admitted short has at most B tokens, every token sits in the
 * slot of its position, so a selection resolves to its own positions with no
 * host IO and no change to the LRU (the pages' kernel returns at once; it does
 * not check for duplicates).  Returns 1 when it applied (0 or an error in *err).
 */
static int short_fast(hso_cache* c, const int32_t* sel, int32_t k, int64_t ctx_len, int32_t* out,
                      int32_t* counts, int32_t* err) {
  if (!c->short_mode || ctx_len > c->B) return 0;
  *err = 0;
  for (int32_t i = 0; i < k; ++i)
    if (sel[i] < 0 || sel[i] >= ctx_len) *err |= HSO_ERR_RANGE;
  if (*err) return 1;
  for (int32_t i = 0; i < k; ++i) out[i] = sel[i];
  counts[0] = k;
  counts[1] = 0;
  return 1;
}

/*
 * Admission of a short request (gentlecold.top §5.3, §5.4): its first ctx_len
 * <= B tokens are staged into slots 0 .. ctx_len-1 in order (from host), the
 * slot map and page table record them (stamps stay 0: never used), and the
 * cache enters short mode.  Needs the admission state (every slot empty).
 */
int32_t hso_admit_short(hso_cache* c, int64_t ctx_len, const uint8_t* host) {
  if (ctx_len < 0 || ctx_len > c->B || ctx_len > c->max_positions) return HSO_ERR_RANGE;
  for (int32_t s = 0; s < c->B; ++s)
    if (c->slot_pos[s] >= 0) return HSO_ERR_CAPACITY;
  const size_t rec = (size_t)c->rec_bytes;
  for (int64_t p = 0; p < ctx_len; ++p) {
    c->slot_pos[p] = (int32_t)p;
    c->page_table[p] = (int32_t)p;
    memcpy(c->hot + (size_t)p * rec, host + (size_t)p * rec, rec);
  }
  c->short_mode = 1;
  return 0;
}

/*
 * One RESOLVE of k selected positions (already expanded from blocks).
 *   host     : [max_positions][rec_bytes] records of this (request, layer)
 *   out      : [k] physical slot per selected entry, aligned with sel
 *              (B for the newest token)
 *   plan_pos, plan_slot : [k] the misses in list order and the slot each got
 *   counts   : [2] hits, misses
 * Returns 0, or an OR of HSO_ERR_* bits; on error nothing changes.
 */
int32_t hso_resolve(hso_cache* c, const int32_t* sel, int32_t k, int64_t ctx_len,
                    const uint8_t* host, int32_t* out, int32_t* plan_pos, int32_t* plan_slot,
                    int32_t* counts) {
  const int32_t B = c->B;
  const size_t rec = (size_t)c->rec_bytes;
  int32_t err = 0;
  if (short_fast(c, sel, k, ctx_len, out, counts, &err)) return err;

  /* 1. validate: every position in the context, no position twice */
  for (int32_t i = 0; i < k; ++i) {
    int64_t p = sel[i];
    if (p < 0 || p >= ctx_len || p >= c->max_positions) { err |= HSO_ERR_RANGE; continue; }
    if (c->selected[p]) err |= HSO_ERR_DUP;
    c->selected[p] = 1;
  }
  int32_t newest_selected =
      c->newest_slot && c->newest_pos >= 0 && c->newest_pos < c->max_positions &&
      c->selected[c->newest_pos];
  if (!err && k - newest_selected > B) err |= HSO_ERR_CAPACITY;
  if (err) {
    for (int32_t i = 0; i < k; ++i)
      if (sel[i] >= 0 && sel[i] < c->max_positions) c->selected[sel[i]] = 0;
    return err;
  }

  int32_t* misses = c->scratch;            /* list indices of misses, in list order */
  int32_t* evictable = c->scratch + B + 1; /* slots that may be given away */
  int32_t* hit_slots = c->scratch + 2 * B + 2;
  int32_t n_miss = 0, n_hit = 0, n_lru_hit = 0;

  /* 2. classify each entry in list order: newest slot, resident slot, or miss */
  for (int32_t i = 0; i < k; ++i) {
    int32_t p = sel[i];
    if (c->newest_slot && p == c->newest_pos) {
      out[i] = B;
      ++n_hit;
    } else if (c->page_table[p] >= 0) {
      out[i] = c->page_table[p];
      hit_slots[n_lru_hit++] = out[i];
      ++n_hit;
    } else {
      misses[n_miss++] = i;
    }
  }

  /* 3. evictable slots (empty or not selected now), oldest stamp first, ties by slot */
  int32_t n_ev = 0;
  for (int32_t s = 0; s < B; ++s) {
    const int32_t p = c->slot_pos[s];
    /* the newest token is served from slot B, so an LRU slot that happens to
     * hold the same position is not selected through the LRU */
    const int32_t is_newest = c->newest_slot && c->newest_pos >= 0 && p == c->newest_pos;
    if (p < 0 || !c->selected[p] || is_newest) evictable[n_ev++] = s;
  }
  sort_evictable(evictable, n_ev, c->stamp);

  /* 4. the j-th miss takes the j-th evictable slot and its record is copied in */
  c->step += 1;
  const int64_t t = c->step;
  for (int32_t j = 0; j < n_miss; ++j) {
    int32_t i = misses[j];
    int32_t p = sel[i];
    int32_t v = evictable[j];
    if (c->slot_pos[v] >= 0) c->page_table[c->slot_pos[v]] = -1; /* old position: host only */
    c->slot_pos[v] = p;
    c->page_table[p] = v;
    c->stamp[v] = 2 * t - 1;
    out[i] = v;
    memcpy(c->hot + (size_t)v * rec, host + (size_t)p * rec, rec);
    if (plan_pos) plan_pos[j] = p;
    if (plan_slot) plan_slot[j] = v;
  }

  /* 5. hits of this step rank newer than the misses of this step */
  for (int32_t h = 0; h < n_lru_hit; ++h) c->stamp[hit_slots[h]] = 2 * t;

  for (int32_t i = 0; i < k; ++i) c->selected[sel[i]] = 0;
  counts[0] = n_hit;
  counts[1] = n_miss;
  return 0;
}

/*
 * RESOLVE with a resident tier in front ("HiSparse 深度解析" (gentlecold.top)
 * §6.5; "HiSparse local KV offload architecture" (docs.vllm.ai), "Hot lookup
 * and LRU" and "Performance invariants"): each selected position is looked up
 * first in the resident block table, then in the hot slots, and only then
 * fetched from host.
 *   rtable     : [n_pages] resident page of each logical page, -1 when the page
 *                is not resident; the page of position p is p >> page_shift
 *   res_rows   : rows of the resident pool; p's row is
 *                rtable[page] * 2^page_shift + (p mod 2^page_shift)
 *   out        : B + 1 + row for a resident entry, else as hso_resolve
 *   counts     : [3] hot hits (newest slot included), misses, resident entries
 * Reading of the pages: when every entry is resident the call returns right
 * after the lookup (no duplicate check, nothing of the cache changes).
 * Otherwise duplicates are checked over the whole list and the entries that
 * are not resident go, in list order, through hso_resolve's steps; a slot
 * holding a position served by the resident tier is not selected through the
 * LRU, so it may be evicted.  Returns 0 or HSO_ERR_* bits; on error nothing
 * changes.
 */
int32_t hso_resolve_tiered(hso_cache* c, const int32_t* sel, int32_t k, int64_t ctx_len,
                           const int32_t* rtable, int64_t n_pages, int32_t page_shift, int64_t res_rows,
                           const uint8_t* host, int32_t* out, int32_t* plan_pos, int32_t* plan_slot,
                           int32_t* counts) {
  const int32_t B = c->B;
  int32_t err = 0, n_res = 0;
  {
    int32_t c2[2];
    if (short_fast(c, sel, k, ctx_len, out, c2, &err)) {
      if (!err) { counts[0] = c2[0]; counts[1] = 0; counts[2] = 0; }
      return err;
    }
  }
  int32_t* rest = (int32_t*)calloc((size_t)(k > 0 ? k : 1), sizeof(int32_t));   /* non-resident list */
  int32_t* where = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));  /* its list indices */
  int32_t* rout = (int32_t*)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
  if (!rest || !where || !rout) { free(rest); free(where); free(rout); return HSO_ERR_CAPACITY; }

  /* 1. resident level */
  int32_t n_rest = 0;
  for (int32_t i = 0; i < k; ++i) {
    const int64_t p = sel[i];
    if (p < 0 || p >= ctx_len || p >= c->max_positions) { err |= HSO_ERR_RANGE; continue; }
    const int64_t page = p >> page_shift;
    const int32_t rp = page < n_pages ? rtable[page] : -1;
    if (rp >= 0) {
      const int64_t row = ((int64_t)rp << page_shift) + (p & (((int64_t)1 << page_shift) - 1));
      if (row >= res_rows) { err |= HSO_ERR_RESIDENT; continue; }
      out[i] = (int32_t)(B + 1 + row);
      ++n_res;
    } else {
      where[n_rest] = i;
      rest[n_rest++] = (int32_t)p;
    }
  }
  if (!err && n_res == k) {  /* everything resident: return at once */
    counts[0] = 0; counts[1] = 0; counts[2] = n_res;
    free(rest); free(where); free(rout);
    return 0;
  }
  /* 2. no position twice in the whole list */
  for (int32_t i = 0; i < k; ++i) {
    const int64_t p = sel[i];
    if (p < 0 || p >= ctx_len || p >= c->max_positions) continue;
    if (c->selected[p]) err |= HSO_ERR_DUP;
    c->selected[p] = 1;
  }
  for (int32_t i = 0; i < k; ++i)
    if (sel[i] >= 0 && sel[i] < c->max_positions) c->selected[sel[i]] = 0;
  /* 3. the rest through the hot slots and the host */
  int32_t c2[2] = {0, 0};
  if (!err) err = hso_resolve(c, rest, n_rest, ctx_len, host, rout, plan_pos, plan_slot, c2);
  if (!err) {
    for (int32_t j = 0; j < n_rest; ++j) out[where[j]] = rout[j];
    counts[0] = c2[0]; counts[1] = c2[1]; counts[2] = n_res;
  }
  free(rest); free(where); free(rout);
  return err;
}

/*
 * RESOLVE of several verification rows of one speculative decode step
 * ("HiSparse 深度解析" (gentlecold.top) §6.5 comparison table; "HiSparse local
 * KV offload architecture" (docs.vllm.ai), speculative decoding): one call
 * resolves the union of the rows' selections, in first-reference order
 * (row by row, then list order), so rows that select the same position share
 * its slot and no row's miss evicts a slot another row reads.
 *   sel      : [Q][k] positions, distinct within each row
 *   out      : [Q][k] slot of each entry (rows sharing a position share it)
 *   plan_pos, plan_slot : [Q*k] misses of the union in first-reference order
 *   counts   : [4] hits, misses, resident entries (of the union), union size
 *   rtable   : resident block table (NULL: no resident tier), as hso_resolve_tiered
 * Returns 0 or HSO_ERR_* bits (a duplicate within a row is HSO_ERR_DUP); on
 * error nothing changes.
 */
int32_t hso_resolve_rows(hso_cache* c, const int32_t* sel, int32_t Q, int32_t k, int64_t ctx_len,
                         const int32_t* rtable, int64_t n_pages, int32_t page_shift, int64_t res_rows,
                         const uint8_t* host, int32_t* out, int32_t* plan_pos, int32_t* plan_slot,
                         int32_t* counts) {
  const int64_t n = (int64_t)Q * k;
  int32_t err = 0;
  int32_t* uni = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));   /* the union */
  int32_t* uidx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));  /* entry -> union index */
  int32_t* uout = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int32_t* where = (int32_t*)malloc(sizeof(int32_t) * (size_t)c->max_positions);   /* position -> union index */
  if (!uni || !uidx || !uout || !where) {
    free(uni); free(uidx); free(uout); free(where);
    return HSO_ERR_CAPACITY;
  }
  /* 1. every position in the context, none twice within a row */
  for (int32_t q = 0; q < Q; ++q) {
    for (int32_t i = 0; i < k; ++i) {
      const int64_t p = sel[(int64_t)q * k + i];
      if (p < 0 || p >= ctx_len || p >= c->max_positions) { err |= HSO_ERR_RANGE; continue; }
      if (c->selected[p]) err |= HSO_ERR_DUP;
      c->selected[p] = 1;
    }
    for (int32_t i = 0; i < k; ++i) {
      const int64_t p = sel[(int64_t)q * k + i];
      if (p >= 0 && p < c->max_positions) c->selected[p] = 0;
    }
  }
  int32_t nu = 0;
  if (!err) {
    /* 2. the union in first-reference order */
    for (int64_t p = 0; p < c->max_positions; ++p) where[p] = -1;
    for (int64_t f = 0; f < n; ++f) {
      const int32_t p = sel[f];
      if (where[p] < 0) { where[p] = nu; uni[nu++] = p; }
      uidx[f] = where[p];
    }
    /* 3. one resolve of the union */
    if (rtable) {
      int32_t c3[3] = {0, 0, 0};
      err = hso_resolve_tiered(c, uni, nu, ctx_len, rtable, n_pages, page_shift, res_rows, host, uout,
                               plan_pos, plan_slot, c3);
      if (!err) { counts[0] = c3[0]; counts[1] = c3[1]; counts[2] = c3[2]; }
    } else {
      int32_t c2[2] = {0, 0};
      err = hso_resolve(c, uni, nu, ctx_len, host, uout, plan_pos, plan_slot, c2);
      if (!err) { counts[0] = c2[0]; counts[1] = c2[1]; counts[2] = 0; }
    }
    if (!err) {
      for (int64_t f = 0; f < n; ++f) out[f] = uout[uidx[f]];
      counts[3] = nu;
    }
  }
  free(uni); free(uidx); free(uout); free(where);
  return err;
}

/* The new token at `pos`: its record goes to the reserved slot B and is
 * written through to the host pool; it becomes the newest position. */
int32_t hso_append(hso_cache* c, int64_t pos, const uint8_t* record, uint8_t* host) {
  if (!c->newest_slot || pos < 0 || pos >= c->max_positions) return HSO_ERR_RANGE;
  memcpy(c->hot + (size_t)c->B * (size_t)c->rec_bytes, record, (size_t)c->rec_bytes);
  if (c->short_mode && pos < c->B) {  /* a short request keeps its tokens in order */
    memcpy(c->hot + (size_t)pos * (size_t)c->rec_bytes, record, (size_t)c->rec_bytes);
    c->slot_pos[pos] = (int32_t)pos;
    c->page_table[pos] = (int32_t)pos;
  }
  if (host) memcpy(host + (size_t)pos * (size_t)c->rec_bytes, record, (size_t)c->rec_bytes);
  c->newest_pos = pos;
  return 0;
}

/* A shared layer follows its anchor: the anchor's plan, applied to this
 * layer's own records (gentlecold.top §3.6, §5.5). */
void hso_replay(const int32_t* plan_pos, const int32_t* plan_slot, int32_t n,
                const uint8_t* host, uint8_t* hot, int32_t rec_bytes) {
  for (int32_t j = 0; j < n; ++j)
    memcpy(hot + (size_t)plan_slot[j] * (size_t)rec_bytes,
           host + (size_t)plan_pos[j] * (size_t)rec_bytes, (size_t)rec_bytes);
}

/* A block id b stands for tokens b*bt .. b*bt+bt-1; blocks keep their list
 * order and tokens ascend within a block (gentlecold.top §5.5). */
void hso_expand_blocks(const int32_t* blocks, int32_t nb, int32_t bt, int32_t* positions) {
  for (int32_t i = 0; i < nb; ++i)
    for (int32_t o = 0; o < bt; ++o) positions[(int64_t)i * bt + o] = blocks[i] * bt + o;
}

/* State views for checks.  lru receives the slots in (stamp, slot) order. */
void hso_export(const hso_cache* c, int32_t* slot_pos, int64_t* stamp, int32_t* lru) {
  if (slot_pos) memcpy(slot_pos, c->slot_pos, sizeof(int32_t) * (size_t)c->B);
  if (stamp) memcpy(stamp, c->stamp, sizeof(int64_t) * (size_t)c->B);
  if (lru) {
    for (int32_t s = 0; s < c->B; ++s) lru[s] = s;
    sort_evictable(lru, c->B, c->stamp);
  }
}

const int32_t* hso_page_table(const hso_cache* c) { return c->page_table; }
uint8_t* hso_hot(hso_cache* c) { return c->hot; }
int64_t hso_newest(const hso_cache* c) { return c->newest_pos; }
int64_t hso_step(const hso_cache* c) { return c->step; }
