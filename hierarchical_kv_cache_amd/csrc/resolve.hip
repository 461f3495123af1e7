// RESOLVE: one fused kernel per layer turns the k selected logical positions
// of every request into physical slots of that request's hot buffer.
//
// Stages ("HiSparse 深度解析" (gentlecold.top) §3.5; "推理系统基础设施手记（六）：
// HiSparse" (naphjohn.github.io) §3):
//   1 stage    selected positions classified; misses -> LDS open-addressing hash
//              (Knuth multiplicative hash, linear probing) for duplicate detection
//   2 mark     hit slots marked.  The pages probe every slot's stored position in
//              the hash; here the page table, which the kernel keeps the exact
//              inverse of the slot map, names each hit's slot directly, so the
//              entry claims it in an LDS owner array (same hit set, no B-slot
//              probe loop)
//   3 scan     block-wide ranks (wave64 ballot + mbcnt, one LDS carry step):
//              misses numbered in list order, evictable slots numbered in LRU
//              order, the j-th evictable is the victim of the j-th miss; new LRU
//              order = untouched evictables (old order), then filled victims,
//              then hits (§3.3: hits rank newer than this step's fetches)
//   4 fetch    missed records copied from pinned host memory with 16-byte
//              non-temporal loads, flattened over (miss, 16-byte chunk)
//   5 publish  page table, slot map, slots aligned with the selection order
//
// Resident tier ("HiSparse 深度解析" §6.5; "HiSparse local KV offload
// architecture" (docs.vllm.ai), "Hot lookup and LRU"): when the caller binds a
// block table of resident pages, each selected position is looked up there
// first.  A resident entry publishes B + 1 + its resident row and takes no part
// in the LRU (its hash key is the complemented position, so no slot matches it
// in stage 2, while duplicates are still caught).  When every entry is resident
// the kernel returns right after the lookup: no hash, no LRU, no copy.
//
// MI355X layout of the work.  G workgroups serve one request.  Each of them
// recomputes stages 1-3 from the current metadata (cheap, all in LDS) and
// copies its 1/G share of the missed bytes, so that a single request keeps
// enough loads in flight to fill the host link; only workgroup 0 writes the
// new metadata.  The slot map and the LRU order are ping-ponged: a 64-bit
// counter per request numbers the launches that changed the metadata (each of
// their workgroups adds its share once it has read the metadata); its parity
// names the half holding the current metadata, and workgroup 0 writes the other
// half.  The page table is updated in place, each entry tagged with the
// generation of the launch that wrote it, so a sibling that reads an entry
// after workgroup 0 has written it still classifies the position as the miss
// it was when the launch began.  A launch that changes nothing (an error, or
// everything resident) leaves the counter alone, so its half stays current.
// No workgroup waits on another.
//
// Latency shape (the all-hit call is bounded by launch and memory latency,
// not bandwidth): every global read that depends on no other -- the selection, both
// halves of the slot map and LRU order, the launch counter, the request's scalars -- is
// issued at entry before any branch, then the page-table entries of the selected
// positions, so the kernel pays two memory round trips before its LDS work.  Threads
// own contiguous runs of slots / LRU positions / selection entries, loaded
// as vectors; hash insertion uses plain LDS stores and a read-back instead
// of atomics (which the LDS serialises lane by lane); all probes of a thread
// are in flight together; two two-field rank scans order everything.
#include <hip/hip_ext.h>

#include "hs_internal.h"
#include "hs_attend.h"

namespace hs {
namespace {

constexpr int NT = kResolveThreads;
constexpr int NW = NT / 64;
constexpr int kUnroll = 4;
constexpr int kEarly = 4;  // 16-byte chunks per lane loaded before the victims are known

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t hash_pos(int32_t pos, int bits) {
  return ((uint32_t)pos * 2654435761u) >> (32 - bits);  // Knuth multiplicative hash
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive block-wide ranks for two flag sets at once.  Thread t owns elements
// [t*E, t*E+E) of each set (bit j of a / b = element t*E+j).  Within a wave the
// rank is the number of set bits in lower lanes (one ballot + mbcnt per bit
// position); across waves one carry step through LDS.  `buf` holds 2*NW ints
// and alternates between consecutive calls, so one barrier suffices.
template <int E>
__device__ __forceinline__ void block_ranks2(uint32_t a, uint32_t b, uint32_t* buf, int& ra, int& rb,
                                             int& ta, int& tb) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int wa = 0, wb = 0, la = 0, lb = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint64_t ma = __ballot((a >> j) & 1u);
    const uint64_t mb = __ballot((b >> j) & 1u);
    la += lanes_below(ma);
    lb += lanes_below(mb);
    wa += __popcll(ma);
    wb += __popcll(mb);
  }
  if (lane == 0) {
    buf[wid] = (uint32_t)wa;
    buf[NW + wid] = (uint32_t)wb;
  }
  __syncthreads();
  int ba = 0, bb = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int ca = (int)buf[w], cb = (int)buf[NW + w];
    if (w < wid) { ba += ca; bb += cb; }
    ta += ca;
    tb += cb;
  }
  ra = ba + la;
  rb = bb + lb;
}

// E consecutive int32 elements base .. base+E-1 of src (n valid, `fill` past the end); 16-byte
// vector loads with vec (n % 4 == 0, so every 4-element group of a run lies wholly inside or
// wholly past the end).  E < 8: vector loads for a whole run, element loads otherwise.  E >= 8:
// the buffer sizes that use these layouts leave the last waves' runs partial or empty, and a
// branch that only some threads of a wave take runs both arms, the second one's loads waiting
// for the first one's (they write the same registers), which waits for every earlier load of
// the wave; so with vec every thread takes the vector loads, a group past the end reads the
// last group instead, and the caller ignores elements past the end.  (At E = 4 the per-thread
// test measured faster.)
template <int E>
__device__ __forceinline__ void load_run32(const int32_t* __restrict__ src, int n, int base, bool vec,
                                           int32_t (&out)[E], int32_t fill) {
  if constexpr (E % 4 == 0) {
    if (vec && (E >= 8 || base + E <= n)) {
#pragma unroll
      for (int v = 0; v < E / 4; ++v) {
        const int gb = base + 4 * v;
        const u32x4 x = *(const u32x4*)(src + (E < 8 || gb + 4 <= n ? gb : n - 4));
        out[4 * v + 0] = (int32_t)x[0];
        out[4 * v + 1] = (int32_t)x[1];
        out[4 * v + 2] = (int32_t)x[2];
        out[4 * v + 3] = (int32_t)x[3];
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < E; ++j) out[j] = (base + j < n) ? src[base + j] : fill;
}

// The same for int16 elements (8 per 16-byte load, 4 per 8-byte load), kept as the packed
// 32-bit words they arrive in (element j in half j & 1 of word j / 2) and unpacked where they
// are used (run16_at), so nothing waits for the loads here.  nalloc (a multiple of 8, >= n):
// elements the array holds; at E >= 8 a 16-byte group may read elements n .. nalloc-1, which
// the caller ignores like every element past n.
template <int E>
struct Run16 {
  uint32_t w[E >= 2 ? E / 2 : 1];
};
template <int E>
__device__ __forceinline__ void load_run16(const int16_t* __restrict__ src, int n, int nalloc, int base, bool vec,
                                           Run16<E>& out, int16_t fill) {
  if constexpr (E >= 4 && E % 4 == 0) {
    if (vec && (E >= 8 || base + E <= n)) {
      if constexpr (E % 8 != 0) {  // E = 4, 12: the run starts 8-byte aligned (8-byte loads)
#pragma unroll
        for (int v = 0; v < E / 4; ++v) {
          const int gb = base + 4 * v;
          const u32x2 x = *(const u32x2*)(src + (E < 8 || gb + 4 <= n ? gb : n - 4));
          out.w[2 * v] = x[0];
          out.w[2 * v + 1] = x[1];
        }
      } else {
#pragma unroll
        for (int v = 0; v < E / 8; ++v) {
          const int gb = base + 8 * v;
          const u32x4 x = *(const u32x4*)(src + (E < 8 || gb + 8 <= nalloc ? gb : nalloc - 8));
#pragma unroll
          for (int q = 0; q < 4; ++q) out.w[4 * v + q] = x[q];
        }
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const uint32_t v = (uint16_t)((base + j < n) ? src[base + j] : fill);
    if (E == 1) out.w[0] = v;
    else if (j & 1) out.w[j >> 1] |= v << 16;
    else out.w[j >> 1] = v;
  }
}
template <int E>
__device__ __forceinline__ int16_t run16_at(const Run16<E>& a, int j) {
  if constexpr (E == 1) return (int16_t)a.w[0];
  else return (int16_t)(a.w[j >> 1] >> (16 * (j & 1)));
}

// A request's scalars read before anything else: the padded-request bound, a speculative union's
// length and the error its union kernel found.  The three loads are issued together and a
// compiler barrier keeps them from being moved to their uses, which would make one round trip
// of each; an absent input costs no load.
struct ReqScalars {
  int32_t nreq, kvr;
  uint32_t pre_err;
};
__device__ __forceinline__ ReqScalars read_req_scalars(const ResolveParams& p, int r) {
  ReqScalars rs;
  rs.nreq = p.num_reqs ? *p.num_reqs : INT32_MAX;
  rs.kvr = p.kvar ? p.kvar[r] : p.k;
  rs.pre_err = p.kerr ? p.kerr[r] : 0u;
  asm volatile("" ::: "memory");
  return rs;
}

// E: slots (and LRU positions) per thread, KE: selection entries per thread (both powers
// of two, KE <= E, EK = ceil(k / NT) <= KE).  ATT: workgroup 0 of the fused kernel (its
// other workgroups run fetch_attend instead).  It resolves as usual but leaves the page
// table alone: it writes the list of its misses (list index, victim slot, evicted position,
// new position) and a per-request header, and the finish kernel that follows applies the
// page-table updates and copies the missed records, which the fetch workgroups staged, into
// their victim slots.  So the page table does not change while the fused kernel runs.
// A request's metadata that RESOLVE reads first (the launch counter, the request's scalars, the
// LRU order's two halves, its host records' base), loaded by resolve_rows_kernel before it builds
// the union so that the loads land during that LDS work (resolve_body issues the same loads
// itself otherwise).
template <int E>
struct EntryLoads {
  uint64_t counter_raw;  // thread 0 only
  uint32_t short_req;
  int32_t newest, capr;
  int64_t ctx;
  Run16<E> lra, lrb;
  const uint8_t* hbase;
};
template <int E>
__device__ __forceinline__ void entry_loads(const ResolveParams& p, int r, EntryLoads<E>& en) {
  const int e0 = (int)threadIdx.x * E;
  const bool bvec = (p.B % 4) == 0;
  en.counter_raw = 0;
  if (threadIdx.x == 0)
    en.counter_raw = __hip_atomic_load((uint64_t*)&p.ctrl[r * 4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  en.short_req = p.ctrl[r * 4 + 3];
  en.newest = (p.flags & kHasNewest) ? p.newest[r] : -1;
  en.ctx = min((int64_t)p.ctx_len[r], p.max_positions);
  en.capr = p.cap ? p.cap[r] : p.B;
  load_run16<E>(p.lru + ((size_t)r * 2 + 0) * p.Bpad, p.B, p.Bpad, e0, bvec, en.lra, 0);
  load_run16<E>(p.lru + ((size_t)r * 2 + 1) * p.Bpad, p.B, p.Bpad, e0, bvec, en.lrb, 0);
  en.hbase = p.host_base[r] + p.host_layer_off;
}

// SL: the list is in LDS (sl: kr positions; the rows' union built by resolve_rows_kernel), not
// in global memory.
// pre (with SL): the entry loads, already issued (entry_loads).
template <int E, int KE, bool ATT, bool SL = false>
__device__ __forceinline__ void resolve_body(const ResolveParams& p, unsigned char* smem, const ReqScalars& rs,
                                             const int32_t* sl = nullptr, const EntryLoads<E>* pre = nullptr) {
  const ResolveLds Ly = resolve_lds(p.k, p.B, p.hash_bits, p.G);
  int32_t* htab = (int32_t*)(smem + Ly.htab);        // [H] list index of the entry in each bucket
  int32_t* selp = (int32_t*)(smem + Ly.selp);        // [k] position (hash key) of each entry
  int16_t* victim = (int16_t*)(smem + Ly.victim);    // [k] slot given to miss j     (stage 3 on,
  int16_t* missidx = (int16_t*)(smem + Ly.missidx);  // [k] list index of miss j   in the bytes
  int16_t* mrank = (int16_t*)(smem + Ly.mrank);      // [k] miss rank of an entry  of the hash)
  int16_t* sown = (int16_t*)(smem + Ly.sown);        // [B] -1 evictable, i >= 0 hit by entry i,
                                                     //     -2-j victim of miss j
  uint32_t* carry = (uint32_t*)(smem + Ly.scratch);  // 2 x 2 x NW scan carries
  uint32_t* rcnt = carry + 4 * NW;                   // [NW] resident entries per wave
  int* sh = (int*)(rcnt + NW);                       // [0] error bits [1] newest hits [2] half
                                                     // [3] slot map / page table disagreement
                                                     // [4] fast-path range error
                                                     // [5] page-table generation

  const int tid = threadIdx.x;
  const int r = blockIdx.x % p.R;
  const int g = blockIdx.x / p.R;
  const bool record = (p.flags & HS_RECORD_PLAN) != 0;
  const uint32_t pre_err = rs.pre_err;
  if (r >= rs.nreq) {
    // a padded request: untouched, and an empty plan so a replay copies nothing
    if (record && g == 0 && tid == 0) p.ctrl[r * 4 + 2] = 0;
    return;
  }
  const int H = 1 << p.hash_bits;
  const uint32_t hmask = (uint32_t)H - 1;
  const int e0 = tid * E;  // first slot / LRU position of this thread
  // entries of this request's list (a speculative union is shorter than its k-entry row), spread
  // over all threads: EK = ceil(kr / NT) <= KE consecutive entries per thread
  const int kr = min(rs.kvr, p.k);
  const int EK = (kr + NT - 1) / NT;
  const int i0 = tid * EK;  // first selection entry of this thread
  if (pre_err) {  // found before the launch (the union of verification rows): nothing changes
    if (g == 0) {
      for (int i = tid; i < p.k; i += NT) p.out[(size_t)r * p.k + i] = -1;
      if (tid == 0 && p.stats) {
        hs_stats st = {0u, 0u, pre_err, 0u, 0ull};
        p.stats[r] = st;
      }
      if (tid == 0 && record) p.ctrl[r * 4 + 2] = 0;
    }
    return;
  }

  // ---- every global read up front -------------------------------------------------------
  // All loads that do not depend on another load are issued before any branch that could
  // make the compiler wait: the launch counter, the request's scalars, the selection (this
  // workgroup's and its fetch share), and both halves of the slot map and LRU order.  Then
  // the page-table entries of the selected positions (which need the selection): two memory
  // round trips in all before the LDS work.
  // Launch counter (launch_number: the launches before this one that changed the
  // metadata, whichever of this launch's siblings have already added their share).  Its
  // parity picks the ping-pong half that holds the current slot map and LRU order, and
  // number + 1 is the generation this launch writes into the page table.  Thread 0 reads it
  // (an agent-scope load; one per wave made the all-hit call slower) and the value is used
  // only where sh[2] and sh[5] are set, so nothing waits for it before the other loads are
  // issued.
  uint64_t* counter = (uint64_t*)&p.ctrl[r * 4];
  uint64_t counter_raw = 0;
  uint32_t short_req;
  int32_t newest, capr;  // capr: LRU slots backed by device memory (an on-demand hot buffer grows)
  int64_t ctx;
  if constexpr (SL) {
    counter_raw = pre->counter_raw;
    short_req = pre->short_req;
    newest = pre->newest;
    ctx = pre->ctx;
    capr = pre->capr;
  } else {
    if (tid == 0) counter_raw = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    short_req = p.ctrl[r * 4 + 3];
    newest = (p.flags & kHasNewest) ? p.newest[r] : -1;
    ctx = min((int64_t)p.ctx_len[r], p.max_positions);
    capr = p.cap ? p.cap[r] : p.B;
  }
  const int32_t* selr = p.sel + (size_t)r * p.kb;
  const uint64_t* ptr = p.page_table + (size_t)r * p.max_positions;
  int32_t raw[KE];
#pragma unroll
  for (int j = 0; j < KE; ++j) {
    const int i = i0 + j;
    if constexpr (SL) raw[j] = (j < EK && i < kr) ? sl[i] : 0;
    else raw[j] = (j < EK && i < kr) ? selr[p.bt_shift ? (i >> p.bt_shift) : i] : 0;
  }
  // Fetch-only workgroups (g > 0 of a launch with several) also read the selection entries of
  // their share of the list, spread over the waves: entry e of the share belongs to wave
  // e % NW, lane (e / NW) % 64, slot e / NT.  Slot 0 is read at entry with everything else;
  // a share longer than NT entries (a long speculative union over few workgroups) reads its
  // further slots at the fetch stage.  A one-workgroup launch (G = 1) takes its misses from
  // its own classified entries instead.
  const bool io = !(p.flags & HS_SKIP_IO);
  const bool fetcher = !ATT && io && (p.G == 1 || g > 0);  // (the fused kernel's fetch workgroups
                                                           // do not run this function)
  const bool share_fetch = fetcher && g > 0;
  const int nf = p.G > 1 ? p.G - 1 : 1;
  const int gf = p.G > 1 ? g - 1 : 0;
  // (32-bit: k * G < 2^23)
  const int f_lo = kr * gf / nf;
  const int f_n = kr * (gf + 1) / nf - f_lo;
  const int wid = tid >> 6, lane = tid & 63;
  auto share_raw = [&](int q) -> int32_t {
    const int e = q * NT + lane * NW + wid;
    const int i = f_lo + e;
    // (unconditional, from entry 0 outside the share: the caller uses the value only inside it,
    // and a load whose value a branch computes on is waited for in that branch)
    if constexpr (SL) return sl[(share_fetch && e < f_n) ? i : 0];
    else return selr[(share_fetch && e < f_n) ? (i >> p.bt_shift) : 0];
  };
  const int32_t fraw0 = share_raw(0);
  // vector loads and stores of a thread's run: every half of the slot map starts 16-byte aligned
  // when B is a multiple of 4 (the LRU halves are padded to 8 entries)
  const bool bvec = (p.B % 4) == 0;
  // Both halves of the slot map are read here, before the launch counter says which one is
  // current, so they share the first round trip.  With 8 or more slots per thread they
  // would hold too many registers until the publish, which then reads the current half.
  constexpr bool kEarlySlotMap = E < 8;
  int32_t spa[kEarlySlotMap ? E : 1], spb[kEarlySlotMap ? E : 1];
  Run16<E> lra, lrb;
  if constexpr (kEarlySlotMap) {
    if (g == 0) {  // only workgroup 0 publishes, and only it needs the slot map
      load_run32<E>(p.slot_pos + ((size_t)r * 2 + 0) * p.B, p.B, e0, bvec, spa, -1);
      load_run32<E>(p.slot_pos + ((size_t)r * 2 + 1) * p.B, p.B, e0, bvec, spb, -1);
    }
  }
  // this (request, layer)'s host records (the pointer table is read at entry with the rest)
  const uint8_t* hbase;
  if constexpr (SL) {
    lra = pre->lra;
    lrb = pre->lrb;
    hbase = pre->hbase;
  } else {
    load_run16<E>(p.lru + ((size_t)r * 2 + 0) * p.Bpad, p.B, p.Bpad, e0, bvec, lra, 0);
    load_run16<E>(p.lru + ((size_t)r * 2 + 1) * p.Bpad, p.B, p.Bpad, e0, bvec, lrb, 0);
    hbase = p.host_base[r] + p.host_layer_off;
  }
  uint8_t* dbase = p.hot + (size_t)r * p.hot_req_stride + p.hot_layer_off;
  // fused: workgroup 0's report to the finish kernel
  uint32_t* hdr = ATT ? p.att_hdr + (size_t)r * 4 : nullptr;
  // (a compiler barrier: the loads above stay here, in the first round trip, instead of being
  // moved past the short-path test to their first use; it emits no instruction)
  asm volatile("" ::: "memory");
  // ---- short-sequence fast path ("HiSparse 深度解析" §5.4, §5.5): a request admitted short
  // keeps its tokens in slot order while its context fits B, so every position is its own
  // slot: no hash, no LRU, no host IO (only the range is checked)
  if (short_req != 0 && ctx <= p.B) {
    uint32_t bad = 0;
#pragma unroll
    for (int j = 0; j < KE; ++j) {
      const int i = i0 + j;
      const int64_t pos64 = p.bt_shift ? ((int64_t)raw[j] << p.bt_shift) + (i & ((1 << p.bt_shift) - 1))
                                       : (int64_t)raw[j];
      if (j < EK && i < kr) bad |= (uint32_t)(pos64 < 0 || pos64 >= ctx);
    }
    // block-wide OR through a scratch word of the dynamic LDS (no static LDS in this kernel)
    if (tid == 0) sh[4] = 0;
    __syncthreads();
    if (bad) atomicOr((unsigned*)&sh[4], HS_ERR_RANGE);
    // slot = position needs every position of the context backed
    if (tid == 0 && ctx > capr) atomicOr((unsigned*)&sh[4], HS_ERR_CAPACITY);
    __syncthreads();
    bad = (uint32_t)sh[4];
    if (g == 0) {
      int32_t* outr = p.out + (size_t)r * p.k;
      if (bad) {
        for (int i = tid; i < p.k; i += NT) outr[i] = -1;
      } else {
#pragma unroll
        for (int j = 0; j < KE; ++j) {
          const int i = i0 + j;
          if (j < EK && i < kr)
            outr[i] = p.bt_shift ? (int32_t)((raw[j] << p.bt_shift) + (i & ((1 << p.bt_shift) - 1))) : raw[j];
        }
      }
      if (tid == 0 && p.stats) {
        hs_stats st = {bad ? 0u : (uint32_t)kr, 0u, bad, 0u, 0ull};
        p.stats[r] = st;
      }
      if (tid == 0 && record) p.ctrl[r * 4 + 2] = 0;
      if (ATT && tid == 0) { hdr[0] = bad; hdr[1] = 0u; }
    }
    return;
  }
  // The second round trip (after the short-path test, which needs only the first): the
  // page-table entries of the selected positions and, with a resident tier, their resident pages.
  const bool tiered = p.rtable != nullptr;
  const int32_t* rtr = p.rtable + (tiered ? (size_t)r * p.rt_stride : 0);
  // Misses known early from the page table: a selected position whose entry is -1 (and
  // that the resident tier does not serve) is not on the device.  Their host loads start
  // right after stage 1 and land while stage 3 runs; stage 3 names the slots they go to.
  // a share entry's position, page-table entry and resident page (slot q, its raw selection)
  struct ShareEntry {
    int32_t pos, res;
    uint64_t pt;
  };
  auto share_entry = [&](int q, int32_t fr) -> ShareEntry {
    const int e = q * NT + lane * NW + wid;
    const int i = f_lo + e;
    int64_t pos64 = -1;
    if (share_fetch && e < f_n)
      pos64 = p.bt_shift ? ((int64_t)fr << p.bt_shift) + (i & ((1 << p.bt_shift) - 1)) : (int64_t)fr;
    const bool ok = pos64 >= 0 && pos64 < ctx;
    ShareEntry se;
    se.pos = ok ? (int32_t)pos64 : -1;
    se.pt = ok ? ptr[pos64] : kPtHostOnly;
    se.res = (ok && tiered) ? rtr[pos64 >> p.page_shift] : -1;
    return se;
  };
  // (the share's entry first: its page-table load waits only for its own selection entry, while
  // a wait after the own entries' loads, some of which are skipped, would wait for all of them)
  const ShareEntry f0 = share_entry(0, fraw0);
  // Each own entry's page-table entry (the page table is kept the exact inverse of the slot
  // map, so it names the slot of a hit) and resident page.
  uint64_t ptv[KE];
  int32_t rpg[KE];
#pragma unroll
  for (int j = 0; j < KE; ++j) {
    const int i = i0 + j;
    const int64_t pos64 = p.bt_shift ? ((int64_t)raw[j] << p.bt_shift) + (i & ((1 << p.bt_shift) - 1))
                                     : (int64_t)raw[j];
    const bool ok = j < EK && i < kr && pos64 >= 0 && pos64 < ctx;
    ptv[j] = ok ? ptr[pos64] : kPtHostOnly;
    rpg[j] = (ok && tiered) ? rtr[pos64 >> p.page_shift] : -1;
  }
  {
    u32x4* h4 = (u32x4*)htab;
    const u32x4 e4 = {~0u, ~0u, ~0u, ~0u};
    for (int h = tid; h < H / 4; h += NT) h4[h] = e4;
    u32x4* s4 = (u32x4*)sown;  // B int16, padded to 16 bytes
    for (int h = tid; h < (p.B + 7) / 8; h += NT) s4[h] = e4;
  }
  if (tid == 0) {
    // (an opaque use: without it the compiler folds the arithmetic below into the load's own
    // branch at entry, and thread 0's wave then waits there for the counter before it issues
    // its other loads, one more memory round trip for the whole workgroup)
    asm volatile("" : "+v"(counter_raw));
    const uint64_t launches = launch_number(counter_raw);
    sh[0] = 0; sh[1] = 0; sh[3] = 0;
    sh[2] = (int)(launches & 1u);
    sh[5] = (int)(uint32_t)(launches + 1);  // this launch's page-table generation
  }
  // resident entries with a row inside the pool, counted per wave
  uint32_t rbits = 0;
  if (tiered) {
    const int64_t pmask = ((int64_t)1 << p.page_shift) - 1;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KE; ++j) {
      const int i = i0 + j;
      const int64_t pos64 = p.bt_shift ? ((int64_t)raw[j] << p.bt_shift) + (i & ((1 << p.bt_shift) - 1))
                                       : (int64_t)raw[j];
      const bool res = rpg[j] >= 0 && (((int64_t)rpg[j] << p.page_shift) + (pos64 & pmask)) < p.res_rows;
      rbits |= (uint32_t)res << j;
      cnt += __popcll(__ballot(res));
    }
    if (lane == 0) rcnt[wid] = (uint32_t)cnt;
  }
  __syncthreads();
  // Page-table entries written by this launch's workgroup 0 (a sibling that reads late can
  // see them) name positions that were host only when the launch began.
  const uint32_t gen = (uint32_t)sh[5];
  int32_t pts[KE];
#pragma unroll
  for (int j = 0; j < KE; ++j) pts[j] = pt_slot_for(ptv[j], gen);
  // ---- resident tier: a selection that is resident throughout returns here ---------------
  int nres = 0;
  if (tiered) {
#pragma unroll
    for (int w = 0; w < NW; ++w) nres += (int)rcnt[w];
    if (nres == kr) {
      if (g == 0) {
        const int64_t pmask = ((int64_t)1 << p.page_shift) - 1;
#pragma unroll
        for (int j = 0; j < KE; ++j) {
          const int i = i0 + j;
          if (j < EK && i < kr) {
            const int64_t pos64 = p.bt_shift ? ((int64_t)raw[j] << p.bt_shift) + (i & ((1 << p.bt_shift) - 1))
                                             : (int64_t)raw[j];
            p.out[(size_t)r * p.k + i] = p.B + 1 + (int32_t)(((int64_t)rpg[j] << p.page_shift) + (pos64 & pmask));
          }
        }
        if (tid == 0 && p.stats) {
          hs_stats st = {0u, 0u, 0u, (uint32_t)kr, 0ull};
          p.stats[r] = st;
        }
        if (tid == 0 && record) p.ctrl[r * 4 + 2] = 0;
        if (ATT && tid == 0) { hdr[0] = 0u; hdr[1] = 0u; }
      }
      return;
    }
  }

  // ---- stages 1 and 2: classify each entry, mark the hit slots, hash the rest -------------
  // An entry is served by the resident tier, by the newest slot, by the slot its page-table
  // entry names (a hit: the entry claims that slot, which marks it), or is a miss.  Misses
  // and resident entries go into the LDS hash, the resident ones under the complemented
  // position, so duplicates are caught in every class: two entries of one position share
  // their class, and a second claim of a slot or a second hash entry of a key reveals it.
  //
  // Hash insertion in two steps.  (a) Every entry stores its list index into its home
  // bucket of the empty table with a plain store; after a barrier an entry whose index
  // reads back owns that bucket, and one that finds another entry of the same key there is
  // a duplicate.  (b) The entries that lost their home bucket (a small fraction: the table
  // is at most a quarter full) insert with compare-and-swap linear probing, which never
  // overwrites a bucket.  LDS atomics are serialised lane by lane, so step (a) keeps most
  // of the table build off them.  Slot claims use the same plain-store-and-read-back.
  uint32_t err = 0;
  uint32_t pending = 0, hitb = 0;
  uint32_t hh[KE];
  int32_t key[KE], cls[KE];  // cls: published value (slot, B, B+1+row), -1 miss, -2 invalid
#pragma unroll
  for (int j = 0; j < KE; ++j) {
    const int i = i0 + j;
    key[j] = -1;
    hh[j] = 0;
    cls[j] = -2;
    if (j >= EK || i >= kr) continue;
    const int64_t pos64 = p.bt_shift ? ((int64_t)raw[j] << p.bt_shift) + (i & ((1 << p.bt_shift) - 1))
                                     : (int64_t)raw[j];
    if (pos64 < 0 || pos64 >= ctx) {
      err |= HS_ERR_RANGE;
      continue;
    }
    if (rpg[j] >= 0) {  // resident page: served from the resident pool
      const int64_t row = ((int64_t)rpg[j] << p.page_shift) + (pos64 & (((int64_t)1 << p.page_shift) - 1));
      if ((rbits >> j) & 1u) cls[j] = p.B + 1 + (int32_t)row;
      else err |= HS_ERR_RESIDENT;
      key[j] = ~(int32_t)pos64;
    } else if ((int32_t)pos64 == newest) {  // the newest token sits in slot B, outside the LRU
      cls[j] = p.B;
      atomicAdd(&sh[1], 1);
      continue;
    } else if (pts[j] >= 0) {  // a hit: the slot holding the position
      selp[i] = (int32_t)pos64;
      if (pts[j] >= p.B) {  // the page table never names a slot outside [0, B)
        err |= HS_ERR_STATE;
        continue;
      }
      cls[j] = pts[j];
      sown[pts[j]] = (int16_t)i;
      hitb |= 1u << j;
      continue;
    } else {
      cls[j] = -1;
      key[j] = (int32_t)pos64;
    }
    selp[i] = key[j];
    hh[j] = hash_pos((int32_t)pos64, p.hash_bits);
    htab[hh[j]] = i;
    pending |= 1u << j;
  }
  __syncthreads();  // home-bucket stores, slot claims and every key are visible
  {
    // branch-free read-back: every read issued before any result is used
    int32_t own[KE], kk[KE];
    int16_t so[KE];
#pragma unroll
    for (int j = 0; j < KE; ++j) own[j] = htab[hh[j]];
#pragma unroll
    for (int j = 0; j < KE; ++j) so[j] = sown[((hitb >> j) & 1u) ? cls[j] : 0];
#pragma unroll
    for (int j = 0; j < KE; ++j) kk[j] = selp[own[j] < 0 ? 0 : own[j]];
#pragma unroll
    for (int j = 0; j < KE; ++j) {
      const bool act = (pending >> j) & 1u;
      const bool mine = own[j] == i0 + j;
      const bool dup = !mine && kk[j] == key[j];
      if (act && dup) err |= HS_ERR_DUP;
      if (act && (mine || dup)) pending &= ~(1u << j);
      if (act && !mine && !dup) hh[j] = (hh[j] + 1) & hmask;
      if (((hitb >> j) & 1u) && so[j] != (int16_t)(i0 + j)) err |= HS_ERR_DUP;
    }
  }
  // (no barrier: compare-and-swap only fills empty buckets, and every home bucket read
  // above is already non-empty)
#pragma unroll
  for (int j = 0; j < KE; ++j) {
    while ((pending >> j) & 1u) {
      const int32_t prev = atomicCAS(&htab[hh[j]], -1, i0 + j);
      if (prev == -1) {
        pending &= ~(1u << j);
      } else if (selp[prev] == key[j]) {
        err |= HS_ERR_DUP;
        pending &= ~(1u << j);
      } else {
        hh[j] = (hh[j] + 1) & hmask;
      }
    }
  }
  // ---- stage 4, first part: per-wave lists of the page-table misses, host loads issued ----
  int32_t* wpos = (int32_t*)(smem + Ly.wpos) + wid * Ly.wcap;  // this wave's misses: position
  int16_t* widx = (int16_t*)(smem + Ly.widx) + wid * Ly.wcap;  // and list index
  const int C = p.rec_bytes >> 4;  // 16-byte chunks per record
  const float invC = __builtin_amdgcn_rcpf((float)C);  // (the +-1 corrections below absorb its error)
  int mw = 0;  // misses of this wave
  auto append = [&](bool miss, int32_t pos, int i) {
    const uint64_t b = __ballot(miss);
    if (miss) {
      const int at = mw + lanes_below(b);
      wpos[at] = pos;
      widx[at] = (int16_t)i;
    }
    mw += __popcll(b);
  };
  auto share_miss = [&](const ShareEntry& se) {
    return se.pos >= 0 && se.pos != newest && se.res < 0 && pt_slot_for(se.pt, gen) < 0;
  };
  if (share_fetch) {
    append(share_miss(f0), f0.pos, f_lo + lane * NW + wid);
    for (int q = 1; q * NT < f_n; ++q) {  // (the same bound in every wave)
      const ShareEntry se = share_entry(q, share_raw(q));
      append(share_miss(se), se.pos, f_lo + q * NT + lane * NW + wid);
    }
  } else if (fetcher) {  // one workgroup per request: its own entries' misses
#pragma unroll
    for (int j = 0; j < KE; ++j) append(j < EK && i0 + j < kr && cls[j] == -1, key[j], i0 + j);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int wtotal = mw * C;  // 16-byte chunks of this wave's misses
  // With 8 list entries or 16 slots per thread these registers would not last through stage 3
  // (the compiler then waits for each load and spills its value), so those layouts load none
  // early; 12 slots with at most 2 entries load 2 chunks per lane early (their registers fit).
  // 12 slots and 4 entries load one chunk early when the entries come from the union list in
  // LDS (the position registers of the list are free by then; measured faster), none otherwise.
  constexpr int kEarlyN = (KE >= 8 || E >= 16) ? 0 : (E >= 12 ? (KE >= 4 ? (SL ? 1 : 0) : 2) : kEarly);
  u32x4 early[kEarlyN > 0 ? kEarlyN : 1];
#pragma unroll
  for (int u = 0; u < kEarlyN; ++u) {
    const int c = lane + 64 * u;
    if (c < wtotal) {
      int l = (int)((float)c * invC);
      int cc = c - l * C;
      if (cc < 0) { --l; cc += C; }
      if (cc >= C) { ++l; cc -= C; }
      early[u] = load_host16(hbase + (size_t)wpos[l] * (size_t)p.rec_bytes + 16 * (size_t)cc);
    }
  }

  // the normal path may fill any of the B slots: all of them must be backed (every workgroup
  // of the request sees the same capacity, so all of them return below and nothing changes)
  if (tid == 0 && capr < p.B) err |= HS_ERR_CAPACITY;
  if (err) atomicOr((unsigned*)&sh[0], err);
  __syncthreads();
  err = (uint32_t)sh[0] | (sh[1] > 1 ? HS_ERR_DUP : 0u);
  const bool h1 = sh[2] != 0;  // current metadata in half 1, new metadata goes to half 0
  int16_t lro[E];
#pragma unroll
  for (int j = 0; j < E; ++j) lro[j] = h1 ? run16_at(lrb, j) : run16_at(lra, j);
  int16_t* lru_new = p.lru + ((size_t)r * 2 + (h1 ? 0 : 1)) * p.Bpad;

  if (err) {  // every workgroup of the request sees the same error; nothing changes
    if (g == 0) {
      for (int i = tid; i < p.k; i += NT) p.out[(size_t)r * p.k + i] = -1;
      if (tid == 0 && p.stats) {
        hs_stats st = {0u, 0u, err, 0u, 0ull};
        p.stats[r] = st;
      }
      if (tid == 0 && record) p.ctrl[r * 4 + 2] = 0;
      if (ATT && tid == 0) { hdr[0] = err; hdr[1] = 0u; }
    }
    return;
  }
  // this launch changes the metadata: the next one finds it in the other half (the shares
  // of the G workgroups add up to one launch unit)
  // (the fused kernel's other workgroups do not resolve: workgroup 0 adds the whole unit)
  if (tid == 0)
    __hip_atomic_fetch_add(counter,
                           g == 0 ? (1ull << kLaunchShift) - (ATT ? 0ull : (uint64_t)(p.G - 1)) : 1ull,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // The entries served without a fetch (hit slot, newest slot, resident row) are published at
  // the end of the publish stage; in the large layouts (8 list entries or 12 slots per thread)
  // already here, so that the per-entry classes are not held through stage 3 and publish.
  constexpr bool kEarlyHitOut = KE >= 8 || E >= 12;
  uint32_t mbits = 0, ebits = 0;
#pragma unroll
  for (int j = 0; j < KE; ++j) {
    if (cls[j] == -1) mbits |= 1u << j;
    if (kEarlyHitOut && g == 0 && cls[j] >= 0) p.out[(size_t)r * p.k + i0 + j] = cls[j];
  }

  // ---- stage 3: misses in list order and evictables in LRU order, one scan -------------
  {
    int16_t sf[E];
#pragma unroll
    for (int j = 0; j < E; ++j) sf[j] = sown[E < 8 || e0 + j < p.B ? lro[j] : 0];  // (past B: not a slot)
#pragma unroll
    for (int j = 0; j < E; ++j)
      if (e0 + j < p.B && sf[j] == -1) ebits |= 1u << j;
  }
  int rm, re, m, E_;
  block_ranks2<E>(mbits, ebits, carry, rm, re, m, E_);  // m misses, E_ evictable slots
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if ((mbits >> j) & 1u) {
      missidx[rm] = (int16_t)(i0 + j);
      mrank[i0 + j] = (int16_t)rm;
      ++rm;
    }
    if ((ebits >> j) & 1u) {
      const int s = lro[j];
      if (re < m) {
        victim[re] = (int16_t)s;
        sown[s] = (int16_t)(-2 - re);
      } else if (g == 0) {
        lru_new[re - m] = (int16_t)s;  // untouched evictables keep their old order
      }
      ++re;
    }
  }
  __syncthreads();

  // with several workgroups, workgroup 0 publishes while the others fetch
  if (g == 0) {
    int32_t spo[E];
#pragma unroll
    for (int j = 0; j < E; ++j) spo[j] = kEarlySlotMap ? (h1 ? spb[j] : spa[j]) : -1;
    if constexpr (!kEarlySlotMap) load_run32<E>(p.slot_pos + ((size_t)r * 2 + (h1 ? 1 : 0)) * p.B, p.B, e0, bvec, spo, -1);
    int32_t* sp_new = p.slot_pos + ((size_t)r * 2 + (h1 ? 0 : 1)) * p.B;
    // filled victims, then hits, each by slot index, after the untouched evictables (the owner
    // of each slot is read from the LDS owner array here and again in the publish loop, so no
    // per-slot array is held across the rank scan beside the slot map)
    uint32_t vb = 0, hb = 0, bad = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int16_t fo = (e0 + j < p.B) ? sown[e0 + j] : (int16_t)-1;
      const int32_t hp = selp[fo >= 0 ? fo : 0];
      vb |= (uint32_t)(fo <= -2) << j;
      hb |= (uint32_t)(fo >= 0) << j;
      bad |= (uint32_t)(fo >= 0 && hp != spo[j]);  // a hit's slot must hold its position
    }
    if (bad) atomicOr((unsigned*)&sh[3], HS_ERR_STATE);
    int rv, rh, tv, th;
    block_ranks2<E>(vb, hb, carry + 2 * NW, rv, rh, tv, th);
    uint64_t* pt = p.page_table + (size_t)r * p.max_positions;
    int32_t* outr = p.out + (size_t)r * p.k;
    int32_t* plan_pos = p.plan + (size_t)r * 2 * p.plan_k;
    int32_t* plan_slot = plan_pos + p.plan_k;

    // ---- stage 5: publish (every value is already on chip); spo becomes the new slot map ----
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int s = e0 + j;
      if (s >= p.B) continue;
      if ((vb >> j) & 1u) {
        lru_new[E_ - m + rv++] = (int16_t)s;
        const int jm = -2 - sown[s];
        const int i = missidx[jm];
        const int32_t np = selp[i];
        if constexpr (ATT) {  // the finish kernel applies it
          const u32x4 e = {(uint32_t)i, (uint32_t)s, (uint32_t)spo[j], (uint32_t)np};
          *(u32x4*)(p.att_mlist + ((size_t)r * p.k + jm) * 4) = e;
        } else {
          if (spo[j] >= 0) pt[spo[j]] = kPtHostOnly;  // the evicted position is host-only again
          pt[np] = pt_entry(s, gen);
        }
        spo[j] = np;
        outr[i] = s;
        if (record) {
          plan_pos[jm] = np;
          plan_slot[jm] = s;
        }
      } else if ((hb >> j) & 1u) {
        lru_new[E_ + rh++] = (int16_t)s;
      }
    }
    bool stored = false;
    if constexpr (E % 4 == 0) {
      if (bvec && e0 + E <= p.B) {
#pragma unroll
        for (int v = 0; v < E / 4; ++v) {
          const u32x4 x = {(uint32_t)spo[4 * v], (uint32_t)spo[4 * v + 1], (uint32_t)spo[4 * v + 2],
                           (uint32_t)spo[4 * v + 3]};
          *((u32x4*)(sp_new + e0) + v) = x;
        }
        stored = true;
      }
    }
    if (!stored) {
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (e0 + j < p.B) sp_new[e0 + j] = spo[j];
    }
    if constexpr (!kEarlyHitOut) {
#pragma unroll
      for (int j = 0; j < KE; ++j)
        if (cls[j] >= 0) outr[i0 + j] = cls[j];
    }
    if (tid == 0) {
      if (p.stats) {
        hs_stats st = {(uint32_t)(kr - m - nres), (uint32_t)m, (uint32_t)sh[3], (uint32_t)nres,
                        io ? (uint64_t)m * (uint64_t)p.rec_bytes : 0ull};
        p.stats[r] = st;
      }
      if (record) p.ctrl[r * 4 + 2] = (uint32_t)m;
      if (ATT) { hdr[0] = 0u; hdr[1] = (uint32_t)m; hdr[2] = gen; }
    }
    if (p.G > 1) return;
  }

  // ---- stage 4, second part: the early chunks go to the slots stage 3 chose, then the rest
  // of this wave's misses
  if (fetcher) {
#pragma unroll
    for (int u = 0; u < kEarlyN; ++u) {
      const int c = lane + 64 * u;
      if (c < wtotal) {
        int l = (int)((float)c * invC);
        int cc = c - l * C;
        if (cc < 0) { --l; cc += C; }
        if (cc >= C) { ++l; cc -= C; }
        const int slot = victim[mrank[widx[l]]];
        *((u32x4*)(dbase + (size_t)slot * (size_t)p.rec_bytes) + cc) = early[u];
      }
    }
    // a wave with more than kEarlyN chunks per lane (miss-heavy steps) continues here
    for (int c0 = lane + 64 * kEarlyN; c0 < wtotal; c0 += 64 * kUnroll) {
      u32x4 v[kUnroll];
      int ll[kUnroll], cc[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + 64 * u;
        if (c < wtotal) {
          int l = (int)((float)c * invC);
          int x = c - l * C;
          if (x < 0) { --l; x += C; }
          if (x >= C) { ++l; x -= C; }
          ll[u] = l;
          cc[u] = x;
          v[u] = load_host16(hbase + (size_t)wpos[l] * (size_t)p.rec_bytes + 16 * (size_t)x);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (c0 + 64 * u < wtotal)
          *((u32x4*)(dbase + (size_t)victim[mrank[widx[ll[u]]]] * (size_t)p.rec_bytes) + cc[u]) = v[u];
    }
  }
}

// A fetch workgroup g >= 1 of the fused kernel: attention over its share (chunk g - 1, at
// most 64 att_tiles entries) of the selection, one 64-row tile at a time.  It does not
// resolve.  Each share entry's record is where the page table (stable while the fused kernel
// runs: workgroup 0 leaves its updates to the finish kernel) and the resident tier put it: a
// resident row, the newest slot, the hot slot of a hit, or for a miss the host record.  All
// share entries' record addresses are found first, in one pass.  A tile's records are loaded
// into registers (5 x 16 bytes per thread) and written to the LDS tile, the missed ones also
// to the staging area (by list index) from which the finish kernel copies them into their
// victim slots, so host bytes cross the link once; the next tile's loads are issued before
// the current tile is attended, so they fly meanwhile.  Entries in error (out of range,
// resident rows outside the pool) load a finite filler row; workgroup 0 reports the error
// and the finish kernel makes the request's output NaN.  F8: FP8 records (tile_load8 /
// tile_store8; the staged misses are the raw 656-byte records; the filler is a zero record).
template <bool F8>
__device__ __forceinline__ void fetch_attend(const ResolveParams& p, unsigned char* smem) {
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int r = blockIdx.x % p.R, g = blockIdx.x / p.R;
  if (p.num_reqs && r >= *p.num_reqs) return;
  const int S = p.G - 1;
  const int f_lo = p.k * (g - 1) / S;  // (32-bit: k * G < 2^23)
  const int f_n = p.k * g / S - f_lo;  // <= 64 att_tiles
  const int nt = (f_n + kTileRows - 1) / kTileRows;
  const FusedLds F = fused_lds(p.k, p.B, p.hash_bits, p.G, p.att_tiles, F8);
  unsigned char* tile = smem + F.tile;
  unsigned char* qs = smem + F.qs;
  const uint8_t* filler = F8 ? p.att_zero : (const uint8_t*)(p.q + (size_t)r * p.heads * kAttnDk);
  // the request's scalars, read before the branches below so that they share the selection's
  // round trip and only the page-table entries come after it
  const uint8_t* hbase = p.host_base[r] + p.host_layer_off;
  const int64_t ctx = min((int64_t)p.ctx_len[r], p.max_positions);
  const int32_t newest = (p.flags & kHasNewest) ? p.newest[r] : -1;
  const uint32_t short_req = p.ctrl[r * 4 + 3];
  const int32_t capr = p.cap ? p.cap[r] : p.B;
  const uint8_t* dbase = p.hot + (size_t)r * p.hot_req_stride + p.hot_layer_off;
  u32x4 qv[kQU];
  q_load(qv, p.q, r, p.heads);
  // share entry e = lane * NW + wid: tile t's rows 16 i + wid (i = 0..3) on lanes 4 t + i of
  // wave wid, so each wave loads the rows its own lanes resolved (wave_rows_load)
  const int e = lane * NW + wid;
  uint64_t my_src = (uint64_t)filler;  // this lane's row: record address, and the list index of a miss
  int32_t my_mi = -1;
  if (e < nt * kTileRows) {
    const uint8_t* src = filler;
    int32_t mi = -1;
    if (e < f_n) {
      const int i = f_lo + e;
      const bool short_path = short_req != 0 && ctx <= p.B;  // slot = position
      const int32_t raw = p.sel[(size_t)r * p.kb + (p.bt_shift ? (i >> p.bt_shift) : i)];
      const int64_t pos64 = p.bt_shift ? ((int64_t)raw << p.bt_shift) + (i & ((1 << p.bt_shift) - 1)) : (int64_t)raw;
      if (pos64 >= 0 && pos64 < ctx) {
        if (short_path) {
          // (a position outside the backed slots keeps the filler: workgroup 0 reports it)
          if (pos64 < capr) src = dbase + (size_t)pos64 * p.rec_bytes;
        } else {
          const int32_t sl = (int32_t)(uint32_t)p.page_table[(size_t)r * p.max_positions + pos64];
          const int32_t rp = p.rtable ? p.rtable[(size_t)r * p.rt_stride + (pos64 >> p.page_shift)] : -1;
          if (rp >= 0) {
            const int64_t row = ((int64_t)rp << p.page_shift) + (pos64 & (((int64_t)1 << p.page_shift) - 1));
            if (row < p.res_rows) src = p.att_res + (size_t)row * p.rec_bytes;
          } else if ((int32_t)pos64 == newest) {
            src = dbase + (size_t)p.B * p.rec_bytes;
          } else if (sl >= 0) {
            if (sl < p.B) src = dbase + (size_t)sl * p.rec_bytes;
          } else {
            src = hbase + (size_t)pos64 * p.rec_bytes;
            mi = i;
          }
        }
      }
    }
    my_src = (uint64_t)src;
    my_mi = mi;
  }
  q_store(qv, qs);  // read after the barrier that precedes the first tile's attention
  const float sl2 = p.att_scale * 1.4426950408889634f;
  constexpr int TU = F8 ? kTU8 : kTU;
  constexpr int RC = F8 ? kF8RowChunks : kRowChunks;
  u32x4 tv[TU];
  wave_rows_load<RC, TU>(tv, my_src, 0);
  AttnAcc acc;
  acc_init(acc);
  for (int t = 0; t < nt; ++t) {
    if (t > 0) __syncthreads();  // the previous tile's readers are done with the tile and P
    // the missed records, as loaded, to the staging area
    int32_t mi4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mi4[i] = __builtin_amdgcn_readlane(my_mi, 4 * t + i);
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const int q = lane + 64 * u;
      if (q < 4 * RC) {
        const int i = q / RC, c = q - i * RC;
        const int a = pick4(mi4, i);
        if (a >= 0) *((u32x4*)(p.att_stage + ((size_t)r * p.k + a) * (size_t)p.rec_bytes) + c) = tv[u];
      }
    }
    wave_rows_store<RC, TU, F8>(tv, tile, tile_scales8(smem + F.scratch));
    if (t + 1 < nt) wave_rows_load<RC, TU>(tv, my_src, 4 * (t + 1));
    __syncthreads();
    attend_tile<F8>(tile, qs, smem + F.scratch, min(kTileRows, f_n - t * kTileRows), sl2, acc);
  }
  float* part = p.part + ((size_t)r * S + (g - 1)) * kPartStride;
  float* out = S == 1 ? p.att_out + (size_t)r * p.heads * kAttnDv : nullptr;
  attend_write(acc, part, out, p.heads);
}

template <int E, int KE, bool ATT>
__global__ void __launch_bounds__(NT) resolve_kernel(ResolveParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if constexpr (ATT) {
    if ((int)(blockIdx.x / p.R) > 0) {
      fetch_attend<false>(p, smem);
      return;
    }
  }
  resolve_body<E, KE, ATT>(p, smem, read_req_scalars(p, blockIdx.x % p.R));
}

// Workgroup 0 of a union's RESOLVE, after resolve_body: every (row, entry) gets the slot of its
// union entry (bad: the union's error bits, which make every row slot -1; real: r is a request
// below *num_reqs).  The rows' entries (rows_n <= kUnionMaxEntries): all union indices are
// loaded at once, then all union slots, so the scatter takes two memory round trips (a loop that
// loads and uses one entry at a time waits for both loads of every entry in turn).
__device__ __forceinline__ void rows_scatter(const ResolveParams& p, int r, uint32_t bad, bool real) {
  constexpr int FR = kUnionMaxEntries / NT;
  const int32_t* mp = p.rows_map + (size_t)r * p.k;
  int32_t u[FR], v[FR];
#pragma unroll
  for (int j = 0; j < FR; ++j) {
    const int f = j * NT + (int)threadIdx.x;
    u[j] = mp[f < p.rows_n ? f : 0];
  }
  if (!real) return;
  __syncthreads();  // workgroup 0's writes of the union's slots are visible to all its threads
  const int32_t* uo = p.out + (size_t)r * p.k;
#pragma unroll
  for (int j = 0; j < FR; ++j) v[j] = uo[(u[j] >= 0 && u[j] < p.k) ? u[j] : 0];
  int32_t* ro = p.rows_out + (size_t)r * p.rows_n;
#pragma unroll
  for (int j = 0; j < FR; ++j) {
    const int f = j * NT + (int)threadIdx.x;
    if (f < p.rows_n) ro[f] = (bad || u[j] < 0) ? -1 : v[j];
  }
}

// RESOLVE over a speculative union whose capacity (rows x k entries) needs KE > kUnionShortKE
// list entries per thread (launch_resolve).  A union of <= kUnionShortKE NT entries, the usual
// case, takes the body with kUnionShortKE entries per thread, whose registers fit; a longer one
// the body with KE.  The choice is per request (every workgroup of the request reads the same
// length).  Workgroup 0 then gives every row entry its union entry's slot (the scatter).
template <int E, int KE>
__global__ void __launch_bounds__(NT) resolve_union_kernel(ResolveParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int r = blockIdx.x % p.R, g = blockIdx.x / p.R;
  const ReqScalars rs = read_req_scalars(p, r);
  const int kr = min(rs.kvr, p.k);
  if (kr <= kUnionShortKE * NT) resolve_body<E, kUnionShortKE, false>(p, smem, rs);
  else resolve_body<E, KE, false>(p, smem, rs);
  // (every return in resolve_body is taken by the whole workgroup, so all its threads are here)
  if (g != 0) return;
  rows_scatter(p, r, rs.pre_err, r < rs.nreq);
}

// The fused kernel over FP8 records: workgroup 0 as in resolve_kernel<E, KE, true>, the fetch
// workgroups on FP8 tiles.
template <int E, int KE>
__global__ void __launch_bounds__(NT) resolve_f8_kernel(ResolveParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if ((int)(blockIdx.x / p.R) > 0) {
    fetch_attend<true>(p, smem);
    return;
  }
  resolve_body<E, KE, true>(p, smem, read_req_scalars(p, blockIdx.x % p.R));
}

// Union of the verification rows of one speculative step ("HiSparse 深度解析" §6.5
// comparison table; "HiSparse local KV offload architecture" (docs.vllm.ai),
// speculative decoding): rows that select the same position share one slot, so the
// rows are resolved as one list, their union in first-reference order (row by row,
// list order within a row).  One workgroup per request; entry f (row-major over the rows)
// belongs to thread f % NT as its slot f / NT, so every load and store of the entries is
// coalesced:
//   - every entry finds or inserts its position in an LDS hash (one bucket per distinct
//     position: a plain store into the home bucket, then compare-and-swap linear probing
//     for the entries whose home bucket holds another position, all of a thread's entries
//     probing together);
//   - each entry adds its row's bit and a count into its bucket's word: once every row's
//     entries are in, fewer set row bits than entries is a duplicate inside a row, and an
//     entry whose word has no lower row bit is its position's first reference;
//   - the first references are ranked in list order (per slot and wave a ballot count, then
//     one scan of those counts); the rank is the position's index in the union, stored in
//     the bucket for the other entries.
constexpr int EU = kUnionMaxEntries / NT;  // entries per thread

// Exclusive ranks in entry order (entry j NT + t for bit j of thread t) of the set bits of
// `bits`, and their total.  cnt: EU x NW words of LDS.  Each wave ballots per slot and
// stores its counts; after one barrier every wave scans all EU x NW counts (two per lane)
// and takes its own prefixes by lane shuffles.
__device__ __forceinline__ void union_ranks(uint32_t bits, uint32_t* cnt, int (&rank)[EU], int& total) {
  static_assert(EU * NW == 128, "two counts per lane");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int below[EU];
#pragma unroll
  for (int j = 0; j < EU; ++j) {
    const uint64_t m = __ballot((bits >> j) & 1u);
    below[j] = lanes_below(m);
    if (lane == 0) cnt[j * NW + wid] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  const int c0 = (int)cnt[2 * lane], c1 = (int)cnt[2 * lane + 1];
  int incl = c0 + c1;  // inclusive scan over the lanes of the pair sums
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  const int ex0 = incl - c0 - c1;  // exclusive prefix of count 2 lane; of 2 lane + 1: ex0 + c0
  total = __shfl(incl, 63);
#pragma unroll
  for (int j = 0; j < EU; ++j) {
    const int idx = j * NW + wid;
    const int e = __shfl(ex0, idx >> 1), a = __shfl(c0, idx >> 1);
    rank[j] = e + ((idx & 1) ? a : 0) + below[j];
  }
}

// The union of request r's rows, in the union's LDS (smem, union_lds_bytes): the union list goes
// to `ulist` (global memory, or the first 4 kmax bytes of smem: the position array, dead when
// the list is written), and with `outputs` each entry's union index to p.map and the union
// size and error bits to p.cnt / p.err.  nu: the union size (0 on an error), err: the error
// bits.  Returns false, having written nothing, for a request past *num_reqs.  Every return is
// taken by the whole workgroup.
__device__ __forceinline__ bool union_build(const UnionParams& p, unsigned char* smem, int r, int32_t* ulist,
                                            bool outputs, int& nu_out, uint32_t& err_out) {
  const int H = 1 << p.hash_bits;
  const uint32_t hmask = (uint32_t)H - 1;
  int32_t* key = (int32_t*)smem;          // [H] position, -1 empty
  uint32_t* meta = (uint32_t*)(key + H);  // [H] row mask, then union index
  uint32_t* cnt = meta + H;               // [EU x NW] rank counts
  int* sh = (int*)(cnt + EU * NW);        // [0] error bits
  const int tid = threadIdx.x;
  const int n = p.rows * p.k;
  const int32_t* selr = p.sel + (size_t)r * p.rows * p.kb;
  // Row of each entry by a reciprocal and one correction step (the quotient is below 8192, so
  // the float estimate is off by at most one): no integer division.
  const float rk = __builtin_amdgcn_rcpf((float)p.k);
  const int bmask = (1 << p.bt_shift) - 1;
  int32_t pos[EU], raw[EU];
  int qr[EU], ir[EU];  // row and index of each entry
  // All loads first, unconditionally (an entry past the end reads the list's first one): a load
  // whose value is used inside its own branch is waited for there, one round trip per entry.
#pragma unroll
  for (int j = 0; j < EU; ++j) {
    const int f = j * NT + tid;
    int q = (int)((float)f * rk);
    int i = f - q * p.k;
    if (i < 0) {
      --q;
      i += p.k;
    } else if (i >= p.k) {
      ++q;
      i -= p.k;
    }
    qr[j] = q;
    ir[j] = i;
    // with block selection (bt_shift > 0) entry i is token i & bmask of block i >> bt_shift
    raw[j] = selr[f < n ? (size_t)q * p.kb + (i >> p.bt_shift) : 0];
  }
  // (a request past *num_reqs has its rows in the arrays too, so the loads above stay in bounds)
  const int32_t ctx_r = p.ctx_len[r];
  if (p.num_reqs && r >= *p.num_reqs) return false;
  const int64_t ctx = min((int64_t)ctx_r, p.max_positions);
  uint32_t err = 0;
#pragma unroll
  for (int j = 0; j < EU; ++j) {
    pos[j] = -1;
    if (j * NT + tid >= n) continue;
    const int64_t pos64 = ((int64_t)raw[j] << p.bt_shift) + (ir[j] & bmask);
    if (pos64 < 0 || pos64 >= ctx) err |= HS_ERR_RANGE;
    else pos[j] = (int32_t)pos64;
  }
  {
    u32x4* k4 = (u32x4*)key;
    u32x4* m4 = (u32x4*)meta;
    const u32x4 e4 = {~0u, ~0u, ~0u, ~0u};
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    for (int h = tid; h < H / 4; h += NT) { k4[h] = e4; m4[h] = z4; }
  }
  if (tid == 0) sh[0] = 0;
  __syncthreads();
  // Insertion in two steps, as in RESOLVE's hash: every entry stores its position into its
  // home bucket with a plain store; after a barrier an entry that reads its own position back
  // has its bucket (entries of one position share it), and the others probe from the next
  // bucket with compare-and-swap, which only fills empty buckets.  LDS atomics serialise lane
  // by lane, so this keeps most of the table build off them.
  int32_t bkt[EU];
  uint32_t hh[EU];
#pragma unroll
  for (int j = 0; j < EU; ++j) {
    hh[j] = pos[j] >= 0 ? hash_pos(pos[j], p.hash_bits) : 0u;
    if (pos[j] >= 0) key[hh[j]] = pos[j];
  }
  __syncthreads();
  uint32_t pend = 0;  // entries still probing
#pragma unroll
  for (int j = 0; j < EU; ++j) {
    bkt[j] = -1;
    if (pos[j] < 0) continue;
    if (key[hh[j]] == pos[j]) bkt[j] = (int32_t)hh[j];
    else {
      pend |= 1u << j;
      hh[j] = (hh[j] + 1) & hmask;
    }
  }
  // The probing entries of a thread take one step each per round, their compare-and-swaps
  // issued together.  (The table is at most half full, so every probe sequence meets an empty
  // bucket or its position within H steps.)
  for (int probe = 1; pend != 0 && probe < H; ++probe) {
    int32_t prev[EU];
#pragma unroll
    for (int j = 0; j < EU; ++j) prev[j] = ((pend >> j) & 1u) ? atomicCAS(&key[hh[j]], -1, pos[j]) : 0;
#pragma unroll
    for (int j = 0; j < EU; ++j) {
      if (!((pend >> j) & 1u)) continue;
      if (prev[j] == -1 || prev[j] == pos[j]) {
        bkt[j] = (int32_t)hh[j];
        pend &= ~(1u << j);
      } else {
        hh[j] = (hh[j] + 1) & hmask;
      }
    }
  }
  // Each entry adds 2^16 + 2^row to its bucket's word, with no return value (the LDS takes
  // these in a stream; returning atomics cost a round trip each): the high half counts the
  // bucket's entries, the low half sums their row bits (rows <= 16).  After the barrier the
  // row bits are all distinct -- no duplicate inside a row -- exactly when the low half has as
  // many set bits as the high half counts (a repeated row bit carries, which leaves fewer set
  // bits than entries).  Then an entry is its position's first reference when no earlier
  // row's bit is set.  A bucket with a duplicate makes the request's error, and none of its
  // entries is a first reference.
#pragma unroll
  for (int j = 0; j < EU; ++j)
    if (bkt[j] >= 0) atomicAdd(&meta[bkt[j]], (1u << 16) + (1u << qr[j]));
  __syncthreads();
  uint32_t first = 0;
#pragma unroll
  for (int j = 0; j < EU; ++j) {
    if (bkt[j] < 0) continue;
    const uint32_t mm = meta[bkt[j]];
    if ((uint32_t)__popc(mm & 0xFFFFu) != (mm >> 16)) err |= HS_ERR_DUP;
    else if ((mm & ((1u << qr[j]) - 1u)) == 0) first |= 1u << j;
  }
  if (err) atomicOr((unsigned*)&sh[0], err);
  int ru[EU], nu;
  union_ranks(first, cnt, ru, nu);  // (its barrier also publishes sh[0])
#pragma unroll
  for (int j = 0; j < EU; ++j) {
    if ((first >> j) & 1u) {
      meta[bkt[j]] = (uint32_t)ru[j];
      ulist[ru[j]] = pos[j];
    }
  }
  __syncthreads();
  const uint32_t e = (uint32_t)sh[0];
  if (outputs) {
    int32_t* mapr = p.map + (size_t)r * p.kmax;
#pragma unroll
    for (int j = 0; j < EU; ++j) {
      const int f = j * NT + tid;
      if (f < n) mapr[f] = bkt[j] >= 0 ? (int32_t)meta[bkt[j]] : -1;
    }
    if (tid == 0) {
      p.cnt[r] = e ? 0 : nu;
      p.err[r] = e;
    }
  }
  nu_out = e ? 0 : nu;
  err_out = e;
  return true;
}

__global__ void __launch_bounds__(NT) union_kernel(UnionParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int nu;
  uint32_t err;
  union_build(p, smem, blockIdx.x, p.uni + (size_t)blockIdx.x * p.kmax, true, nu, err);
}

// Speculative rows in one launch (hs_resolve_rows, where its LDS fits): every workgroup of the
// request builds the union of the rows in its own LDS (union_build), resolves it with the list
// read from LDS (resolve_body<.., SL>), and workgroup 0 then gives the rows their slots.
// Against the union kernel followed by resolve_union_kernel: one launch fewer, and the union
// list does not go through global memory.  LDS (rows_lds): the union's table, the list then in
// its first 4 kmax bytes; RESOLVE's carve-up from byte rows_ulist_bytes(kmax) on, once the
// union is built.
template <int E, int KE>
__global__ void __launch_bounds__(NT) resolve_rows_kernel(ResolveParams p, UnionParams u) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int r = blockIdx.x % p.R, g = blockIdx.x / p.R;
  EntryLoads<E> en;
  entry_loads<E>(p, r, en);  // (they land while the union is built)
  int nu = 0;
  uint32_t uerr = 0;
  if (!union_build(u, smem, r, (int32_t*)smem, g == 0, nu, uerr)) {
    // a padded request: untouched, and an empty plan so a replay copies nothing
    if ((p.flags & HS_RECORD_PLAN) && g == 0 && threadIdx.x == 0) p.ctrl[r * 4 + 2] = 0;
    return;
  }
  __syncthreads();  // the union list is complete; the rest of the union's LDS is free
  ReqScalars rs;
  rs.nreq = INT32_MAX;  // (a request past *num_reqs returned above)
  rs.kvr = nu;
  rs.pre_err = uerr;
  const int32_t* ul = (const int32_t*)smem;
  unsigned char* rsm = smem + rows_ulist_bytes(p.k);
  if (nu <= kUnionShortKE * NT) resolve_body<E, kUnionShortKE, false, true>(p, rsm, rs, ul, &en);
  else resolve_body<E, KE, false, true>(p, rsm, rs, ul, &en);
  // (every return in resolve_body is taken by the whole workgroup, so all its threads are here)
  if (g != 0) return;
  rows_scatter(p, r, uerr, true);
}

// Slots of the union back to every (row, entry): out[r][f] = union slot of entry f.
__global__ void __launch_bounds__(256) scatter_kernel(ScatterParams p) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)p.R * p.n) return;
  const int r = (int)(t / p.n), f = (int)(t - (int64_t)r * p.n);
  if (p.num_reqs && r >= *p.num_reqs) return;
  const int32_t u = p.map[(size_t)r * p.kmax + f];
  p.out[t] = (p.err[r] || u < 0) ? -1 : p.uout[(size_t)r * p.kmax + u];
}

template <int E, int KE, bool ATT>
hipError_t launch_e(const ResolveParams& p, size_t lds, hipStream_t s, const KernelTiming* tm) {
  // the fused kernel over FP8 records is a kernel of its own
  if constexpr (ATT) {
    if (p.rec_bytes == kF8RecordBytes) {
      if (tm && tm->start) {
        hipExtLaunchKernelGGL((resolve_f8_kernel<E, KE>), dim3(p.R * p.G), dim3(NT), (uint32_t)lds, s, tm->start,
                              tm->stop, 0u, p);
      } else {
        hipLaunchKernelGGL((resolve_f8_kernel<E, KE>), dim3(p.R * p.G), dim3(NT), lds, s, p);
      }
      return hipGetLastError();
    }
  }
  if (tm && tm->start) {
    hipExtLaunchKernelGGL((resolve_kernel<E, KE, ATT>), dim3(p.R * p.G), dim3(NT), (uint32_t)lds, s, tm->start,
                          tm->stop, 0u, p);
  } else {
    hipLaunchKernelGGL((resolve_kernel<E, KE, ATT>), dim3(p.R * p.G), dim3(NT), lds, s, p);
  }
  return hipGetLastError();
}

// the union kernel (E >= 8: a union longer than kUnionShortKE NT entries needs that many)
template <int E, int KE>
hipError_t launch_union_resolve_e(const ResolveParams& p, size_t lds, hipStream_t s, const KernelTiming* tm) {
  if (tm && tm->start) {
    hipExtLaunchKernelGGL((resolve_union_kernel<E, KE>), dim3(p.R * p.G), dim3(NT), (uint32_t)lds, s, tm->start,
                          tm->stop, 0u, p);
  } else {
    hipLaunchKernelGGL((resolve_union_kernel<E, KE>), dim3(p.R * p.G), dim3(NT), lds, s, p);
  }
  return hipGetLastError();
}
template <int E>
hipError_t launch_union_resolve(const ResolveParams& p, size_t lds, hipStream_t s, int KE, const KernelTiming* tm) {
  static_assert(E >= 8, "a union longer than kUnionShortKE NT entries");
  if (KE <= 8) return launch_union_resolve_e<E, 8>(p, lds, s, tm);
  if constexpr (E >= 16) return launch_union_resolve_e<E, 16>(p, lds, s, tm);
  return hipErrorInvalidValue;
}

template <int E, int KE>
hipError_t launch_rows_e(const ResolveParams& p, const UnionParams& u, size_t lds, hipStream_t s,
                         const KernelTiming* tm) {
  if (tm && tm->start) {
    hipExtLaunchKernelGGL((resolve_rows_kernel<E, KE>), dim3(p.R * p.G), dim3(NT), (uint32_t)lds, s, tm->start,
                          tm->stop, 0u, p, u);
  } else {
    hipLaunchKernelGGL((resolve_rows_kernel<E, KE>), dim3(p.R * p.G), dim3(NT), lds, s, p, u);
  }
  return hipGetLastError();
}
template <int E>
hipError_t launch_rows(const ResolveParams& p, const UnionParams& u, size_t lds, hipStream_t s, int KE,
                       const KernelTiming* tm) {
  static_assert(E >= 8, "a union longer than kUnionShortKE NT entries");
  if (KE <= 8) return launch_rows_e<E, 8>(p, u, lds, s, tm);
  if constexpr (E >= 16) return launch_rows_e<E, 16>(p, u, lds, s, tm);
  return hipErrorInvalidValue;
}

// The fused variant exists for KE <= 4 and E <= 8 (top_k <= 4096, B <= 8192): larger lists
// leave no LDS for the record tile.
constexpr int kFusedMaxE = 8, kFusedMaxKE = 4;

template <int E, bool ATT>
hipError_t launch_ke(const ResolveParams& p, size_t lds, hipStream_t s, int KE, const KernelTiming* tm) {
  if constexpr (ATT && E > kFusedMaxE) {
    return hipErrorInvalidValue;
  } else {
    if constexpr (E >= 1) if (KE <= 1) return launch_e<E, 1, ATT>(p, lds, s, tm);
    if constexpr (E >= 2) if (KE <= 2) return launch_e<E, 2, ATT>(p, lds, s, tm);
    if constexpr (E >= 4) if (KE <= 4) return launch_e<E, 4, ATT>(p, lds, s, tm);
    if constexpr (!ATT && E >= 8) if (KE <= 8) return launch_e<E, 8, ATT>(p, lds, s, tm);
    if constexpr (!ATT && E >= 16) return launch_e<E, 16, ATT>(p, lds, s, tm);
    return hipErrorInvalidValue;
  }
}

// Maximum dynamic LDS of a kernel: the device's per-block LDS less the kernel's static LDS.
hipError_t set_dynamic_lds(const void* fn, int v) {
  hipFuncAttributes a;
  hipError_t e = hipFuncGetAttributes(&a, fn);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, v - (int)a.sharedSizeBytes);
}

template <int E>
hipError_t set_limit_ke(int v) {
  hipError_t e = hipSuccess;
  if constexpr (E >= 1) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_kernel<E, 1, false>, v);
  if constexpr (E >= 2) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_kernel<E, 2, false>, v);
  if constexpr (E >= 4) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_kernel<E, 4, false>, v);
  if constexpr (E >= 8) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_kernel<E, 8, false>, v);
  if constexpr (E >= 16) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_kernel<E, 16, false>, v);
  if constexpr (E >= 8) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_union_kernel<E, 8>, v);
  if constexpr (E >= 16) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_union_kernel<E, 16>, v);
  if constexpr (E >= 8) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_rows_kernel<E, 8>, v);
  if constexpr (E >= 16) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_rows_kernel<E, 16>, v);
  if constexpr (E <= kFusedMaxE) {
    if constexpr (E >= 1) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_kernel<E, 1, true>, v);
    if constexpr (E >= 2) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_kernel<E, 2, true>, v);
    if constexpr (E >= 4) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_kernel<E, 4, true>, v);
    if constexpr (E >= 1) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_f8_kernel<E, 1>, v);
    if constexpr (E >= 2) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_f8_kernel<E, 2>, v);
    if constexpr (E >= 4) if (e == hipSuccess) e = set_dynamic_lds((const void*)resolve_f8_kernel<E, 4>, v);
  }
  return e;
}

}  // namespace

int resolve_elems_per_thread(int k, int B) {
  const int n = (k > B ? k : B);
  const int e = (n + NT - 1) / NT;
  // 12 slots per thread for 8192 < B <= 12288 (with at most 8 list entries per thread): the
  // power of two 16 would leave a quarter or more of the threads without slots and every
  // thread's slot arrays a third larger
  if (e > 8 && e <= 12 && k <= 8 * NT) return 12;
  int E = 1;
  while (E < e) E <<= 1;
  return E;
}

static int pow2_at_least(int x) {
  int v = 1;
  while (v < x) v <<= 1;
  return v;
}

hipError_t set_resolve_lds_limit(size_t lds_bytes) {
  const int v = (int)lds_bytes;
  hipError_t e;
  if ((e = set_limit_ke<1>(v)) != hipSuccess) return e;
  if ((e = set_limit_ke<2>(v)) != hipSuccess) return e;
  if ((e = set_limit_ke<4>(v)) != hipSuccess) return e;
  if ((e = set_limit_ke<8>(v)) != hipSuccess) return e;
  if ((e = set_limit_ke<12>(v)) != hipSuccess) return e;
  return set_limit_ke<16>(v);
}


hipError_t set_union_lds_limit(size_t lds_bytes) {
  return set_dynamic_lds((const void*)union_kernel, (int)lds_bytes);
}

hipError_t launch_union(const UnionParams& p, hipStream_t s) {
  hipLaunchKernelGGL(union_kernel, dim3(p.R), dim3(NT), union_lds_bytes(p.hash_bits), s, p);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.R * p.n;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_resolve(const ResolveParams& p, size_t lds_bytes, hipStream_t s, const KernelTiming* tm) {
  const int KE = pow2_at_least((p.k + NT - 1) / NT);
  const int E = resolve_elems_per_thread(p.k, p.B);
  // A speculative union longer than kUnionShortKE entries per thread at capacity: the union
  // kernel, which also writes the rows' slots (KE > kUnionShortKE puts E at 8 or more)
  if (p.rows_out && KE > kUnionShortKE) {
    switch (E) {
      case 8: return launch_union_resolve<8>(p, lds_bytes, s, KE, tm);
      case 12: return launch_union_resolve<12>(p, lds_bytes, s, KE, tm);
      default: return launch_union_resolve<16>(p, lds_bytes, s, KE, tm);
    }
  }
  hipError_t e;
  switch (E) {
    case 1: e = launch_ke<1, false>(p, lds_bytes, s, KE, tm); break;
    case 2: e = launch_ke<2, false>(p, lds_bytes, s, KE, tm); break;
    case 4: e = launch_ke<4, false>(p, lds_bytes, s, KE, tm); break;
    case 8: e = launch_ke<8, false>(p, lds_bytes, s, KE, tm); break;
    case 12: e = launch_ke<12, false>(p, lds_bytes, s, KE, tm); break;
    default: e = launch_ke<16, false>(p, lds_bytes, s, KE, tm); break;
  }
  if (e != hipSuccess || !p.rows_out) return e;
  // a short union: the rows' slots by a kernel of their own
  ScatterParams c{};
  c.uout = p.out; c.map = p.rows_map; c.err = p.kerr; c.num_reqs = p.num_reqs; c.out = p.rows_out; c.R = p.R;
  c.n = p.rows_n; c.kmax = p.k;
  return launch_scatter(c, s);
}

hipError_t launch_resolve_rows(const ResolveParams& p, const UnionParams& u, size_t lds_bytes, hipStream_t s,
                               const KernelTiming* tm) {
  const int KE = pow2_at_least((p.k + NT - 1) / NT);
  if (!p.rows_out || KE <= kUnionShortKE) return hipErrorInvalidValue;
  switch (resolve_elems_per_thread(p.k, p.B)) {
    case 8: return launch_rows<8>(p, u, lds_bytes, s, KE, tm);
    case 12: return launch_rows<12>(p, u, lds_bytes, s, KE, tm);
    default: return launch_rows<16>(p, u, lds_bytes, s, KE, tm);
  }
}

bool fused_supported(int k, int B) {
  return resolve_elems_per_thread(k, B) <= kFusedMaxE && pow2_at_least((k + NT - 1) / NT) <= kFusedMaxKE;
}

hipError_t launch_resolve_attn(const ResolveParams& p, size_t lds_bytes, hipStream_t s, const KernelTiming* tm) {
  const int KE = pow2_at_least((p.k + NT - 1) / NT);
  switch (resolve_elems_per_thread(p.k, p.B)) {
    case 1: return launch_ke<1, true>(p, lds_bytes, s, KE, tm);
    case 2: return launch_ke<2, true>(p, lds_bytes, s, KE, tm);
    case 4: return launch_ke<4, true>(p, lds_bytes, s, KE, tm);
    case 8: return launch_ke<8, true>(p, lds_bytes, s, KE, tm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hs
