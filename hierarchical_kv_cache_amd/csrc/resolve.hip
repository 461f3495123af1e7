// RESOLVE: one fused kernel per layer turns the k selected logical positions
// of every request into physical slots of that request's hot buffer.
//
// Stages ("HiSparse 深度解析" (gentlecold.top) §3.5; "推理系统基础设施手记（六）：
// HiSparse" (naphjohn.github.io) §3):
//   1 stage    selected positions -> LDS open-addressing hash (Knuth
//              multiplicative hash, compare-and-swap insertion)
//   2 mark     every slot's stored position probed in the hash: hit or evictable
//   3 scan     wave64 ballot/popcount ranks: misses numbered in list order,
//              evictable slots numbered in LRU order, the j-th evictable is the
//              victim of the j-th miss; new LRU order = untouched evictables (old
//              order), then filled victims, then hits (§3.3: hits rank newer)
//   4 fetch    missed records copied from pinned host memory with 16-byte
//              non-temporal loads, flattened over (miss, 16-byte chunk)
//   5 publish  page table, slot map, slots aligned with the selection order
//
// MI355X layout of the work.  G workgroups serve one request.  Each of them
// recomputes stages 1-3 from the current metadata (cheap, all in LDS) and
// copies its 1/G share of the missed bytes, so that a single request can
// keep enough loads in flight to fill the host link; only workgroup 0 writes
// the new metadata.  The slot map and the LRU order are ping-ponged: readers
// use half `epoch & 1`, workgroup 0 writes the other half, and the last
// workgroup of a request to arrive flips the epoch.  No workgroup ever waits
// on another.
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int NT = kResolveThreads;
constexpr int NW = NT / 64;
constexpr int32_t kEmpty = -1;
constexpr int kUnroll = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t hash_pos(int32_t pos, int bits) {
  return ((uint32_t)pos * 2654435761u) >> (32 - bits);  // Knuth multiplicative hash
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// Exclusive block-wide ranks of flags.  Element e = p * NT + threadIdx.x for
// pass p < P; bit p of fbits is its flag.  rank[p] gets the number of set
// flags at smaller e.  Returns the total.  Contains barriers: every thread of
// the workgroup must call it.
__device__ int block_ranks(uint32_t fbits, int P, int (&rank)[kMaxScanPasses], int* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int p = 0; p < kMaxScanPasses; ++p) {
    if (p < P) {
      const uint64_t m = __ballot((fbits >> p) & 1u);
      rank[p] = __popcll(m & lt);
      if (lane == 0) scratch[p * NW + wid] = __popcll(m);
    }
  }
  __syncthreads();
  if (wid == 0) {
    // exclusive scan of the n = P * NW wave counts, four per lane (n <= 256)
    const int n = P * NW;
    int v[4], s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = lane * 4 + j;
      v[j] = idx < n ? scratch[idx] : 0;
      s += v[j];
    }
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    int run = incl - s;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = lane * 4 + j;
      if (idx < n) scratch[idx] = run;
      run += v[j];
    }
    if (lane == 63) scratch[kMaxScanPasses * NW] = incl;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kMaxScanPasses; ++p)
    if (p < P) rank[p] += scratch[p * NW + wid];
  const int total = scratch[kMaxScanPasses * NW];
  __syncthreads();
  return total;
}

__global__ void __launch_bounds__(NT) resolve_kernel(ResolveParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const ResolveLds Ly = resolve_lds(p.k, p.B, p.hash_bits);
  int32_t* hkey = (int32_t*)(smem + Ly.hkey);        // [H] selected positions (keys)
  int32_t* selp = (int32_t*)(smem + Ly.selp);        // [k] expanded selection
  int32_t* selslot = (int32_t*)(smem + Ly.selslot);  // [k] >= 0 slot of a hit, -1 miss
  int16_t* hval = (int16_t*)(smem + Ly.hval);        // [H] list index of each key
  int16_t* victim = (int16_t*)(smem + Ly.victim);    // [k] slot given to miss j
  int16_t* missidx = (int16_t*)(smem + Ly.missidx);  // [k] list index of miss j
  uint8_t* sflag = (uint8_t*)(smem + Ly.sflag);      // [B] 0 evictable, 1 hit, 2 victim
  int* scratch = (int*)(smem + Ly.scratch);          // scan carries + shared scalars
  int* sh = scratch + kMaxScanPasses * NW + 1;       // [0] epoch [1] error bits [2] newest hits

  const int tid = threadIdx.x;
  const int r = blockIdx.x % p.R;
  const int g = blockIdx.x / p.R;
  const bool record = (p.flags & HS_RECORD_PLAN) != 0;
  if (p.num_reqs && r >= *p.num_reqs) {
    // a padded request: untouched, and an empty plan so a replay copies nothing
    if (record && g == 0 && tid == 0) p.ctrl[r * 4 + 2] = 0;
    return;
  }
  const int H = 1 << p.hash_bits;
  const uint32_t hmask = (uint32_t)H - 1;

  if (tid == 0) {
    sh[0] = (int)__hip_atomic_load(&p.ctrl[r * 4], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    sh[1] = 0;
    sh[2] = 0;
  }
  for (int h = tid; h < H; h += NT) hkey[h] = kEmpty;
  __syncthreads();

  const uint32_t epoch = (uint32_t)sh[0];
  const int cur = epoch & 1, nxt = cur ^ 1;
  const int32_t* sp_old = p.slot_pos + ((size_t)r * 2 + cur) * p.B;
  int32_t* sp_new = p.slot_pos + ((size_t)r * 2 + nxt) * p.B;
  const int16_t* lru_old = p.lru + ((size_t)r * 2 + cur) * p.Bpad;
  int16_t* lru_new = p.lru + ((size_t)r * 2 + nxt) * p.Bpad;
  const int32_t newest = (p.flags & kHasNewest) ? p.newest[r] : -1;
  const int64_t ctx = min((int64_t)p.ctx_len[r], p.max_positions);

  // ---- stage 1: expand blocks, validate, hash the selected positions ----
  uint32_t err = 0;
  const int32_t* selr = p.sel + (size_t)r * p.kb;
  for (int i = tid; i < p.k; i += NT) {
    int64_t pos64;
    if (p.bt_shift) {
      const int32_t b = selr[i >> p.bt_shift];
      pos64 = ((int64_t)b << p.bt_shift) + (i & ((1 << p.bt_shift) - 1));
    } else {
      pos64 = selr[i];
    }
    if (pos64 < 0 || pos64 >= ctx) {
      err |= HS_ERR_RANGE;
      selp[i] = -1;
      selslot[i] = -2;
      continue;
    }
    const int32_t pos = (int32_t)pos64;
    selp[i] = pos;
    if (pos == newest) {  // the newest token sits in slot B, outside the LRU
      selslot[i] = p.B;
      atomicAdd(&sh[2], 1);
      continue;
    }
    selslot[i] = -1;
    uint32_t h = hash_pos(pos, p.hash_bits);
    while (true) {  // the table has >= H/2 empty entries, so the probe ends
      const int32_t prev = atomicCAS(&hkey[h], kEmpty, pos);
      if (prev == kEmpty) {
        hval[h] = (int16_t)i;
        break;
      }
      if (prev == pos) {
        err |= HS_ERR_DUP;
        break;
      }
      h = (h + 1) & hmask;
    }
  }
  if (err) atomicOr((unsigned*)&sh[1], err);
  __syncthreads();
  err = (uint32_t)sh[1] | (sh[2] > 1 ? HS_ERR_DUP : 0u);
  if (err) {  // every workgroup of the request sees the same error: nothing changes
    if (g == 0) {
      for (int i = tid; i < p.k; i += NT) p.out[(size_t)r * p.k + i] = -1;
      if (tid == 0 && p.stats) {
        hs_stats st = {0u, 0u, err, 0u};
        p.stats[r] = st;
      }
      if (tid == 0 && record) p.ctrl[r * 4 + 2] = 0;
    }
    return;
  }
  if (tid == 0) {
    // every workgroup has read the epoch; the last one to arrive flips it for the next launch
    const uint32_t arrived =
        __hip_atomic_fetch_add(&p.ctrl[r * 4 + 1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (arrived == (uint32_t)p.G - 1) {
      __hip_atomic_store(&p.ctrl[r * 4 + 1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.ctrl[r * 4], epoch + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- stage 2: mark each slot hit (its position is selected) or evictable ----
  const int PB = (p.B + NT - 1) / NT;
  for (int s = tid; s < p.B; s += NT) {
    const int32_t ps = sp_old[s];
    uint8_t f = 0;
    if (ps >= 0) {
      uint32_t h = hash_pos(ps, p.hash_bits);
      int32_t key;
      while ((key = hkey[h]) != kEmpty) {
        if (key == ps) {
          selslot[hval[h]] = s;
          f = 1;
          break;
        }
        h = (h + 1) & hmask;
      }
    }
    sflag[s] = f;
  }
  __syncthreads();

  // ---- stage 3: misses in list order, evictables in LRU order, victims ----
  int rk[kMaxScanPasses];
  const int PK = (p.k + NT - 1) / NT;
  uint32_t fb = 0;
#pragma unroll
  for (int q = 0; q < kMaxScanPasses; ++q) {
    const int i = q * NT + tid;
    if (q < PK && i < p.k && selslot[i] == -1) fb |= 1u << q;
  }
  const int m = block_ranks(fb, PK, rk, scratch);
#pragma unroll
  for (int q = 0; q < kMaxScanPasses; ++q)
    if ((fb >> q) & 1u) missidx[rk[q]] = (int16_t)(q * NT + tid);

  int16_t lslot[kMaxScanPasses];
  fb = 0;
#pragma unroll
  for (int q = 0; q < kMaxScanPasses; ++q) {
    const int e = q * NT + tid;
    lslot[q] = 0;
    if (q < PB && e < p.B) {
      lslot[q] = lru_old[e];
      if (sflag[lslot[q]] == 0) fb |= 1u << q;
    }
  }
  const int E = block_ranks(fb, PB, rk, scratch);
#pragma unroll
  for (int q = 0; q < kMaxScanPasses; ++q) {
    if ((fb >> q) & 1u) {
      if (rk[q] < m) {
        victim[rk[q]] = lslot[q];
        sflag[lslot[q]] = 2;
      } else if (g == 0) {
        lru_new[rk[q] - m] = lslot[q];  // untouched evictables keep their old order
      }
    }
  }
  __syncthreads();

  if (g == 0) {
    // filled victims then hits, each group by slot index, after the untouched evictables
    uint32_t fv = 0, fh = 0;
#pragma unroll
    for (int q = 0; q < kMaxScanPasses; ++q) {
      const int s = q * NT + tid;
      if (q < PB && s < p.B) {
        const uint8_t f = sflag[s];
        if (f == 2) fv |= 1u << q;
        if (f == 1) fh |= 1u << q;
      }
    }
    int rv[kMaxScanPasses];
    block_ranks(fv, PB, rv, scratch);
    block_ranks(fh, PB, rk, scratch);
#pragma unroll
    for (int q = 0; q < kMaxScanPasses; ++q) {
      const int s = q * NT + tid;
      if ((fv >> q) & 1u) lru_new[E - m + rv[q]] = (int16_t)s;
      if ((fh >> q) & 1u) lru_new[E + rk[q]] = (int16_t)s;
    }

    // ---- stage 5: publish ----
    int32_t* pt = p.page_table + (size_t)r * p.max_positions;
    int32_t* outr = p.out + (size_t)r * p.k;
    int32_t* plan_pos = p.plan + (size_t)r * 2 * p.k;
    int32_t* plan_slot = plan_pos + p.k;
    for (int j = tid; j < m; j += NT) {
      const int i = missidx[j];
      const int v = victim[j];
      const int32_t pos = selp[i];
      const int32_t old = sp_old[v];
      if (old >= 0) pt[old] = -1;  // evicted position: host only again
      pt[pos] = v;
      sp_new[v] = pos;
      outr[i] = v;
      if (record) {
        plan_pos[j] = pos;
        plan_slot[j] = v;
      }
    }
    for (int i = tid; i < p.k; i += NT) {
      const int s = selslot[i];
      if (s >= 0) outr[i] = s;
    }
    for (int s = tid; s < p.B; s += NT)
      if (sflag[s] != 2) sp_new[s] = sp_old[s];
    if (tid == 0) {
      if (p.stats) {
        hs_stats st = {(uint32_t)(p.k - m), (uint32_t)m, 0u, 0u};
        p.stats[r] = st;
      }
      if (record) p.ctrl[r * 4 + 2] = (uint32_t)m;
    }
  }

  // ---- stage 4: fetch the missed records from pinned host memory ----
  if (!(p.flags & HS_SKIP_IO) && m > 0) {
    const uint8_t* hbase = p.host_base[r] + p.host_layer_off;
    uint8_t* dbase = p.hot + (size_t)r * p.hot_req_stride + p.hot_layer_off;
    const int C = p.rec_bytes >> 4;  // 16-byte chunks per record
    const float invC = 1.0f / (float)C;
    const int total = m * C;  // <= 2^24: exact in float
    const int stride = p.G * NT;
    for (int f0 = g * NT + tid; f0 < total; f0 += stride * kUnroll) {
      u32x4 v[kUnroll];
      int jj[kUnroll], cc[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int f = f0 + u * stride;
        if (f < total) {
          int j = (int)((float)f * invC);
          int c = f - j * C;
          if (c < 0) { --j; c += C; }
          if (c >= C) { ++j; c -= C; }
          jj[u] = j;
          cc[u] = c;
          const u32x4* src =
              (const u32x4*)(hbase + (size_t)selp[missidx[j]] * (size_t)p.rec_bytes) + c;
          v[u] = __builtin_nontemporal_load(src);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (f0 + u * stride < total) {
          u32x4* dst = (u32x4*)(dbase + (size_t)victim[jj[u]] * (size_t)p.rec_bytes) + cc[u];
          *dst = v[u];
        }
      }
    }
  }
}

}  // namespace

hipError_t set_resolve_lds_limit(size_t lds_bytes) {
  return hipFuncSetAttribute((const void*)resolve_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
}

hipError_t launch_resolve(const ResolveParams& p, size_t lds_bytes, hipStream_t s) {
  hipLaunchKernelGGL(resolve_kernel, dim3(p.R * p.G), dim3(NT), lds_bytes, s, p);
  return hipGetLastError();
}

}  // namespace hs
