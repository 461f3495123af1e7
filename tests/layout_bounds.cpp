// Host-side bounds check of the LDS carve-ups and per-wave capacities the kernels index, for
// every configuration shape the library accepts (built with hipcc as a host program; it
// calls no HIP API).  It includes the kernels' own layout header, so it checks the offsets
// the kernels use, not a copy of them.  Exit status 0: every check held; otherwise the first
// failing check is printed.
#include <cstdio>
#include <cstdlib>

#include "../hierarchical_kv_cache_amd/csrc/hs_internal.h"

using namespace hs;

static long checks = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    ++checks;                                              \
    if (!(cond)) {                                         \
      std::printf("FAILED %s: ", #cond);                   \
      std::printf(__VA_ARGS__);                            \
      std::printf("\n");                                   \
      std::exit(1);                                        \
    }                                                      \
  } while (0)

constexpr size_t kLdsMax = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int NT = kResolveThreads, NW = NT / 64;

static size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }

// RESOLVE's carve-up: the hash and the per-miss arrays that reuse its bytes, then the
// per-entry positions, the slot owners, the per-wave miss lists and the scan scratch.
static void check_resolve(int k, int B, int bits, int G) {
  const ResolveLds L = resolve_lds(k, B, bits, G);
  const size_t H = size_t(1) << bits;
  // stage 3's per-miss arrays (victim, missidx, mrank: int16 per list entry) inside the hash's
  // bytes or below selp, in order
  CHECK(L.victim == 0 && L.missidx >= L.victim + 2 * size_t(k) && L.mrank >= L.missidx + 2 * size_t(k),
        "k %d B %d bits %d G %d", k, B, bits, G);
  CHECK(L.selp >= L.mrank + 2 * size_t(k) && L.selp >= 4 * H, "k %d B %d bits %d G %d", k, B, bits, G);
  // the table is cleared as 16-byte words: H / 4 of them
  CHECK(H % 4 == 0 && 16 * (H / 4) <= L.selp, "bits %d", bits);
  CHECK(L.sown >= L.selp + 4 * size_t(k), "k %d", k);
  // the owner array is cleared as 16-byte words: ceil(B / 8) of them
  CHECK(L.wpos >= L.sown + 16 * ceil_div(B, 8), "B %d", B);
  CHECK(L.widx >= L.wpos + 4 * size_t(NW) * L.wcap, "G %d", G);
  CHECK(L.scratch >= L.widx + 2 * size_t(NW) * L.wcap, "G %d", G);
  // scan carries (2 x 2 x NW), per-wave resident counts (NW), six shared words
  CHECK(L.total >= L.scratch + 4 * size_t(4 * NW + NW + 6), "total");
  for (size_t o : {L.missidx, L.mrank, L.selp, L.sown, L.wpos, L.widx, L.scratch})
    CHECK(o % 16 == 0, "offset %zu aligned", o);
  // per-wave miss lists: a fetch workgroup's wave owns share entries e = q NT + lane NW + wid,
  // at most ceil(f_n / NW) of them; a one-workgroup launch's wave its lanes' own entries, at
  // most 64 ceil(kr / NT)
  const int nf = G > 1 ? G - 1 : 1;
  for (int kr : {1, k / 3 + 1, k - 1, k}) {
    if (kr < 1) continue;
    for (int gf = 0; gf < nf; ++gf) {
      const int f_lo = (int)((long long)kr * gf / nf), f_n = (int)((long long)kr * (gf + 1) / nf) - f_lo;
      CHECK(ceil_div(f_n, NW) <= L.wcap, "k %d kr %d G %d share %d wcap %zu", k, kr, G, f_n, L.wcap);
    }
    if (G == 1) CHECK(64 * ceil_div(kr, NT) <= L.wcap, "k %d kr %d wcap %zu", k, kr, L.wcap);
  }
}

// The attention scratch: the heads' maxima and sums, the partial scores, P (NB variants of hi
// and lo), the FP8 block scales; the largest index each step of attend_tile forms.
static void check_attention_scratch() {
  const int spart_off = 2 * 16 * 4;
  int hi = 0;
  for (int kp = 0; kp < 4; ++kp)
    for (int tb = 0; tb < 4; ++tb)
      for (int h = 0; h < 16; ++h)
        for (int col = 0; col < 16; ++col) {
          const int i = (kp * 4 + tb) * kSpartTB + h * kSpartRow + col;
          hi = i > hi ? i : hi;
        }
  CHECK(spart_off + 4 * (hi + 1) <= kAttnSpart + spart_off, "partial scores %d", hi);
  CHECK(kAttnPOff >= spart_off + kAttnSpart, "P after the partial scores");
  for (int NB : {1, 4}) {
    // P hi at [b][2 token halves][16 heads][kPRow] (k index < 32), P lo after NB of them
    const int p_hi_last = ((NB - 1) * 2 + 1) * 16 * kPRow + 15 * kPRow + 31;
    const int p_lo_last = NB * 2 * 16 * kPRow + p_hi_last;
    CHECK(kAttnPOff + 2 * (p_lo_last + 1) <= kAttnPOff + NB * kAttnPVariant, "P of %d variants", NB);
    // the P operand reads: 8 bf16 from (pb 16 + col) kPRow + 8 qd, pb < 2 NB
    CHECK(2 * ((2 * NB - 1) * 16 * kPRow + 15 * kPRow + 3 * 8 + 8) <= NB * kAttnPVariant / 2, "P reads %d", NB);
  }
  CHECK(kAttnScratch == kAttnPOff + kAttnPVariant, "bf16 scratch");
  CHECK(kAttnScales8Off >= kAttnPOff + 4 * kAttnPVariant && kAttnScratch8 >= kAttnScales8Off + 64 * 4 * 4,
        "FP8 scales after the four P variants");
  // the tile: 64 rows at kTileStride, a 1152-byte record and the transposed V reads (8 bytes
  // at channel c0 + 4 (s % 4) of rows < 64) inside a row
  CHECK(kTileStride >= 1152 && kTileStride % 8 == 0 && kQStride >= 1152 && kQStride % 16 == 0, "strides");
  // the attention kernel's static LDS: tile, query rows, scratch, chunk addresses
  for (int f8 = 0; f8 < 2; ++f8) {
    const size_t lds = size_t(kTileRows) * kTileStride + 16 * size_t(kQStride) +
                       (f8 ? kAttnScratch8 : kAttnScratch) + 8 * size_t(kAttnMaxChunk);
    CHECK(lds <= kLdsMax, "attention kernel LDS %zu", lds);
  }
}

int main() {
  // top_k and buffer sizes the library takes (k <= 16384 with B >= k; speculative unions up to
  // kUnionMaxEntries entries), workgroups per request 1 .. 32, hash sizes from a half-full
  // table up (the library picks 4k entries, or 2k when LDS is short)
  const int ks[] = {1, 2, 3, 64, 100, 513, 1000, 2048, 2650, 4096, 5000, 8192, 12000, 16384};
  const int Bs[] = {2, 3, 4, 6, 8, 64, 128, 1040, 2048, 4096, 5120, 8192, 10240, 12000, 12288, 16384};
  long fits = 0;
  for (int k : ks)
    for (int B : Bs) {
      if (B < k) continue;
      for (int G = 1; G <= 33; ++G) {
        int bits = 6;
        while ((size_t(1) << bits) < 2 * size_t(k)) ++bits;
        for (int b = bits; b <= bits + 1; ++b) {
          check_resolve(k, B, b, G);
          if (resolve_lds(k, B, b, G).total <= kLdsMax) ++fits;
        }
      }
    }
  // the speculative rows of the pages' default: 4 rows of k 2048 into B = 5 k, 32 workgroups
  // (one request): the union's RESOLVE fits with a table of 2 kmax or 4 kmax entries
  {
    const int kmax = 4 * 2048, B = 10240;
    const ResolveLds L = resolve_lds(kmax, B, 14, 32);
    CHECK(L.total <= kLdsMax, "rows RESOLVE LDS %zu", L.total);
    // the union kernel: key and meta per bucket, a table at most half full, the scan scratch
    int bits = 6;
    while ((size_t(1) << bits) < 2 * size_t(kmax)) ++bits;
    CHECK(union_lds_bytes(bits) <= kLdsMax && (size_t(1) << bits) >= 2 * size_t(kUnionMaxEntries),
          "union LDS %zu", union_lds_bytes(bits));
    // the union kernel's entries: EU slots per thread cover every entry, and after the table its
    // rank counts (one per slot and wave) and the shared error word
    CHECK(size_t(kUnionMaxEntries / NT) * NT >= size_t(kUnionMaxEntries), "union entries per thread");
    CHECK(union_lds_bytes(bits) >= (size_t(8) << bits) + 4 * (size_t(kUnionMaxEntries / NT) * NW + 1),
          "union rank counts");
  }
  // the one-launch rows kernel: for every union capacity past kUnionShortKE entries per thread
  // and every buffer size, where its LDS fits (the library takes it only then), the union list
  // (4 kmax bytes) lies inside the union table's position array (4 H bytes, H >= 2 kmax), which
  // is dead once the list is written, and RESOLVE's carve-up starts after the list
  for (int kmax : {4097, 6144, 8192})
    for (int B : Bs) {
      if (B < kmax) continue;
      for (int G = 1; G <= 33; ++G) {
        int ubits = 6;
        while ((size_t(1) << ubits) < 2 * size_t(kmax)) ++ubits;
        int rbits = 6;
        while ((size_t(1) << rbits) < 4 * size_t(kmax)) ++rbits;
        for (int b = rbits - 1; b <= rbits; ++b) {
          const size_t lds = rows_lds(kmax, B, b, G, ubits);
          if (lds > kLdsMax) continue;
          CHECK(rows_ulist_bytes(kmax) >= 4 * size_t(kmax) && rows_ulist_bytes(kmax) % 16 == 0 &&
                    rows_ulist_bytes(kmax) <= (size_t(4) << ubits),
                "rows list kmax %d", kmax);
          CHECK(lds >= rows_ulist_bytes(kmax) + resolve_lds(kmax, B, b, G).total && lds >= union_lds_bytes(ubits),
                "rows LDS kmax %d B %d G %d", kmax, B, G);
          check_resolve(kmax, B, b, G);
        }
      }
    }
  {
    // the pages' default shape takes the one-launch kernel: 4 rows of 2048 into B = 5 k, 32
    // workgroups, with the table size the library picks (4 kmax entries, or 2 kmax when short)
    int b = 15;
    if (resolve_lds(8192, 10240, b, 32).total > kLdsMax) --b;
    const size_t lds = rows_lds(8192, 10240, b, 32, 14);
    CHECK(lds <= kLdsMax, "rows kernel LDS %zu at 4 x 2048 into B 10240", lds);
  }
  // the fused kernel: the fetch workgroups' tile, query rows and scratch
  for (int f8 = 0; f8 < 2; ++f8) {
    const FusedLds F = fused_lds(2048, 4096, 13, 33, 1, f8 != 0);
    CHECK(F.qs >= F.tile + size_t(kTileRows) * kTileStride && F.scratch >= F.qs + 16 * size_t(kQStride),
          "fused carve-up");
    CHECK(F.total >= F.scratch + (f8 ? kAttnScratch8 : kAttnScratch) && F.total <= kLdsMax, "fused LDS %zu",
          F.total);
  }
  check_attention_scratch();
  std::printf("ok: %ld checks, %ld resolve layouts within %zu bytes\n", checks, fits, kLdsMax);
  return 0;
}
