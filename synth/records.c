/*
 * Seeded synthetic inputs shared by the oracle and the HIP path.
 *
 * This file holds no part of the cache method: it only produces the bytes of
 * KV records and query vectors.  Every value is a function of a counter, so
 * any record can be regenerated on its own, in any order, on any thread.
 *
 * Definition (stated once, used everywhere):
 *   key(seed, a, b, c)   = mix(mix(mix(seed ^ G) ^ (a*G2 + b)) ^ c)
 *   z_n                  = mix(key + (n + 1) * G)          (SplitMix64 stream)
 *   u1 = (hi32(z_n) + 0.5) / 2^32,  u2 = (lo32(z_n) + 0.5) / 2^32
 *   element 2n   = sqrt(-2 ln u1) * cos(2 pi u2)            (Box-Muller 1958)
 *   element 2n+1 = sqrt(-2 ln u1) * sin(2 pi u2)
 *   each element is rounded double -> float -> bfloat16 (round to nearest even)
 * with mix() the SplitMix64 finaliser (Steele, Lea, Flood 2014) and
 * G = 0x9E3779B97F4A7C15.  For a KV record (a, b, c) = (request, layer,
 * position); for a query vector (a, b, c) = (request, layer, step).
 *
 * FP8 records (656 bytes, the layout of an fp8 latent KV cache): the same 576
 * draws, rounded double -> float; the first 512 are stored as OCP FP8 E4M3
 * codes in four blocks of 128, each with a float32 scale = (block max |x|) /
 * 448, code = round-to-nearest-even(x / scale) (saturated at 448); the last 64
 * as bfloat16.  Layout: [512 codes][4 float32 scales][64 bf16].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL
#define G2 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t record_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c) {
  return mix64(mix64(mix64(seed ^ GOLDEN) ^ (a * G2 + b)) ^ c);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t rounding = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + rounding) >> 16);
}

/* Writes `nelem` bf16 values (nelem even) of the stream for `key` into dst. */
static void fill_stream(uint16_t* dst, uint64_t key, int64_t nelem) {
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t n = 0; n < nelem / 2; ++n) {
    uint64_t z = mix64(key + (uint64_t)(n + 1) * GOLDEN);
    double u1 = ((double)(z >> 32) + 0.5) * (1.0 / 4294967296.0);
    double u2 = ((double)(z & 0xFFFFFFFFULL) + 0.5) * (1.0 / 4294967296.0);
    double rad = sqrt(-2.0 * log(u1));
    dst[2 * n] = f32_to_bf16_rne((float)(rad * cos(two_pi * u2)));
    dst[2 * n + 1] = f32_to_bf16_rne((float)(rad * sin(two_pi * u2)));
  }
}

/* One record (or query vector) identified by (a, b, c). */
void synth_one(uint16_t* dst, uint64_t seed, int64_t a, int64_t b, int64_t c, int64_t nelem) {
  fill_stream(dst, record_key(seed, (uint64_t)a, (uint64_t)b, (uint64_t)c), nelem);
}

/* OCP FP8 E4M3 code of v (|v| <= 448 after scaling), round to nearest even. */
static uint8_t e4m3_rne(float v) {
  uint8_t sign = v < 0.0f ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a >= 448.0) return sign | 0x7E; /* largest finite */
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): a in [2^(e-1), 2^e) */
  int ex = e - 1; /* a in [2^ex, 2^(ex+1)) */
  if (a == 0.0 || ex < -6) {
    double q = nearbyint(a / ldexp(1.0, -9)); /* subnormal steps of 2^-9 (ties to even) */
    if (q >= 8.0) return sign | 0x08;          /* rounds up to the smallest normal */
    return sign | (uint8_t)q;
  }
  double m = nearbyint((a / ldexp(1.0, ex) - 1.0) * 8.0);
  if (m >= 8.0) { m = 0.0; ++ex; }
  if (ex > 8 || (ex == 8 && m > 6.0)) return sign | 0x7E;
  return sign | (uint8_t)(((ex + 7) << 3) | (int)m);
}

/* One FP8 record (656 bytes) identified by (a, b, c). */
void synth_one_fp8(uint8_t* dst, uint64_t seed, int64_t a, int64_t b, int64_t c) {
  const double two_pi = 6.283185307179586476925286766559;
  const uint64_t key = record_key(seed, (uint64_t)a, (uint64_t)b, (uint64_t)c);
  float x[576];
  for (int n = 0; n < 288; ++n) {
    uint64_t z = mix64(key + (uint64_t)(n + 1) * GOLDEN);
    double u1 = ((double)(z >> 32) + 0.5) * (1.0 / 4294967296.0);
    double u2 = ((double)(z & 0xFFFFFFFFULL) + 0.5) * (1.0 / 4294967296.0);
    double rad = sqrt(-2.0 * log(u1));
    x[2 * n] = (float)(rad * cos(two_pi * u2));
    x[2 * n + 1] = (float)(rad * sin(two_pi * u2));
  }
  for (int blk = 0; blk < 4; ++blk) {
    float amax = 0.0f;
    for (int d = 0; d < 128; ++d) amax = fmaxf(amax, fabsf(x[128 * blk + d]));
    float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    for (int d = 0; d < 128; ++d) dst[128 * blk + d] = e4m3_rne(x[128 * blk + d] / scale);
    memcpy(dst + 512 + 4 * blk, &scale, 4);
  }
  uint16_t* rope = (uint16_t*)(dst + 528);
  for (int d = 0; d < 64; ++d) rope[d] = f32_to_bf16_rne(x[512 + d]);
}

/* A record of either format: 656 bytes means FP8, else rec_bytes / 2 bf16 values. */
static void synth_record(uint8_t* dst, uint64_t seed, int64_t a, int64_t b, int64_t c, int64_t rec_bytes) {
  if (rec_bytes == 656) synth_one_fp8(dst, seed, a, b, c);
  else synth_one((uint16_t*)dst, seed, a, b, c, rec_bytes / 2);
}

typedef struct {
  uint8_t* base; /* [L][lmax][rec] region of one request */
  int64_t req, L, lmax, pos_lo, pos_hi, rec_bytes;
  uint64_t seed;
} fill_job;

static void* fill_worker(void* arg) {
  fill_job* j = (fill_job*)arg;
  for (int64_t l = 0; l < j->L; ++l) {
    uint8_t* lbase = j->base + (size_t)l * (size_t)j->lmax * (size_t)j->rec_bytes;
    for (int64_t p = j->pos_lo; p < j->pos_hi; ++p)
      synth_record(lbase + (size_t)p * (size_t)j->rec_bytes, j->seed, j->req, l, p, j->rec_bytes);
  }
  return NULL;
}

/*
 * Fills one request's host region [L][lmax][rec_bytes]: positions [0, ctx)
 * get the records of request `req`; positions [ctx, lmax) get the poison
 * byte (not yet written).  Thread t generates positions
 * [ctx*t/n, ctx*(t+1)/n) of every layer.
 */
int synth_fill_request(uint8_t* base, int64_t req, int64_t L, int64_t lmax, int64_t ctx,
                       int64_t rec_bytes, uint64_t seed, int poison, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (ctx > lmax || ctx < 0 || rec_bytes % 4) return -1;
  fill_job jobs[256];
  pthread_t th[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].base = base; jobs[t].req = req; jobs[t].L = L; jobs[t].lmax = lmax;
    jobs[t].pos_lo = ctx * t / nthreads; jobs[t].pos_hi = ctx * (t + 1) / nthreads;
    jobs[t].rec_bytes = rec_bytes; jobs[t].seed = seed;
  }
  int started = 1;
  for (; started < nthreads; ++started)
    if (pthread_create(&th[started], NULL, fill_worker, &jobs[started])) break;
  for (int t = started; t < nthreads; ++t) fill_worker(&jobs[t]); /* threads we could not start */
  fill_worker(&jobs[0]);
  for (int t = 1; t < started; ++t) pthread_join(th[t], NULL);
  if (lmax > ctx)
    for (int64_t l = 0; l < L; ++l)
      memset(base + ((size_t)l * (size_t)lmax + (size_t)ctx) * (size_t)rec_bytes, poison,
             (size_t)(lmax - ctx) * (size_t)rec_bytes);
  return 0;
}

/* Records at one position per (request, layer): dst[R][L][rec], position pos[r]. */
void synth_records_at(uint8_t* dst, int64_t R, int64_t L, const int64_t* pos, int64_t rec_bytes,
                      uint64_t seed) {
  for (int64_t r = 0; r < R; ++r)
    for (int64_t l = 0; l < L; ++l)
      synth_record(dst + ((size_t)r * (size_t)L + (size_t)l) * (size_t)rec_bytes, seed, r, l, pos[r],
                   rec_bytes);
}
