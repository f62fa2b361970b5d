/*
 * Seeded, counter-based input generator for the selective-scan workloads.
 *
 * This module produces synthetic inputs only; it holds none of the scan's arithmetic. Both the
 * HIP path's tests/bench and the CPU oracle draw their inputs from it, so both sides see the
 * same bits.
 *
 * Definition (every value is a pure function of (seed, tensor_id, flat index)):
 *   mix64(z)     : the SplitMix64 output finaliser (Vigna, 2015):
 *                  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
 *                  z ^= z >> 31.
 *   key          = mix64(seed + tensor_id * GAMMA),            GAMMA = 0x9E3779B97F4A7C15
 *   raw(i)       = mix64(key + (i + 1) * GAMMA)                 (i-th output of SplitMix64 from key)
 *   uniform(i)   = (raw(i) >> 11) * 2^-53                       in [0, 1)
 *   normal(i)    : Box-Muller on the pair p = i / 2:
 *                  r = sqrt(-2 ln(1 - uniform(2p))), th = 2 pi uniform(2p + 1),
 *                  normal(i) = r cos(th) for even i, r sin(th) for odd i.
 * Distributions (all evaluated in double):
 *   NORMAL(m, s)               : m + s * normal(i)
 *   UNIFORM(a, b)              : a + (b - a) * uniform(i)
 *   INV_SOFTPLUS_UNIFORM(a, b) : log(expm1(v)), v = a + (b - a) * uniform(i)
 *                                (a value whose softplus is v; used for the dt bias recipe)
 *   NEG_ARANGE(m)              : -((i mod m) + 1)          (no randomness)
 * Output quantisation: double -> float by round-to-nearest-even (the C cast); BF16 then rounds
 * the float to its upper 16 bits with round-to-nearest-even (NaN kept quiet).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define SSMGEN_GAMMA 0x9E3779B97F4A7C15ULL

enum { SSMGEN_NORMAL = 0, SSMGEN_UNIFORM = 1, SSMGEN_INV_SOFTPLUS_UNIFORM = 2, SSMGEN_NEG_ARANGE = 3 };
enum { SSMGEN_F64 = 0, SSMGEN_F32 = 1, SSMGEN_BF16 = 2 };

static inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27; z *= 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tensor_id) {
  return mix64(seed + tensor_id * SSMGEN_GAMMA);
}

static inline double uniform_at(uint64_t key, uint64_t i) {
  return (double)(mix64(key + (i + 1) * SSMGEN_GAMMA) >> 11) * 0x1.0p-53;
}

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = uniform_at(key, 2 * p), u2 = uniform_at(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(1.0 - u1));
  double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u; memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static double value_at(uint64_t key, int dist, double p0, double p1, uint64_t i) {
  switch (dist) {
    case SSMGEN_NORMAL: return p0 + p1 * normal_at(key, i);
    case SSMGEN_UNIFORM: return p0 + (p1 - p0) * uniform_at(key, i);
    case SSMGEN_INV_SOFTPLUS_UNIFORM: {
      double v = p0 + (p1 - p0) * uniform_at(key, i);
      return log(expm1(v));
    }
    case SSMGEN_NEG_ARANGE: return -(double)((i % (uint64_t)p0) + 1);
    default: return NAN;
  }
}

typedef struct {
  uint64_t key; int dist; double p0, p1; uint64_t start, count; int dtype; void* out;
} fill_job;

static void fill_range(const fill_job* j, uint64_t lo, uint64_t hi) {
  for (uint64_t k = lo; k < hi; ++k) {
    double v = value_at(j->key, j->dist, j->p0, j->p1, j->start + k);
    if (j->dtype == SSMGEN_F64) ((double*)j->out)[k] = v;
    else if (j->dtype == SSMGEN_F32) ((float*)j->out)[k] = (float)v;
    else ((uint16_t*)j->out)[k] = f32_to_bf16_rne((float)v);
  }
}

typedef struct { const fill_job* job; uint64_t lo, hi; } fill_part;

static void* fill_worker(void* arg) {
  fill_part* p = (fill_part*)arg;
  fill_range(p->job, p->lo, p->hi);
  return NULL;
}

/* Fill out[0..count) with values start..start+count of stream (seed, tensor_id).
 * Returns 0, or -1 on a bad dist/dtype. Uses up to nthreads POSIX threads. */
int ssmgen_fill(uint64_t seed, uint64_t tensor_id, int dist, double p0, double p1,
                uint64_t start, uint64_t count, int dtype, void* out, int nthreads) {
  if (dist < 0 || dist > SSMGEN_NEG_ARANGE || dtype < 0 || dtype > SSMGEN_BF16) return -1;
  if (dist == SSMGEN_NEG_ARANGE && !(p0 >= 1.0)) return -1;
  if (count == 0) return 0;
  if (!out) return -1;
  fill_job job = {stream_key(seed, tensor_id), dist, p0, p1, start, count, dtype, out};
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (count < (uint64_t)65536 || nthreads == 1) { fill_range(&job, 0, count); return 0; }
  pthread_t th[256]; fill_part parts[256];
  uint64_t per = (count + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
  int launched = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t lo = per * (uint64_t)t, hi = lo + per;
    if (lo >= count) break;
    if (hi > count) hi = count;
    parts[t].job = &job; parts[t].lo = lo; parts[t].hi = hi;
    if (pthread_create(&th[t], NULL, fill_worker, &parts[t]) != 0) { fill_range(&job, lo, hi); parts[t].job = NULL; }
    launched = t + 1;
  }
  for (int t = 0; t < launched; ++t) if (parts[t].job) pthread_join(th[t], NULL);
  return 0;
}

/* Single raw 64-bit draw, exposed so tests can check the stream against SplitMix64's definition. */
uint64_t ssmgen_raw(uint64_t seed, uint64_t tensor_id, uint64_t i) {
  return mix64(stream_key(seed, tensor_id) + (i + 1) * SSMGEN_GAMMA);
}

/* float -> bf16 bits with round-to-nearest-even, exposed for tests of the quantiser. */
uint16_t ssmgen_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }
