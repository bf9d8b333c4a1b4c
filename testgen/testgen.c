/*
 * testgen.c - seeded, counter-based synthetic input generator.
 *
 * Holds none of the SSM arithmetic: it only turns (seed, stream, index)
 * into numbers with a stated distribution, so that the HIP path and the
 * float64 oracle receive bit-identical inputs, and so that any slice of a
 * large tensor can be regenerated on the host without the rest of it.
 *
 * Published methods used:
 *   - SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
 *     pseudorandom number generators", OOPSLA 2014): an add-then-mix
 *     counter generator; here the counter is the element index.
 *   - Box-Muller transform (Box and Muller, "A note on the generation of
 *     random normal deviates", 1958): two uniforms -> two normals.  Element
 *     2k takes the cosine branch and 2k+1 the sine branch of pair k.
 *   - bfloat16 rounding: round-to-nearest-even on the top 16 bits of the
 *     IEEE-754 binary32 pattern.
 *
 * Distributions: 0 = normal(a = mean, b = standard deviation),
 *                1 = uniform(a, b),
 *                2 = -exp(uniform(a, b))   (negative log-uniform).
 *
 * The value drawn for element i of a tensor depends only on
 * (seed, stream, offset + i); threads split the index range.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define TG_GOLDEN 0x9E3779B97F4A7C15ull
#define TG_TWO_PI 6.283185307179586476925286766559

static inline uint64_t tg_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* key for one (seed, stream) pair */
static inline uint64_t tg_key(uint64_t seed, uint64_t stream) {
  return tg_mix64(seed + TG_GOLDEN * (tg_mix64(stream + TG_GOLDEN) | 1ull));
}

/* 64 random bits for counter c under key k */
static inline uint64_t tg_bits(uint64_t key, uint64_t c) {
  return tg_mix64(key + (c + 1ull) * TG_GOLDEN);
}

/* uniform on the open interval (0, 1), 53-bit resolution */
static inline double tg_u01(uint64_t key, uint64_t c) {
  return ((double)(tg_bits(key, c) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double tg_normal(uint64_t key, uint64_t i) {
  uint64_t k = i >> 1;
  double u1 = tg_u01(key, 2 * k);
  double u2 = tg_u01(key, 2 * k + 1);
  double r = sqrt(-2.0 * log(u1));
  double t = TG_TWO_PI * u2;
  return (i & 1) ? r * sin(t) : r * cos(t);
}

static inline double tg_value(uint64_t key, uint64_t i, int dist, double a, double b) {
  switch (dist) {
    case 0: return a + b * tg_normal(key, i);
    case 1: return a + (b - a) * tg_u01(key, i);
    case 2: return -exp(a + (b - a) * tg_u01(key, i));
    default: return 0.0;
  }
}

uint16_t tg_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

typedef struct {
  void* out;
  int64_t lo, hi;
  uint64_t key;
  int64_t offset;
  int dist;
  double a, b;
  int bf16;
} tg_job;

/* normal draws two at a time: one log/sqrt and one sin/cos pair per pair
 * index k gives elements 2k and 2k+1 (same values as tg_normal) */
static void tg_normal_run(const tg_job* j) {
  int64_t i = j->lo;
  while (i < j->hi) {
    uint64_t gi = (uint64_t)(j->offset + i);
    if ((gi & 1) == 0 && i + 1 < j->hi) {
      uint64_t k = gi >> 1;
      double u1 = tg_u01(j->key, 2 * k), u2 = tg_u01(j->key, 2 * k + 1);
      double r = sqrt(-2.0 * log(u1)), t = TG_TWO_PI * u2;
      double z0 = j->a + j->b * (r * cos(t)), z1 = j->a + j->b * (r * sin(t));
      if (j->bf16) {
        ((uint16_t*)j->out)[i] = tg_f32_to_bf16((float)z0);
        ((uint16_t*)j->out)[i + 1] = tg_f32_to_bf16((float)z1);
      } else {
        ((float*)j->out)[i] = (float)z0;
        ((float*)j->out)[i + 1] = (float)z1;
      }
      i += 2;
    } else {
      double z = tg_value(j->key, gi, 0, j->a, j->b);
      if (j->bf16)
        ((uint16_t*)j->out)[i] = tg_f32_to_bf16((float)z);
      else
        ((float*)j->out)[i] = (float)z;
      i += 1;
    }
  }
}

static void* tg_worker(void* p) {
  tg_job* j = (tg_job*)p;
  if (j->dist == 0) {
    tg_normal_run(j);
    return NULL;
  }
  if (j->bf16) {
    uint16_t* o = (uint16_t*)j->out;
    for (int64_t i = j->lo; i < j->hi; ++i)
      o[i] = tg_f32_to_bf16((float)tg_value(j->key, (uint64_t)(j->offset + i), j->dist, j->a, j->b));
  } else {
    float* o = (float*)j->out;
    for (int64_t i = j->lo; i < j->hi; ++i)
      o[i] = (float)tg_value(j->key, (uint64_t)(j->offset + i), j->dist, j->a, j->b);
  }
  return NULL;
}

#define TG_MAX_THREADS 64

static int tg_fill(void* out, int64_t n, uint64_t seed, uint64_t stream, int64_t offset, int dist,
                   double a, double b, int bf16, int nthreads) {
  if (n <= 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > TG_MAX_THREADS) nthreads = TG_MAX_THREADS;
  if (n < 65536) nthreads = 1;
  tg_job jobs[TG_MAX_THREADS];
  pthread_t th[TG_MAX_THREADS];
  uint64_t key = tg_key(seed, stream);
  int64_t per = (n + nthreads - 1) / nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t lo = (int64_t)t * per, hi = lo + per;
    if (hi > n) hi = n;
    if (lo >= hi) break;
    jobs[t] = (tg_job){out, lo, hi, key, offset, dist, a, b, bf16};
    if (t == 0) continue;
    if (pthread_create(&th[t], NULL, tg_worker, &jobs[t]) != 0) {
      tg_worker(&jobs[t]);
      th[t] = 0;
    }
    started = t;
  }
  tg_worker(&jobs[0]);
  for (int t = 1; t <= started; ++t)
    if (th[t]) pthread_join(th[t], NULL);
  return 0;
}

/* Fill n float32 values; element i is value (offset + i) of the stream. */
int tg_fill_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, int64_t offset, int dist,
                double a, double b, int nthreads) {
  return tg_fill(out, n, seed, stream, offset, dist, a, b, 0, nthreads);
}

/* Same draws rounded float64 -> float32 -> bfloat16 (round to nearest even). */
int tg_fill_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream, int64_t offset, int dist,
                 double a, double b, int nthreads) {
  return tg_fill(out, n, seed, stream, offset, dist, a, b, 1, nthreads);
}

/* Raw 64-bit draws (tests of the generator itself). */
void tg_raw_bits(uint64_t* out, int64_t n, uint64_t seed, uint64_t stream, int64_t offset) {
  uint64_t key = tg_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = tg_bits(key, (uint64_t)(offset + i));
}
