/*
 * synth.c -- seeded synthetic bf16 tensors for tests and benchmarks.
 *
 * This module holds no NVFP4 arithmetic: it only draws random numbers and
 * rounds them to bf16.  Both the oracle checks and the GPU runs consume the
 * same host buffers it produces.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: draw k of stream `seed` is mix64(seed + (k + 1) * 0x9E3779B97F4A7C15),
 * so every element can be generated independently and the output does not
 * depend on the number of threads.
 *   uniform   u = ((z >> 11) + 0.5) * 2^-53, in (0, 1)
 *   normal    Box-Muller, Z = sqrt(-2 ln u1) * cos(2 pi u2) (and sin for a pair)
 *   Student-t(3)  Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3)
 *   Laplace(0, beta)  -beta * sgn(u - 1/2) * ln(1 - 2 |u - 1/2|)
 *   exact-count sampling without replacement: Floyd's algorithm (Bentley and
 *   Floyd, "A sample of brilliance", CACM 1987) with Lemire's multiply-shift
 *   for bounded integers.
 * Values are produced in binary64, rounded to binary32 (RN) and then to
 * bf16 (RNE).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_draw(uint64_t seed, uint64_t k) { return mix64(seed + (k + 1) * GAMMA); }

static inline double u01(uint64_t z) { return ((double)(z >> 11) + 0.5) * 0x1.0p-53; }

static inline uint16_t f64_to_bf16(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline double bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static const double TWO_PI = 6.283185307179586476925286766559;

static inline double normal_at(uint64_t seed, uint64_t i) {
  double u1 = u01(synth_draw(seed, 2 * i)), u2 = u01(synth_draw(seed, 2 * i + 1));
  return sqrt(-2.0 * log(u1)) * cos(TWO_PI * u2);
}

static inline double student_t3_at(uint64_t seed, uint64_t i) {
  double u1 = u01(synth_draw(seed, 4 * i)), u2 = u01(synth_draw(seed, 4 * i + 1));
  double u3 = u01(synth_draw(seed, 4 * i + 2)), u4 = u01(synth_draw(seed, 4 * i + 3));
  double r1 = sqrt(-2.0 * log(u1)), r2 = sqrt(-2.0 * log(u3));
  double z0 = r1 * cos(TWO_PI * u2), z1 = r1 * sin(TWO_PI * u2);
  double z2 = r2 * cos(TWO_PI * u4), z3 = r2 * sin(TWO_PI * u4);
  return z0 / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
}

static inline double laplace_at(uint64_t seed, uint64_t i, double beta) {
  double u = u01(synth_draw(seed, i)) - 0.5;
  double sg = u < 0 ? -1.0 : (u > 0 ? 1.0 : 0.0);
  return -beta * sg * log(1.0 - 2.0 * fabs(u));
}

/* ---- element-parallel fill ------------------------------------------------ */

enum { SYNTH_NORMAL = 0, SYNTH_STUDENT_T3 = 1, SYNTH_LAPLACE = 2, SYNTH_UNIFORM = 3 };

typedef struct {
  int dist;
  double scale, param;
  uint64_t seed;
  int64_t begin, end;
  uint16_t* out;
} fill_job_t;

static void* fill_worker(void* arg) {
  fill_job_t* j = (fill_job_t*)arg;
  for (int64_t i = j->begin; i < j->end; ++i) {
    double v;
    switch (j->dist) {
      case SYNTH_STUDENT_T3: v = student_t3_at(j->seed, (uint64_t)i); break;
      case SYNTH_LAPLACE: v = laplace_at(j->seed, (uint64_t)i, 1.0); break;
      case SYNTH_UNIFORM: v = 2.0 * u01(synth_draw(j->seed, (uint64_t)i)) - 1.0; break;
      default: v = normal_at(j->seed, (uint64_t)i); break;
    }
    j->out[i] = f64_to_bf16(j->scale * v);
  }
  return NULL;
}

/* out[i] = bf16(scale * D_i) for i in [0, n), D from distribution `dist`
 * (uniform is on (-1, 1)).  `threads` only changes speed, never values. */
void synth_fill(int dist, double scale, uint64_t seed, int64_t n, uint16_t* out, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  if (n < 65536) threads = 1;
  pthread_t tid[64];
  fill_job_t jobs[64];
  int64_t chunk = (n + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    int64_t b = t * chunk, e = b + chunk;
    if (b > n) b = n;
    if (e > n) e = n;
    jobs[t] = (fill_job_t){dist, scale, 0.0, seed, b, e, out};
  }
  if (threads == 1) {
    fill_worker(&jobs[0]);
    return;
  }
  for (int t = 0; t < threads; ++t) pthread_create(&tid[t], NULL, fill_worker, &jobs[t]);
  for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
}

/* ---- exact-count sampling without replacement ------------------------------ */

static inline uint64_t bounded(uint64_t z, uint64_t n) {
  /* Lemire's multiply-shift on the full 64-bit draw: floor(z * n / 2^64). */
  return (uint64_t)(((unsigned __int128)z * n) >> 64);
}

/* Floyd's algorithm: writes k distinct indices of [0, n) to idx (in the order
 * drawn) and returns k, or -1 on bad arguments / allocation failure. */
int64_t synth_sample(uint64_t seed, int64_t n, int64_t k, int64_t* idx) {
  if (n <= 0 || k < 0 || k > n) return -1;
  uint8_t* seen = (uint8_t*)calloc((size_t)((n + 7) / 8), 1);
  if (!seen) return -1;
  int64_t c = 0;
  for (int64_t j = n - k; j < n; ++j) {
    int64_t t = (int64_t)bounded(synth_draw(seed, (uint64_t)c), (uint64_t)j + 1);
    if (seen[t >> 3] & (1u << (t & 7))) t = j;
    seen[t >> 3] |= (uint8_t)(1u << (t & 7));
    idx[c++] = t;
  }
  free(seen);
  return c;
}

/* ---- structured outliers ---------------------------------------------------- */

/* Multiply the elements at idx[0..k) by `factor` (binary64, one rounding). */
void synth_scale_at(uint16_t* x, const int64_t* idx, int64_t k, double factor) {
  for (int64_t i = 0; i < k; ++i) x[idx[i]] = f64_to_bf16(bf16_to_f64(x[idx[i]]) * factor);
}

/* Replace the elements at idx[0..k) by Laplace(0, beta) draws of stream seed. */
void synth_replace_laplace(uint16_t* x, const int64_t* idx, int64_t k, uint64_t seed, double beta) {
  for (int64_t i = 0; i < k; ++i) x[idx[i]] = f64_to_bf16(laplace_at(seed, (uint64_t)i, beta));
}

/* Multiply whole columns cols_idx[0..k) of a [rows][cols] tensor by factor. */
void synth_scale_columns(uint16_t* x, int64_t rows, int64_t cols, const int64_t* cols_idx,
                         int64_t k, double factor) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < k; ++i) {
      uint16_t* p = &x[r * cols + cols_idx[i]];
      *p = f64_to_bf16(bf16_to_f64(*p) * factor);
    }
}

/* FNV-1a 64 of a byte buffer: identifies an input in logs. */
uint64_t synth_fnv1a64(const void* data, int64_t nbytes) {
  const uint8_t* p = (const uint8_t*)data;
  uint64_t h = 0xCBF29CE484222325ull;
  for (int64_t i = 0; i < nbytes; ++i) {
    h ^= p[i];
    h *= 0x100000001B3ull;
  }
  return h;
}
