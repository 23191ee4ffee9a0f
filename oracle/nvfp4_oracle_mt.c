/*
 * nvfp4_oracle_mt.c -- the oracle's whole-tensor quantizer run on several host
 * threads, for the CPU baseline that is timed beside the GPU.
 *
 * TEST INFRASTRUCTURE ONLY (like nvfp4_oracle.c, whose functions it calls and
 * whose arithmetic it does not touch).  Blocks are independent, and the only
 * quantity coupling them is the tensor amax behind the global scale
 * ("Technical summary: Four Over Six (4/6)", "Implementation details").  So:
 *   1. each thread takes the amax of one slice of x (nvfp4o_amax), and the
 *      largest of those is the tensor amax; g follows as nvfp4o_quantize
 *      forms it (nvfp4o_global_scale);
 *   2. the rows are split into contiguous ranges of a multiple of 8 rows
 *      (so every range's part of the selection bitmap starts on a byte), and
 *      each thread runs nvfp4o_quantize on its range with g given.
 * The codes, scale bytes, bitmap and g equal the single-threaded call's bit
 * for bit; the error sum adds the ranges' binary64 sums in range order.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#include "nvfp4_oracle.h"

typedef struct {
  const uint16_t* x;
  int64_t n;
  float amax;
} amax_job_t;

typedef struct {
  const uint16_t* x;
  int64_t rows, cols;
  int mode, rule;
  float g;
  uint8_t* packed;
  uint8_t* scales;
  uint8_t* selmap;
  double err;
  int status;
} range_job_t;

static void* amax_worker(void* p) {
  amax_job_t* j = (amax_job_t*)p;
  j->amax = j->n > 0 ? nvfp4o_amax(j->x, j->n) : 0.0f;
  return NULL;
}

static void* range_worker(void* p) {
  range_job_t* j = (range_job_t*)p;
  float g = j->g;
  j->err = 0.0;
  j->status = NVFP4O_OK;
  if (j->rows > 0)
    j->status = nvfp4o_quantize(j->x, j->rows, j->cols, NVFP4O_AXIS_COLS, j->mode, j->rule, 1,
                                &g, j->packed, j->scales, j->selmap, &j->err);
  return NULL;
}

/* Runs fn over jobs[0..n-1] on n threads (job 0 on the calling thread). */
static int run_all(void* (*fn)(void*), void* jobs, size_t size, int n) {
  pthread_t* tid = (pthread_t*)calloc((size_t)n, sizeof(pthread_t));
  if (!tid) return NVFP4O_ERR_ALLOC;
  int started = 1, st = NVFP4O_OK;
  for (int t = 1; t < n; ++t, ++started)
    if (pthread_create(&tid[t], NULL, fn, (char*)jobs + (size_t)t * size) != 0) {
      st = NVFP4O_ERR_ALLOC;
      break;
    }
  fn(jobs);
  for (int t = 1; t < started; ++t) pthread_join(tid[t], NULL);
  free(tid);
  return st;
}

int nvfp4o_quantize_mt(const uint16_t* x, int64_t rows, int64_t cols, int mode, int rule,
                       int threads, int gscale_given, float* gscale, uint8_t* packed,
                       uint8_t* scales, uint8_t* selmap, double* err_sum) {
  if (!x || !gscale || !packed || !scales) return NVFP4O_ERR_NULL;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0) return NVFP4O_ERR_SHAPE;
  if (threads < 1) threads = 1;
  if (threads > 1024) threads = 1024;
  /* The E4M3 encoder fills a static table on its first call; make that call
   * here, before any thread exists, so that the threads only read it. */
  (void)nvfp4o_e4m3_encode(1.0f);

  float g;
  if (gscale_given) {
    g = *gscale;
  } else {
    amax_job_t* aj = (amax_job_t*)calloc((size_t)threads, sizeof(amax_job_t));
    if (!aj) return NVFP4O_ERR_ALLOC;
    const int64_t n = rows * cols, per = (n + threads - 1) / threads;
    for (int t = 0; t < threads; ++t) {
      const int64_t a = (int64_t)t * per < n ? (int64_t)t * per : n;
      const int64_t b = a + per < n ? a + per : n;
      aj[t].x = x + a;
      aj[t].n = b - a;
    }
    int st = run_all(amax_worker, aj, sizeof(amax_job_t), threads);
    float amax = 0.0f;
    for (int t = 0; t < threads; ++t)
      if (aj[t].amax > amax) amax = aj[t].amax;
    free(aj);
    if (st != NVFP4O_OK) return st;
    g = nvfp4o_global_scale(amax, mode);
  }
  *gscale = g;

  range_job_t* rj = (range_job_t*)calloc((size_t)threads, sizeof(range_job_t));
  if (!rj) return NVFP4O_ERR_ALLOC;
  /* Ranges of a multiple of 8 rows: 8 rows hold cols/2 blocks, a multiple of
   * 8, so each range's bitmap bytes are its own. */
  int64_t per = (rows + threads - 1) / threads;
  per = (per + 7) / 8 * 8;
  for (int t = 0; t < threads; ++t) {
    const int64_t r0 = (int64_t)t * per < rows ? (int64_t)t * per : rows;
    const int64_t r1 = r0 + per < rows ? r0 + per : rows;
    const int64_t b0 = r0 * (cols / 16);
    rj[t].x = x + r0 * cols;
    rj[t].rows = r1 - r0;
    rj[t].cols = cols;
    rj[t].mode = mode;
    rj[t].rule = rule;
    rj[t].g = g;
    rj[t].packed = packed + b0 * 8;
    rj[t].scales = scales + b0;
    rj[t].selmap = selmap ? selmap + b0 / 8 : NULL;
  }
  int st = run_all(range_worker, rj, sizeof(range_job_t), threads);
  double sum = 0.0;
  for (int t = 0; t < threads && st == NVFP4O_OK; ++t) {
    if (rj[t].status != NVFP4O_OK) st = rj[t].status;
    sum += rj[t].err;
  }
  free(rj);
  if (st == NVFP4O_OK && err_sum) *err_sum = sum;
  return st;
}
