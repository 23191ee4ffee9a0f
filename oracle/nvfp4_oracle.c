/*
 * nvfp4_oracle.c -- plain CPU oracle for NVFP4 block-scaled quantization with
 * "Four Over Six" (4/6) adaptive block scales.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline of the benchmark load this file.  The product path (the HIP library)
 * never links, calls or includes it, and this file includes nothing from the
 * product path.
 *
 * Sources (web pages; cited by title and section):
 *  [FOS]  "Technical summary: Four Over Six (4/6)" (gist.science, paper 2512.02010)
 *        - "Problem statement": E2M1 step sizes 0.5 / 1 / 2 on [0,2] / [2,4] /
 *          [4,6]; standard NVFP4 scales every block so that its max maps to 6.
 *        - "Core mechanism": the 4/6 alternative maps the block max to 4.
 *        - "Adaptive block scaling algorithm": quantize each block twice (max->6
 *          and max->4), measure both errors against the original values, keep
 *          the candidate with the smaller error.  The page evaluates three
 *          rules: minimum maximum error, minimum MAE, minimum MSE.
 *        - "Implementation details": block scales are FP8 E4M3; under 4/6 the
 *          per-tensor scale is formed with 256 in place of 448.
 *  [MIN] "Why Gated DeltaNet in hybrid 27B LLMs withstands 4-bit quantization"
 *        (sns.style) - "Background": every linear layer in NVFP4 W4A4 (weights
 *        and activations both 4-bit); "Deep analysis": NVFP4 scales blocks of
 *        16 elements.
 *  [ARC] "ARCQuant" summary (gist.science, paper 2601.07475) - "Problem
 *        definition": NVFP4 requires block size 16; "Methodology": channels
 *        reordered by absolute maximum, the top-S outlier channels get a
 *        residual stage (original minus primary reconstruction) quantized as
 *        a second NVFP4 channel set appended along the reduction dimension;
 *        the authors fuse channel reordering, RMSNorm and both quantization
 *        stages into one kernel; the matching weight channels are duplicated
 *        and the whole layer runs as one GEMM over K_in + S.
 *
 * The pages fix the formats and the steps, not the floating-point operation
 * order.  This file fixes it, taking the plainest reading where the pages are
 * silent.  In short:
 *   g   = RN(A / (6*M)),  M = 448 (standard) or 256 (4/6), A = max |x|
 *   G   = RN(1/g), replaced by 0 unless 0 < G <= FLT_MAX
 *   k_c = RN(G / c)                              c in {6} or {6, 4}
 *   per block: b = max |x_i|;  s_c = RN(b * k_c);  S_c = E4M3_rne_sat(s_c)
 *              d_c = RN(dec(S_c) * g);  r_c = min(RN(G * T[S_c]), FLT_MAX)
 *              with T[S] = RN(1/dec(S)) and T[0] = 0
 *   per element: y = RN(x * r_c);  m = E2M1 index of |y| (RNE, saturating)
 *                code = sign(x) << 3 | m;  xhat = RN(+-VAL[m] * d_c)
 *                delta = fma(+-VAL[m], d_c, -x)   (the error of the candidate's
 *                reconstruction against the original value, rounded once)
 *   block error: two sequential halves of 8 elements (lo, hi), e = RN(lo + hi)
 *                MSE: h = fma(delta, delta, h)      MAE: h = RN(h + |delta|)
 *                MAX: e = max |delta| over the block (exact, order-free)
 *   selection:   c* = 4 iff e_4 < e_6 (ties and NaN go to 6)
 * RN is one IEEE-754 binary32 operation with round-to-nearest-even.
 *
 * Parity pins: every function here is checked by the CPU test suite against
 * facts fixed outside this file (the pages' worked facts, torch's float8
 * and bfloat16 casts, closed forms, brute force).  The fp32 operation order
 * of the block pipeline (G, k_c, r_c, y, xhat, delta, the error sums) is a
 * reading of the pages, not something the pages print: it is pinned only by
 * invariants and bounds, and is "parity unpinned" at the level of the
 * individual rounding choices.  The dequantized value is RN(v * d); the error
 * is taken against the unrounded v * d (one rounding of v * d - x).
 *
 * Build: gcc -std=c99 -O2 -ffp-contract=off -fno-fast-math (SSE binary32,
 * FLT_EVAL_METHOD == 0).  Single-threaded, no SIMD intrinsics, no tables
 * beyond the eight E2M1 magnitudes.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4_oracle.h"

/* ------------------------------------------------------------------------ */
/* Formats                                                                  */
/* ------------------------------------------------------------------------ */

/* The eight E2M1 magnitudes [FOS, "Problem statement"]: the grid steps by 0.5
 * up to 2, by 1 up to 4, by 2 up to 6.  Index = the 3-bit magnitude field. */
static const float E2M1_VAL[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float nvfp4o_bf16_to_f32(uint16_t h) {
  /* bf16 is the upper half of a binary32 word: widening is exact. */
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

uint16_t nvfp4o_f32_to_bf16(float f) {
  /* Round-to-nearest-even onto the upper 16 bits. */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* Magnitude index of the E2M1 value nearest to a >= 0.  Ties go to the even
 * index (even mantissa bit), values at or above 6 saturate to 6, NaN maps to
 * 0.  Written as a nearest-neighbour search over the eight magnitudes. */
int nvfp4o_e2m1_index(float a) {
  if (a != a) return 0;
  if (a >= 6.0f) return 7;
  int best = 0;
  double best_dist = fabs((double)a - (double)E2M1_VAL[0]);
  for (int m = 1; m < 8; ++m) {
    double dist = fabs((double)a - (double)E2M1_VAL[m]);
    if (dist < best_dist || (dist == best_dist && (m & 1) == 0)) {
      best = m;
      best_dist = dist;
    }
  }
  return best;
}

float nvfp4o_e2m1_decode(uint8_t code) {
  float v = E2M1_VAL[code & 7u];
  return (code & 8u) ? -v : v;
}

/* OCP E4M3FN: bias 7, 3 mantissa bits, subnormals m*2^-9, max 448 (0x7E),
 * 0x7F is NaN, no infinities. */
float nvfp4o_e4m3_decode(uint8_t S) {
  uint32_t e = (S >> 3) & 15u, m = S & 7u;
  float v;
  if ((S & 0x7Fu) == 0x7Fu)
    v = NAN;
  else if (e == 0)
    v = ldexpf((float)m, -9);
  else
    v = ldexpf((float)(8u + m), (int)e - 10);
  return (S & 0x80u) ? -v : v;
}

/* Block-scale encoder: the E4M3 value nearest to s >= 0 among the 127 finite
 * non-negative codes 0x00..0x7E, ties to the even code (even mantissa),
 * saturating: anything at or above 448 (including +inf) gives 0x7E.  NaN,
 * zero and negative inputs give 0x00.  Written as a nearest-neighbour search
 * over all finite codes. */
uint8_t nvfp4o_e4m3_encode(float s) {
  /* The 127 candidate values, filled once by the decoder above. */
  static double value_of[0x7F];
  static int filled = 0;
  if (!filled) {
    for (int S = 0; S < 0x7F; ++S) value_of[S] = (double)nvfp4o_e4m3_decode((uint8_t)S);
    filled = 1;
  }
  if (!(s > 0.0f)) return 0;
  if (s >= 448.0f) return 0x7E;
  int best = 0;
  double best_dist = fabs((double)s);
  for (int S = 1; S <= 0x7E; ++S) {
    double dist = fabs((double)s - value_of[S]);
    if (dist < best_dist || (dist == best_dist && (S & 1) == 0)) {
      best = S;
      best_dist = dist;
    }
  }
  return (uint8_t)best;
}

/* Array forms of the two encoders, for exhaustive checks. */
void nvfp4o_e2m1_index_array(const float* a, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)nvfp4o_e2m1_index(a[i]);
}

void nvfp4o_e4m3_encode_array(const float* s, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = nvfp4o_e4m3_encode(s[i]);
}

/* T[S]: correctly rounded reciprocal of a block scale; T[0] = 0 so that a
 * zero block scale encodes every element of the block as zero. */
float nvfp4o_e4m3_recip(uint8_t S) {
  S &= 0x7Fu;
  if (S == 0 || S == 0x7F) return 0.0f;
  return 1.0f / nvfp4o_e4m3_decode(S);
}

/* ------------------------------------------------------------------------ */
/* Per-tensor scales                                                         */
/* ------------------------------------------------------------------------ */

float nvfp4o_amax(const uint16_t* x, int64_t n) {
  float a = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float v = fabsf(nvfp4o_bf16_to_f32(x[i]));
    if (v > a) a = v;
  }
  return a;
}

/* The "FP8 max" constant of the global scale: 448 for standard NVFP4, 256 under
 * 4/6 ([FOS, "Implementation details"]); the 6 is the E2M1 max. */
static float six_m(int mode) { return mode == NVFP4O_MODE_4OVER6 ? 1536.0f : 2688.0f; }

float nvfp4o_global_scale(float amax, int mode) { return amax / six_m(mode); }

static float encode_scale_of(float g) {
  float G = 1.0f / g;
  if (!(G > 0.0f && G <= FLT_MAX)) G = 0.0f;
  return G;
}

/* ------------------------------------------------------------------------ */
/* One block                                                                 */
/* ------------------------------------------------------------------------ */

void nvfp4o_quantize_block(const float x[16], float g, int mode, int rule,
                           nvfp4o_block_t* out) {
  memset(out, 0, sizeof *out);
  const float G = encode_scale_of(g);
  const float cands[2] = {6.0f, 4.0f};
  const int ncand = (mode == NVFP4O_MODE_4OVER6) ? 2 : 1;
  /* The error measure: MAE or maximum error only when asked for under 4/6;
   * the standard mode reports squared error. */
  const int use_mae = (mode == NVFP4O_MODE_4OVER6 && rule == NVFP4O_RULE_MAE);
  const int use_max = (mode == NVFP4O_MODE_4OVER6 && rule == NVFP4O_RULE_MAX);

  float b = 0.0f;
  for (int i = 0; i < 16; ++i) {
    float a = fabsf(x[i]);
    if (a > b) b = a;
  }
  out->b = b;
  out->ncand = ncand;

  for (int c = 0; c < ncand; ++c) {
    const float k = G / cands[c];
    const float s = b * k;
    const uint8_t S = nvfp4o_e4m3_encode(s);
    const float d = nvfp4o_e4m3_decode(S) * g;
    float r = G * nvfp4o_e4m3_recip(S);
    if (r > FLT_MAX) r = FLT_MAX;
    out->k[c] = k;
    out->s[c] = s;
    out->S[c] = S;
    out->d[c] = d;
    out->r[c] = r;

    float half[2] = {0.0f, 0.0f};
    for (int i = 0; i < 16; ++i) {
      const float y = x[i] * r;
      const int m = nvfp4o_e2m1_index(fabsf(y));
      const int neg = signbit(x[i]) ? 1 : 0;
      const uint8_t code = (uint8_t)((neg << 3) | m);
      const float v = neg ? -E2M1_VAL[m] : E2M1_VAL[m];
      const float xhat = v * d;
      /* Error against the original value ([FOS, "Adaptive block scaling
       * algorithm"]): the exact difference v*d - x, rounded once. */
      const float delta = fmaf(v, d, -x[i]);
      out->y[c][i] = y;
      out->code[c][i] = code;
      out->xhat[c][i] = xhat;
      out->delta[c][i] = delta;
      float* h = &half[i >> 3];
      if (use_max)
        *h = fmaxf(*h, fabsf(delta));
      else if (use_mae)
        *h = *h + fabsf(delta);
      else
        *h = fmaf(delta, delta, *h);
    }
    /* Minimum-maximum-error rule [FOS, "Adaptive block scaling algorithm"]:
     * the block error is the largest |delta|, the larger of the halves'. */
    out->err[c] = use_max ? fmaxf(half[0], half[1]) : half[0] + half[1];
  }
  out->chosen = 0;
  if (ncand == 2 && out->err[1] < out->err[0]) out->chosen = 1;
}

/* ------------------------------------------------------------------------ */
/* Whole tensors                                                             */
/* ------------------------------------------------------------------------ */

static int check_args(int64_t rows, int64_t cols, int block_axis, int mode, int rule) {
  if (rows <= 0 || cols <= 0) return NVFP4O_ERR_SHAPE;
  if (block_axis != NVFP4O_AXIS_ROWS && block_axis != NVFP4O_AXIS_COLS) return NVFP4O_ERR_ENUM;
  if (mode != NVFP4O_MODE_STD && mode != NVFP4O_MODE_4OVER6) return NVFP4O_ERR_ENUM;
  if (rule != NVFP4O_RULE_MSE && rule != NVFP4O_RULE_MAE && rule != NVFP4O_RULE_MAX)
    return NVFP4O_ERR_ENUM;
  if (block_axis == NVFP4O_AXIS_COLS && cols % 16 != 0) return NVFP4O_ERR_SHAPE;
  if (block_axis == NVFP4O_AXIS_ROWS && rows % 16 != 0) return NVFP4O_ERR_SHAPE;
  return NVFP4O_OK;
}

/* Blocks along contiguous memory: x is [n_rows][n_cols], blocks are 16
 * consecutive elements of one row, outputs are row-major in block order. */
static void quantize_row_major(const uint16_t* x, int64_t n_rows, int64_t n_cols, float g, int mode,
                               int rule, uint8_t* packed, uint8_t* scales, uint8_t* selmap,
                               double* err_sum) {
  const int64_t bpr = n_cols / 16;
  const int64_t nblocks = n_rows * bpr;
  double sum = 0.0;
  if (selmap) memset(selmap, 0, (size_t)((nblocks + 7) / 8));
  for (int64_t blk = 0; blk < nblocks; ++blk) {
    float xb[16];
    for (int i = 0; i < 16; ++i) xb[i] = nvfp4o_bf16_to_f32(x[blk * 16 + i]);
    nvfp4o_block_t q;
    nvfp4o_quantize_block(xb, g, mode, rule, &q);
    const int c = q.chosen;
    for (int j = 0; j < 8; ++j)
      packed[blk * 8 + j] = (uint8_t)(q.code[c][2 * j] | (q.code[c][2 * j + 1] << 4));
    scales[blk] = q.S[c];
    if (selmap && c == 1) selmap[blk >> 3] |= (uint8_t)(1u << (blk & 7));
    sum += (double)q.err[c];
  }
  if (err_sum) *err_sum = sum;
}

int nvfp4o_quantize(const uint16_t* x, int64_t rows, int64_t cols, int block_axis, int mode,
                    int rule, int gscale_given, float* gscale, uint8_t* packed, uint8_t* scales,
                    uint8_t* selmap, double* err_sum) {
  int st = check_args(rows, cols, block_axis, mode, rule);
  if (st != NVFP4O_OK) return st;
  if (!x || !gscale || !packed || !scales) return NVFP4O_ERR_NULL;
  float g = gscale_given ? *gscale : nvfp4o_global_scale(nvfp4o_amax(x, rows * cols), mode);
  *gscale = g;
  if (block_axis == NVFP4O_AXIS_COLS) {
    quantize_row_major(x, rows, cols, g, mode, rule, packed, scales, selmap, err_sum);
    return NVFP4O_OK;
  }
  /* Blocks of 16 rows within one column: defined as the row-wise case applied
   * to the transposed tensor. */
  uint16_t* xt = (uint16_t*)malloc((size_t)(rows * cols) * sizeof(uint16_t));
  if (!xt) return NVFP4O_ERR_ALLOC;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) xt[c * rows + r] = x[r * cols + c];
  quantize_row_major(xt, cols, rows, g, mode, rule, packed, scales, selmap, err_sum);
  free(xt);
  return NVFP4O_OK;
}

int nvfp4o_dequantize(const uint8_t* packed, const uint8_t* scales, float g, int64_t rows,
                      int64_t cols, int block_axis, int out_bf16, void* out) {
  int st = check_args(rows, cols, block_axis, NVFP4O_MODE_STD, NVFP4O_RULE_MSE);
  if (st != NVFP4O_OK) return st;
  if (!packed || !scales || !out) return NVFP4O_ERR_NULL;
  /* Stored layout is row-major in block order over [n_rows][n_cols]; for
   * blocks along rows that is the transposed tensor. */
  const int64_t n_rows = block_axis == NVFP4O_AXIS_COLS ? rows : cols;
  const int64_t n_cols = block_axis == NVFP4O_AXIS_COLS ? cols : rows;
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int64_t c = 0; c < n_cols; ++c) {
      const int64_t e = r * n_cols + c;
      const uint8_t byte = packed[e >> 1];
      const uint8_t code = (e & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u);
      const float d = nvfp4o_e4m3_decode(scales[e >> 4]) * g;
      const float xhat = nvfp4o_e2m1_decode(code) * d;
      /* Output index in the caller's [rows][cols] layout. */
      const int64_t o = block_axis == NVFP4O_AXIS_COLS ? e : c * cols + r;
      if (out_bf16)
        ((uint16_t*)out)[o] = nvfp4o_f32_to_bf16(xhat);
      else
        ((float*)out)[o] = xhat;
    }
  }
  return NVFP4O_OK;
}

/* ------------------------------------------------------------------------ */
/* Residual channels [ARC, "Methodology"]                                    */
/* ------------------------------------------------------------------------ */

/* Per-channel statistic of the outlier identification: absmax[c] = max over
 * rows of |x[r][c]|. */
void nvfp4o_channel_absmax(const uint16_t* x, int64_t rows, int64_t cols, float* absmax) {
  for (int64_t c = 0; c < cols; ++c) absmax[c] = 0.0f;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      const float a = fabsf(nvfp4o_bf16_to_f32(x[r * cols + c]));
      if (a > absmax[c]) absmax[c] = a;
    }
}

/* Channels reordered by absolute maximum, largest first; equal maxima keep
 * the lower channel index first.  perm[j] = channel placed at position j.
 * (Insertion into a sorted list: O(cols^2), plain.) */
void nvfp4o_channel_order(const float* absmax, int64_t cols, int32_t* perm) {
  for (int64_t i = 0; i < cols; ++i) {
    int64_t j = i;
    while (j > 0 && absmax[perm[j - 1]] < absmax[i]) {
      perm[j] = perm[j - 1];
      --j;
    }
    perm[j] = (int32_t)i;
  }
}

/* Two-stage quantization of x [rows][cols] with reordered channels.
 * Primary stage: row r's reordered values x[r][perm[j]] quantized in blocks
 * of 16 consecutive positions (nvfp4o_quantize_block), stored as blocks
 * 0 .. cols/16 - 1 of output row r.  Residual stage: for the first nres
 * positions (the largest channels), the residual of each element against
 * its primary reconstruction, x - v*d rounded once, quantized in blocks of 16 with the same tensor scale g and
 * stored as blocks cols/16 .. (cols + nres)/16 - 1.  Output rows hold
 * (cols + nres)/2 code bytes and (cols + nres)/16 scale bytes. */
int nvfp4o_quantize_residual(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* perm,
                             int64_t nres, int mode, int rule, int gscale_given, float* gscale,
                             uint8_t* packed, uint8_t* scales) {
  return nvfp4o_quantize_augmented(x, rows, cols, perm, nres, mode, rule, gscale_given, gscale,
                                   packed, scales, 0);
}

/* The two sides of the augmented product [ARC, "Methodology"].  duplicate = 0:
 * the activation side above (residual blocks appended).  duplicate = 1: the
 * weight side, whose channels matching the residual ones are repeated: the
 * appended blocks hold the same codes and scales as the primary blocks of the
 * first nres positions, so the product over K + nres adds w * (x - v*d) for
 * those channels. */
int nvfp4o_quantize_augmented(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* perm,
                              int64_t nres, int mode, int rule, int gscale_given, float* gscale,
                              uint8_t* packed, uint8_t* scales, int duplicate) {
  int st = check_args(rows, cols, NVFP4O_AXIS_COLS, mode, rule);
  if (st != NVFP4O_OK) return st;
  if (nres < 0 || nres > cols || nres % 16 != 0) return NVFP4O_ERR_SHAPE;
  if (!x || !perm || !gscale || !packed || !scales) return NVFP4O_ERR_NULL;
  for (int64_t j = 0; j < cols; ++j)
    if (perm[j] < 0 || perm[j] >= cols) return NVFP4O_ERR_SHAPE;
  const float g = gscale_given ? *gscale : nvfp4o_global_scale(nvfp4o_amax(x, rows * cols), mode);
  *gscale = g;
  const int64_t bpr = cols / 16, bout = (cols + nres) / 16;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < bpr; ++b) {
      float xb[16];
      for (int i = 0; i < 16; ++i) xb[i] = nvfp4o_bf16_to_f32(x[r * cols + perm[b * 16 + i]]);
      nvfp4o_block_t q;
      nvfp4o_quantize_block(xb, g, mode, rule, &q);
      const int c = q.chosen;
      uint8_t* pk = packed + (r * bout + b) * 8;
      for (int j = 0; j < 8; ++j) pk[j] = (uint8_t)(q.code[c][2 * j] | (q.code[c][2 * j + 1] << 4));
      scales[r * bout + b] = q.S[c];
      if (b * 16 < nres && duplicate) {
        uint8_t* pr = packed + (r * bout + bpr + b) * 8;
        for (int j = 0; j < 8; ++j) pr[j] = pk[j];
        scales[r * bout + bpr + b] = q.S[c];
      } else if (b * 16 < nres) {
        /* Residual x - v*d of the kept candidate, rounded once.  An exact
         * reconstruction leaves +0 (not the -0 that negating delta gives). */
        float res[16];
        for (int i = 0; i < 16; ++i) {
          const uint8_t code = q.code[c][i];
          const float v = (code & 8u) ? -E2M1_VAL[code & 7u] : E2M1_VAL[code & 7u];
          res[i] = fmaf(-v, q.d[c], xb[i]);
        }
        nvfp4o_block_t qr;
        nvfp4o_quantize_block(res, g, mode, rule, &qr);
        const int cr = qr.chosen;
        uint8_t* pr = packed + (r * bout + bpr + b) * 8;
        for (int j = 0; j < 8; ++j)
          pr[j] = (uint8_t)(qr.code[cr][2 * j] | (qr.code[cr][2 * j + 1] << 4));
        scales[r * bout + bpr + b] = qr.S[cr];
      }
    }
  }
  return NVFP4O_OK;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm before the two stages [ARC, "Methodology": the fused kernel]     */
/* ------------------------------------------------------------------------ */

/* Reciprocal RMS of one row of bf16 values, with the operation order fixed
 * here (the page names RMSNorm only; these are readings):
 *   s_v = sum of x*x over the 8 consecutive elements 8v .. 8v+7, sequential
 *         fma from 0 (every product of two bf16 values is exact in binary32);
 *   ss  = pairwise sum of the s_v: the array s_0 .. s_{V-1} is padded with
 *         zeros to P entries (P the smallest power of two >= V, at least 64)
 *         and adjacent pairs are added level by level;
 *   rstd = RN(1 / RN(sqrt(RN(RN(ss / cols) + eps)))).
 * cols is a positive multiple of 8. */
float nvfp4o_rms_rstd(const uint16_t* xrow, int64_t cols, float eps) {
  const int64_t nv = cols / 8;
  int64_t p = 64;
  while (p < nv) p *= 2;
  float* a = (float*)calloc((size_t)p, sizeof(float));
  if (!a) return 0.0f;
  for (int64_t v = 0; v < nv; ++v) {
    float t = 0.0f;
    for (int i = 0; i < 8; ++i) {
      const float x = nvfp4o_bf16_to_f32(xrow[v * 8 + i]);
      t = fmaf(x, x, t);
    }
    a[v] = t;
  }
  for (int64_t n = p; n > 1; n /= 2)
    for (int64_t i = 0; i < n / 2; ++i) a[i] = a[2 * i] + a[2 * i + 1];
  const float ss = a[0];
  free(a);
  const float ms = ss / (float)cols;
  const float var = ms + eps;
  const float sd = sqrtf(var);
  return 1.0f / sd;
}

/* y = bf16(x * rstd), then, with a weight vector, bf16(w[c] * y) (the
 * product of two bf16 values is exact in binary32, so that step rounds
 * once).  x, y: [rows][cols] bf16; w: cols bf16 or NULL. */
int nvfp4o_rmsnorm(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* w, float eps,
                   uint16_t* y) {
  if (!x || !y) return NVFP4O_ERR_NULL;
  if (rows <= 0 || cols <= 0 || cols % 8 != 0) return NVFP4O_ERR_SHAPE;
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* xr = x + r * cols;
    const float rstd = nvfp4o_rms_rstd(xr, cols, eps);
    for (int64_t c = 0; c < cols; ++c) {
      uint16_t t = nvfp4o_f32_to_bf16(nvfp4o_bf16_to_f32(xr[c]) * rstd);
      if (w) t = nvfp4o_f32_to_bf16(nvfp4o_bf16_to_f32(w[c]) * nvfp4o_bf16_to_f32(t));
      y[r * cols + c] = t;
    }
  }
  return NVFP4O_OK;
}

/* ------------------------------------------------------------------------ */
/* W4A4 product [ARC, "Methodology"; MIN, "Background"]                      */
/* ------------------------------------------------------------------------ */

/* Element value without the tensor scale: a = v * dec(S) for the code at
 * position k of a row blocked along k (the AXIS_COLS layout).  At most 6
 * significant bits, so a and a product of two are exact in binary64. */
static double element_value(const uint8_t* packed_row, const uint8_t* scales_row, int64_t k) {
  const uint8_t byte = packed_row[k / 2];
  const uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15u);
  const double v = (code & 8u) ? -(double)E2M1_VAL[code & 7u] : (double)E2M1_VAL[code & 7u];
  return v * (double)nvfp4o_e4m3_decode(scales_row[k / 16]);
}

/* out[m][n] = ga * gb * sum_k a(m,k) * b(n,k) for A [M][K] and B [N][K], both
 * NVFP4 with blocks of 16 along K (packed [rows][K/2], scales [rows][K/16]):
 * Y = X W^T for activations X and a weight W stored [out][in].  The sum runs
 * over k in order in binary64 (each product exact; the sum within
 * K * 2^-53 of sum |a b| of the exact value).  abs_out (nullable) gets
 * ga * gb * sum_k |a(m,k) * b(n,k)|, the scale of any summation error. */
int nvfp4o_gemm(const uint8_t* pa, const uint8_t* sa, float ga, const uint8_t* pb,
                const uint8_t* sb, float gb, int64_t M, int64_t N, int64_t K, double* out,
                double* abs_out) {
  if (!pa || !sa || !pb || !sb || !out) return NVFP4O_ERR_NULL;
  if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return NVFP4O_ERR_SHAPE;
  const double gab = (double)ga * (double)gb;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double sum = 0.0, asum = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double t = element_value(pa + m * (K / 2), sa + m * (K / 16), k) *
                         element_value(pb + n * (K / 2), sb + n * (K / 16), k);
        sum += t;
        asum += fabs(t);
      }
      out[m * N + n] = gab * sum;
      if (abs_out) abs_out[m * N + n] = gab * asum;
    }
  return NVFP4O_OK;
}
