/*
 * nvfp4_oracle.h -- declarations of the CPU oracle (test infrastructure only).
 * The product library has its own header and shares nothing with this one.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  NVFP4O_OK = 0,
  NVFP4O_ERR_NULL = 1,
  NVFP4O_ERR_ENUM = 2,
  NVFP4O_ERR_SHAPE = 3,
  NVFP4O_ERR_ALLOC = 6
};
/* Block axis: 1 = 16 consecutive elements of a row; 0 = 16 consecutive rows of
 * a column (results stored in the layout of the transposed tensor). */
enum { NVFP4O_AXIS_ROWS = 0, NVFP4O_AXIS_COLS = 1 };
enum { NVFP4O_MODE_STD = 0, NVFP4O_MODE_4OVER6 = 1 };
enum { NVFP4O_RULE_MSE = 0, NVFP4O_RULE_MAE = 1, NVFP4O_RULE_MAX = 2 };

/* Everything the oracle computes for one 16-element block.  Candidate index 0
 * maps the block max to 6, index 1 maps it to 4 (4/6 mode only). */
typedef struct {
  float b;           /* block max |x| */
  int ncand;         /* 1 (standard) or 2 (4/6) */
  float k[2];        /* RN(G / c) */
  float s[2];        /* unrounded block scale RN(b * k) */
  uint8_t S[2];      /* E4M3 block scale byte */
  float d[2];        /* decode multiplier RN(dec(S) * g) */
  float r[2];        /* encode multiplier min(RN(G * T[S]), FLT_MAX) */
  float y[2][16];    /* scaled values RN(x * r) */
  uint8_t code[2][16];
  float xhat[2][16]; /* reconstructed values RN(v * d) */
  float delta[2][16]; /* fma(v, d, -x) */
  float err[2];      /* block error (SSE; SAE under the MAE rule; max |delta| under MAX) */
  int chosen;        /* 0 -> max mapped to 6, 1 -> max mapped to 4 */
} nvfp4o_block_t;

float nvfp4o_bf16_to_f32(uint16_t h);
uint16_t nvfp4o_f32_to_bf16(float f);
int nvfp4o_e2m1_index(float a);
float nvfp4o_e2m1_decode(uint8_t code);
float nvfp4o_e4m3_decode(uint8_t S);
uint8_t nvfp4o_e4m3_encode(float s);
float nvfp4o_e4m3_recip(uint8_t S);
void nvfp4o_e2m1_index_array(const float* a, int64_t n, uint8_t* out);
void nvfp4o_e4m3_encode_array(const float* s, int64_t n, uint8_t* out);
float nvfp4o_amax(const uint16_t* x, int64_t n);
float nvfp4o_global_scale(float amax, int mode);
void nvfp4o_quantize_block(const float x[16], float g, int mode, int rule, nvfp4o_block_t* out);
int nvfp4o_quantize(const uint16_t* x, int64_t rows, int64_t cols, int block_axis, int mode,
                    int rule, int gscale_given, float* gscale, uint8_t* packed, uint8_t* scales,
                    uint8_t* selmap, double* err_sum);
/* nvfp4o_quantize (blocks along rows, AXIS_COLS) on `threads` host threads:
 * amax reduced over slices first, then rows split into ranges of a multiple
 * of 8 rows.  Bit-identical outputs; err_sum adds the ranges in order.
 * (nvfp4_oracle_mt.c, for the CPU baseline.) */
int nvfp4o_quantize_mt(const uint16_t* x, int64_t rows, int64_t cols, int mode, int rule,
                       int threads, int gscale_given, float* gscale, uint8_t* packed,
                       uint8_t* scales, uint8_t* selmap, double* err_sum);
int nvfp4o_dequantize(const uint8_t* packed, const uint8_t* scales, float g, int64_t rows,
                      int64_t cols, int block_axis, int out_bf16, void* out);
void nvfp4o_channel_absmax(const uint16_t* x, int64_t rows, int64_t cols, float* absmax);
void nvfp4o_channel_order(const float* absmax, int64_t cols, int32_t* perm);
int nvfp4o_quantize_residual(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* perm,
                             int64_t nres, int mode, int rule, int gscale_given, float* gscale,
                             uint8_t* packed, uint8_t* scales);
int nvfp4o_quantize_augmented(const uint16_t* x, int64_t rows, int64_t cols, const int32_t* perm,
                              int64_t nres, int mode, int rule, int gscale_given, float* gscale,
                              uint8_t* packed, uint8_t* scales, int duplicate);
int nvfp4o_gemm(const uint8_t* pa, const uint8_t* sa, float ga, const uint8_t* pb,
                const uint8_t* sb, float gb, int64_t M, int64_t N, int64_t K, double* out,
                double* abs_out);
float nvfp4o_rms_rstd(const uint16_t* xrow, int64_t cols, float eps);
int nvfp4o_rmsnorm(const uint16_t* x, int64_t rows, int64_t cols, const uint16_t* w, float eps,
                   uint16_t* y);

#ifdef __cplusplus
}
#endif
#endif
