/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 block-scaled quantization
 * library with "Four Over Six" (4/6) adaptive block scales.
 *
 * The format (NVFP4): 4-bit E2M1 element codes packed two per byte, one FP8
 * E4M3 scale per block of 16 elements, one fp32 scale per tensor.
 *   - blocks of 16 elements: "Why Gated DeltaNet in hybrid 27B LLMs
 *     withstands 4-bit quantization" (sns.style), "Deep analysis"; "ARCQuant"
 *     summary (gist.science 2601.07475), "Problem definition";
 *   - E2M1 grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} and the standard max->6 block
 *     scaling: "Technical summary: Four Over Six (4/6)" (gist.science
 *     2512.02010), "Problem statement";
 *   - the max->4 alternative, quantizing each block both ways and keeping the
 *     one with the lower error under one of three rules (maximum error, MAE,
 *     MSE): same page, "Core mechanism" and "Adaptive block scaling
 *     algorithm";
 *   - E4M3 block scales and the tensor scale formed with 256 instead of 448
 *     under 4/6: same page, "Implementation details".
 *
 * Arithmetic (every step one IEEE binary32 operation, round to nearest even):
 *   g   = A / (6*M)   A = max |x|, M = 448 (standard) or 256 (4/6)
 *   G   = 1/g, or 0 when that is not a positive finite number
 *   per block, for c in {6} (standard) or {6, 4} (4/6):
 *     s_c = b * (G / c)               b = max |x| over the block
 *     S_c = E4M3(s_c)                 round to nearest even, saturating at 448
 *     d_c = dec(S_c) * g              decode multiplier
 *     r_c = min(G * (1/dec(S_c)), FLT_MAX), and 0 when S_c == 0
 *     code_i = sign(x_i) | E2M1(|x_i * r_c|)   nearest even, saturating at 6
 *     e_c = sum of delta_i^2 (MSE), of |delta_i| (MAE), or max |delta_i|
 *           (maximum error), delta_i = dec(code_i) * d_c - x_i evaluated
 *           exactly and rounded once (fused multiply-add); sums run as two
 *           sequential halves of 8 elements (fused multiply-add for the
 *           squares) and are then added; the maximum is exact
 *   keep c = 4 iff e_4 < e_6 (ties go to 6).
 *
 * Conventions shared by every call:
 *   - Every pointer is caller-owned DEVICE memory (e.g. torch tensors); the
 *     library allocates nothing and keeps no pointer after returning.  One
 *     exception: nvfp4_gemm_splitk_noalloc uses a fixed scratch array the
 *     library holds on each device it runs on.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued on it; no call synchronizes the host.
 *   - Arguments are checked before any HIP call, in the order null pointers,
 *     enums, shape, alignment, aliasing.  On a failed check nothing is launched and
 *     nothing is written.  NVFP4_ERR_HIP reports a failed launch; device
 *     faults surface at the caller's next synchronization.
 *   - Tensors are row-major [rows][cols] bf16 bit patterns.  Non-finite
 *     inputs are outside the contract.
 *   - Calls on different streams may run concurrently; they share no state
 *     (nvfp4_gemm_splitk_noalloc aside: its calls share the device's
 *     scratch, so calls of it that overlap in time on one device race).
 *   - Alignment: bf16 inputs and dequantized outputs 16 bytes; packed codes
 *     and the selection bitmap 4 bytes; err_sum 8 bytes; scalars 4 bytes.
 *
 * Layouts.  Block axis NVFP4_AXIS_COLS (=1): a block is 16 consecutive
 * elements of one row; packed is [rows][cols/2] with element 2j in bits 0-3
 * of byte j and element 2j+1 in bits 4-7; scales is [rows][cols/16]; block b
 * (row-major block order) owns bit (b & 7) of byte b >> 3 of the selection
 * bitmap (1 = the max->4 candidate was kept).  Block axis NVFP4_AXIS_ROWS
 * (=0): a block is 16 consecutive rows of one column and every output is laid
 * out as the NVFP4_AXIS_COLS output of the transposed tensor: packed
 * [cols][rows/2], scales [cols][rows/16], bitmap bit c*(rows/16) + rb.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,  /* a required pointer is NULL                        */
  NVFP4_ERR_ENUM = 2,  /* block_axis, mode, rule, out_dtype, flags or eps invalid */
  NVFP4_ERR_SHAPE = 3, /* non-positive extent, or block-axis extent % 16 != 0 */
  NVFP4_ERR_ALIGN = 4, /* a pointer violates the alignment listed above      */
  NVFP4_ERR_HIP = 5,   /* a kernel launch failed                            */
  NVFP4_ERR_ALIAS = 6, /* an output aliases an input it must not overwrite  */
  NVFP4_ERR_SCRATCH = 7 /* more scratch needed than the library's fixed buffer */
} nvfp4_status;

enum { NVFP4_AXIS_ROWS = 0, NVFP4_AXIS_COLS = 1 };
enum { NVFP4_MODE_STD = 0, NVFP4_MODE_4OVER6 = 1 };
enum { NVFP4_RULE_MSE = 0, NVFP4_RULE_MAE = 1, NVFP4_RULE_MAX = 2 }; /* ignored for NVFP4_MODE_STD */
enum { NVFP4_OUT_F32 = 0, NVFP4_OUT_BF16 = 1 };
enum {
  NVFP4_FLAG_GSCALE_GIVEN = 1u,   /* use *gscale_inout as g; skip the amax pass          */
  NVFP4_FLAG_ERR_ACCUMULATE = 2u, /* add the error sum to *err_sum_out, do not zero it  */
  NVFP4_FLAG_STATS_ACCUMULATE = 4u, /* fold channel maxima into *absmax_inout's values   */
  NVFP4_FLAG_RESIDUAL_DUPLICATE = 8u /* appended blocks repeat the primary ones (weights)  */
};

/* Tensor amax A = max |x| over `numel` bf16 values, written as fp32 to
 * *amax_out (device).  numel >= 1.  The global scale of the pages is formed
 * from it ("Technical summary: Four Over Six (4/6)", "Implementation
 * details").  *amax_out is used as the accumulator, so it must not alias the
 * input. */
nvfp4_status nvfp4_amax(const uint16_t* in_bf16, int64_t numel, float* amax_out, void* stream);

/* Global (per-tensor) decode scale g = A / (6*M) from a device amax, with
 * M = 448 for NVFP4_MODE_STD and 256 for NVFP4_MODE_4OVER6 ("Technical
 * summary: Four Over Six (4/6)", "Implementation details").  amax and
 * gscale_out may be the same pointer. */
nvfp4_status nvfp4_global_scale(const float* amax, int mode, float* gscale_out, void* stream);

/* Quantize a [rows][cols] bf16 tensor.  Computes A and g itself and writes g
 * to *gscale_out, then the packed codes and the E4M3 scale bytes (sizes
 * rows*cols/2 and rows*cols/16 bytes).  mode: NVFP4_MODE_STD (every block's
 * max mapped to 6) or NVFP4_MODE_4OVER6 (both candidates, keep the lower
 * error under `rule`) -- "Technical summary: Four Over Six (4/6)",
 * "Adaptive block scaling algorithm". */
nvfp4_status nvfp4_quantize(const uint16_t* in_bf16, int64_t rows, int64_t cols, int block_axis,
                            int mode, int rule, uint8_t* packed_out, uint8_t* scales_out,
                            float* gscale_out, void* stream);

/* As nvfp4_quantize, plus:
 *   flags & NVFP4_FLAG_GSCALE_GIVEN: read g from *gscale_inout instead of
 *     computing it (a calibrated or shared tensor scale); g must be finite
 *     and in [0, 2^117].  Without the flag g is computed and written there.
 *   selmap_out (nullable): the selection bitmap, ceil(rows*cols/128) bytes;
 *     bits past the last block are written as 0.  All zero in standard mode.
 *   err_sum_out (nullable): one double that receives the sum over blocks of
 *     the kept candidate's block error -- squared error under
 *     NVFP4_RULE_MSE and in standard mode, absolute error under
 *     NVFP4_RULE_MAE, the block's largest absolute error under
 *     NVFP4_RULE_MAX -- accumulated in binary64 in an unspecified order.
 *     The call zeroes it first unless flags has NVFP4_FLAG_ERR_ACCUMULATE,
 *     in which case the sum is added to its current value (e.g. a total over
 *     several tensors, or a value the caller zeroed on the same stream).
 *     Divide by rows*cols for the per-tensor MSE / MAE (by the number of
 *     blocks for the mean block maximum error).
 *   Outputs -- packed_out, scales_out, gscale_inout, selmap_out,
 *   err_sum_out -- must not overlap the input or each other
 *   (NVFP4_ERR_ALIAS). */
nvfp4_status nvfp4_quantize_ex(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                               int block_axis, int mode, int rule, uint32_t flags,
                               uint8_t* packed_out, uint8_t* scales_out, float* gscale_inout,
                               uint8_t* selmap_out, double* err_sum_out, void* stream);

/* As nvfp4_quantize_ex, and in addition binds two events to the
 * quantization kernels of the call: start_event takes the start timestamp of
 * the first one and stop_event the end timestamp of the last one (hipEvent_t
 * handles passed as void*, created with timing enabled; either may be NULL).
 * hipEventElapsedTime over the pair is then the execution time of the
 * quantization kernels alone -- the zeroing and amax kernels and the dispatch
 * gaps around them fall outside -- i.e. the figure a kernel profiler reports.
 * Argument checks and errors as nvfp4_quantize_ex; on an error the events
 * are not recorded. */
nvfp4_status nvfp4_quantize_ex_timed(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                                     int block_axis, int mode, int rule, uint32_t flags,
                                     uint8_t* packed_out, uint8_t* scales_out,
                                     float* gscale_inout, uint8_t* selmap_out,
                                     double* err_sum_out, void* start_event, void* stop_event,
                                     void* stream);

/* Both block layouts from one read of x: the row-blocked outputs
 * (packed_r [rows][cols/2], scales_r [rows][cols/16], selmap_r, err_sum_r:
 * those of nvfp4_quantize_ex with NVFP4_AXIS_COLS) and the column-blocked
 * outputs (packed_c [cols][rows/2], scales_c [cols][rows/16], selmap_c,
 * err_sum_c: those of NVFP4_AXIS_ROWS), with one tensor scale g.  Each set
 * is bit-identical to the single-layout call with the same g.  For a tensor
 * used along both of its dimensions (activations, weights and gradients in
 * training: "Technical summary: Four Over Six (4/6)", "Key contributions"),
 * this reads x once instead of twice.
 *   rows and cols: positive multiples of 16.
 *   selmap_r / selmap_c and err_sum_r / err_sum_c: both or neither
 *     (NVFP4_ERR_NULL otherwise); the error sums are zeroed first unless
 *     flags has NVFP4_FLAG_ERR_ACCUMULATE.
 *   flags, gscale_inout, mode, rule, alignment: as nvfp4_quantize_ex.
 *   No output may overlap the input or another output (NVFP4_ERR_ALIAS). */
nvfp4_status nvfp4_quantize_dual(const uint16_t* in_bf16, int64_t rows, int64_t cols, int mode,
                                 int rule, uint32_t flags, uint8_t* packed_r, uint8_t* scales_r,
                                 uint8_t* packed_c, uint8_t* scales_c, float* gscale_inout,
                                 uint8_t* selmap_r, uint8_t* selmap_c, double* err_sum_r,
                                 double* err_sum_c, void* stream);

/* Delayed scaling: quantize with a given tensor scale and record this
 * tensor's amax for the next call, in one pass over the input (no separate
 * amax read).  The per-tensor scale of NVFP4 is formed from the amax
 * ("Technical summary: Four Over Six (4/6)", "Implementation details"); a
 * calibrated or previous-step amax gives the same format with a scale that
 * lags by one call.
 *   gscale_in: device pointer to g (e.g. nvfp4_global_scale of the previous
 *     call's *amax_out); read only; finite and in [0, 2^117].
 *   amax_out: device float that receives A = max |x| of this tensor (zeroed
 *     by the call first); must not alias gscale_in (NVFP4_ERR_ALIAS).
 *   flags: 0 or NVFP4_FLAG_ERR_ACCUMULATE.  Other arguments, outputs and
 *     checks as nvfp4_quantize_ex with NVFP4_FLAG_GSCALE_GIVEN; the codes,
 *     scales, bitmap and error sum are identical to that call's. */
nvfp4_status nvfp4_quantize_delayed(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                                    int block_axis, int mode, int rule, uint32_t flags,
                                    uint8_t* packed_out, uint8_t* scales_out,
                                    const float* gscale_in, float* amax_out,
                                    uint8_t* selmap_out, double* err_sum_out, void* stream);

/* Dequantize: x_hat = dec(code) * (dec(S) * g), each product one binary32
 * rounding (x_hat is the rounding of the reconstruction dec(code) * d whose
 * error the quantizer measured).
 * out_dtype NVFP4_OUT_F32 writes float, NVFP4_OUT_BF16 writes the bf16
 * (round to nearest even) of it.  `out` is [rows][cols] in the caller's
 * layout for either block axis; packed/scales are laid out as produced by
 * nvfp4_quantize with the same block_axis.  A scale byte 0x7F (the E4M3
 * NaN code, never written by the quantizers themselves) decodes to NaN.
 * out must not overlap packed, scales or gscale (NVFP4_ERR_ALIAS). */
nvfp4_status nvfp4_dequantize(const uint8_t* packed, const uint8_t* scales, const float* gscale,
                              int64_t rows, int64_t cols, int block_axis, int out_dtype,
                              void* out, void* stream);

/* Outlier channels, step 1 (calibration): the per-channel statistic and the
 * channel order of the "ARCQuant" summary (gist.science 2601.07475),
 * "Methodology" -- channels ranked by their absolute maximum.
 *   in_bf16: [rows][cols] activations (channels are columns).
 *   absmax_inout: cols floats; receives absmax[c] = max_r |x[r][c]|.  With
 *     flags NVFP4_FLAG_STATS_ACCUMULATE the maxima are folded into the
 *     values already there (non-negative floats, e.g. a previous call's
 *     output: a running maximum over calibration batches); otherwise the
 *     call zeroes them first.
 *   perm_out: cols int32; perm_out[k] = the channel of rank k, largest
 *     maximum first, equal maxima in increasing channel order.
 *   cols: a positive multiple of 16, at most 32768.  absmax_inout and
 *   perm_out must not overlap each other or the input (NVFP4_ERR_ALIAS). */
nvfp4_status nvfp4_channel_order(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                                 uint32_t flags, float* absmax_inout, int32_t* perm_out,
                                 void* stream);

/* Whether a channel order is a permutation of [0, cols): writes to *bad_out
 * (device uint32) the number of entries that keep it from being one, i.e.
 * cols minus the number of distinct values of perm inside [0, cols) -- 0
 * for a valid order.  The orders of the "ARCQuant" summary (gist.science
 * 2601.07475, "Methodology") reorder the channels, so an order given to
 * nvfp4_quantize_residual is expected to be a permutation.
 *   perm: cols int32 (device); cols in [1, 32768].
 *   bad_out must not overlap perm (NVFP4_ERR_ALIAS). */
nvfp4_status nvfp4_check_order(const int32_t* perm, int64_t cols, uint32_t* bad_out,
                               void* stream);

/* Outlier channels, step 2 (per step): two-stage quantization with
 * reordered channels ("ARCQuant" summary, gist.science 2601.07475,
 * "Methodology": the leading channels get a residual stage, x minus its
 * first-stage reconstruction, quantized again and appended along the
 * reduction dimension).  Output row r holds W = cols + nres channels:
 *   block j < cols/16: the 16 values x[r][perm[16j + i]], quantized as by
 *     nvfp4_quantize_ex (NVFP4_AXIS_COLS) with tensor scale g;
 *   block cols/16 + j, j < nres/16: the residual of block j, each element
 *     x - dec(code) * d rounded once (an exact reconstruction gives +0),
 *     quantized the same way with the same g, mode and rule.
 *   packed_out [rows][W/2] and scales_out [rows][W/16], layouts as
 *   nvfp4_quantize; dequantizing them as a [rows][W] tensor and adding
 *   column cols + k to column k (k < nres) reconstructs the reordered x.
 *   perm: cols int32 (device), normally nvfp4_channel_order's, i.e. a
 *     permutation of the channels ("Methodology": channels are reordered).
 *     Entries inside [0, cols) are gathered as given (a repeated channel is
 *     read twice; nvfp4_check_order tells whether perm is a permutation).
 *     If any entry lies outside [0, cols), the call fails on the device:
 *     every output scale byte is written as 0x7F (the E4M3 NaN code) and
 *     every code as 0, so that nvfp4_dequantize of the result, and any
 *     product over it, is NaN rather than plausible numbers (the host call
 *     cannot see device data; check perm first where that matters).
 *   nres: residual channels, a multiple of 16 in [0, cols].
 *   cols: a positive multiple of 16, at most 32768.
 *   flags: 0 (g computed from the tensor amax as nvfp4_quantize does and
 *     written to *gscale_inout) or NVFP4_FLAG_GSCALE_GIVEN (read g from it),
 *     optionally with NVFP4_FLAG_RESIDUAL_DUPLICATE: the weight side of the
 *     augmented product (same page: the weight channels matching the
 *     residual ones are duplicated), where block cols/16 + j repeats the
 *     codes and scale of block j instead of quantizing a residual.  With it,
 *     nvfp4_gemm over K = cols + nres of an activation quantized without the
 *     flag and a weight [out][cols] quantized with it (the same perm and
 *     nres) adds w * (x - dec(code) * d) for the nres leading channels.
 *   Outputs must not overlap the input, perm or each other (NVFP4_ERR_ALIAS). */
nvfp4_status nvfp4_quantize_residual(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                                     const int32_t* perm, int64_t nres, int mode, int rule,
                                     uint32_t flags, uint8_t* packed_out, uint8_t* scales_out,
                                     float* gscale_inout, void* stream);

/* Outlier channels with RMSNorm in front, in one pass over x: the fused
 * kernel of the "ARCQuant" summary (gist.science 2601.07475),
 * "Methodology" -- channel reordering, RMSNorm, the primary and the residual
 * stage.  The result is that of nvfp4_quantize_residual applied to
 * y = RMSNorm(x), bf16 [rows][cols], defined here as
 *   ss   = sum over the row of x^2: per 8 consecutive elements a sequential
 *          fma sum, those sums added pairwise (zero-padded power-of-two tree)
 *   rstd = 1 / sqrt(ss / cols + eps)   (each step one IEEE binary32 operation)
 *   y    = bf16(w[c] * bf16(x * rstd)), w = 1 without a weight vector
 * (bf16 rounding to nearest even).
 *   weight_bf16: cols bf16 (16-byte aligned), or NULL.
 *   eps: finite and >= 0 (NVFP4_ERR_ENUM otherwise).
 *   cols: a positive multiple of 16, at most 24576 (rows of up to 8192
 *     channels are held one per wave in LDS, wider ones shared by a workgroup).
 *   flags: 0 -- a first pass over x computes g from max |y| (g = A/(6M) as
 *     nvfp4_quantize) and writes it to *gscale_inout; or
 *     NVFP4_FLAG_GSCALE_GIVEN -- read g from *gscale_inout (one pass).
 *   amax_out (nullable): receives max |y| of this tensor (for a delayed
 *     scale); must not overlap *gscale_inout.
 *   perm, nres, mode, rule, packed_out, scales_out: as
 *   nvfp4_quantize_residual.  Outputs must not overlap the inputs or each
 *   other (NVFP4_ERR_ALIAS). */
nvfp4_status nvfp4_rmsnorm_quantize_residual(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                                             const uint16_t* weight_bf16, float eps,
                                             const int32_t* perm, int64_t nres, int mode,
                                             int rule, uint32_t flags, uint8_t* packed_out,
                                             uint8_t* scales_out, float* gscale_inout,
                                             float* amax_out, void* stream);

/* W4A4 product of two NVFP4 tensors blocked along the reduction axis:
 *   out[m][n] = ga * gb * sum over k of a(m,k) * b(n,k),  a = v * dec(S)
 * with v the E2M1 value of the code and dec(S) its block's E4M3 scale: a
 * linear layer Y = X W^T with NVFP4 activations X [m][k] and weights W
 * [n][k] ("Why Gated DeltaNet in hybrid 27B LLMs withstands 4-bit
 * quantization", "Background": W4A4), and the augmented product of the
 * "ARCQuant" summary ("Methodology": one GEMM over K_in + S; pass the
 * outputs of nvfp4_quantize_residual without and with
 * NVFP4_FLAG_RESIDUAL_DUPLICATE and k = cols + nres).
 *   a_packed [m][k/2], a_scales [m][k/16], *a_gscale: A in the
 *     NVFP4_AXIS_COLS layout of nvfp4_quantize (e.g. its outputs);
 *   b_packed [n][k/2], b_scales [n][k/16], *b_gscale: B likewise.
 *   out: [m][n] row-major, fp32 (out_dtype NVFP4_OUT_F32) or bf16
 *     (NVFP4_OUT_BF16, the fp32 result rounded to nearest even).
 * Arithmetic: a(m,k) and b(n,k) are exact in binary16 and their products in
 * fp32 (matrix cores, fp32 accumulation); the sum runs in fp32 in an order
 * the library chooses, then is multiplied by RN(ga * gb).  So
 *   |out - exact| <= (k + k/16 + 2) * 2^-23 * ga * gb * sum_k |a b|
 * (plus the bf16 rounding with NVFP4_OUT_BF16).  For a given library
 * build every output is summed in an order fixed by k alone: results are
 * deterministic and do not depend on m, n or the device's compute-unit
 * count (which choose the tile shape).
 *   k: a positive multiple of 16, at most 2^24; n positive, at most 2^24;
 *     m positive; each of m*n, m*k and n*k at most 2^46.
 *   Alignment: packed codes 4 bytes, scalars 4 bytes, out 4 (fp32) or 2
 *   (bf16) bytes.  out must not overlap any input (NVFP4_ERR_ALIAS). */
nvfp4_status nvfp4_gemm(const uint8_t* a_packed, const uint8_t* a_scales, const float* a_gscale,
                        const uint8_t* b_packed, const uint8_t* b_scales, const float* b_gscale,
                        int64_t m, int64_t n, int64_t k, int out_dtype, void* out, void* stream);

/* The product of nvfp4_gemm with the reduction axis split into `splits`
 * contiguous ranges of whole 128-wide chunks of k, computed side by side
 * (products with few output tiles, e.g. decode-sized m, would otherwise
 * leave most compute units idle while a few walk all of k), then added.
 *   workspace: caller-owned device memory of workspace_floats fp32 values,
 *     at least splits * m * n, 4-byte aligned, overlapping no input or the
 *     output; its contents on entry do not matter and on return are the
 *     per-range sums (unscaled).  The library allocates nothing.
 *   splits: 1 .. min(64, ceil(k / 128)) (NVFP4_ERR_SHAPE otherwise); see
 *     nvfp4_gemm_splits_hint.
 *   Other arguments, layouts, checks and the error bound as nvfp4_gemm.
 * Each range is summed in fp32 as nvfp4_gemm sums all of k, the range sums
 * are then added in order in fp32 and multiplied by RN(ga * gb): results
 * are deterministic for a given split count, and with splits = 1 equal
 * nvfp4_gemm's bit for bit. */
nvfp4_status nvfp4_gemm_splitk(const uint8_t* a_packed, const uint8_t* a_scales,
                               const float* a_gscale, const uint8_t* b_packed,
                               const uint8_t* b_scales, const float* b_gscale, int64_t m,
                               int64_t n, int64_t k, int splits, int out_dtype, void* out,
                               float* workspace, int64_t workspace_floats, void* stream);

/* nvfp4_gemm_splitk for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same product, kernels and result -- bit for bit that of
 * nvfp4_gemm_splitk with the same split count -- with the per-range sums
 * kept in a scratch buffer the library owns instead of a caller workspace.
 *   The scratch is a fixed device array of 2^23 fp32 values (32 MiB) that
 *     every device the library runs on holds until the process ends; its
 *     address on a device is looked up on the first call made with that
 *     device current.  splits * m * n must be at most 2^23
 *     (NVFP4_ERR_SCRATCH otherwise, before any HIP call).  The call itself
 *     allocates nothing.
 *   Every call on a device uses that device's one array, and the array
 *     keeps the last call's sums (each call overwrites every value it reads,
 *     so nothing needs clearing).  Calls that overlap in time on one device
 *     -- on different streams, or from different host threads without
 *     ordering -- race on it and give wrong results; order them on one
 *     stream, or use nvfp4_gemm_splitk with separate workspaces.
 *   Other arguments, checks (those of the workspace aside), layouts and the
 *   error bound: as nvfp4_gemm_splitk. */
nvfp4_status nvfp4_gemm_splitk_noalloc(const uint8_t* a_packed, const uint8_t* a_scales,
                                       const float* a_gscale, const uint8_t* b_packed,
                                       const uint8_t* b_scales, const float* b_gscale, int64_t m,
                                       int64_t n, int64_t k, int splits, int out_dtype,
                                       void* out, void* stream);

/* Split count suggested for an m x n x k nvfp4_gemm_splitk on the current
 * device: the count with the lowest time under a model of the launch
 * (rounds of units over the compute units, the per-chunk cost of the tile
 * shape used, the extra pass over the workspace), each range keeping at
 * least four 128-wide chunks of k; 1 where splitting does not help (then
 * nvfp4_gemm is the faster call).  Host only; returns 0 for shapes
 * nvfp4_gemm rejects. */
int nvfp4_gemm_splits_hint(int64_t m, int64_t n, int64_t k);

/* Static description of a status code. */
const char* nvfp4_status_string(nvfp4_status s);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
