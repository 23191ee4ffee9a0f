/*
 * nvfp4_verify.h -- device codec sweeps exported for the test suite.
 *
 * They apply the quantization kernels' own E2M1 / E4M3 encoders (impl 0) --
 * or, for comparison, gfx950's conversion instructions (impl 1) -- to a
 * contiguous range of fp32 bit patterns, so that tests can compare them with
 * the CPU reference over every input.  The formats are those of NVFP4:
 * E2M1 element codes on {0, 0.5, 1, 1.5, 2, 3, 4, 6} and E4M3 block scales
 * ("Technical summary: Four Over Six (4/6)", gist.science 2512.02010,
 * "Problem statement" and "Implementation details").  Not part of the
 * quantization path.  Same conventions as nvfp4.h: device pointers, stream
 * as void*, checks before any HIP call.
 */
#ifndef NVFP4_VERIFY_H
#define NVFP4_VERIFY_H

#include <stdint.h>

#include "nvfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* codes_out[i] = E2M1 code (sign in bit 3, magnitude index in bits 0-2) of
 * the fp32 value with bit pattern first_bits + i, i < count; round to
 * nearest even, saturating at 6.  impl 0: the kernels' encoder; impl 1: the
 * gfx950 v_cvt_scalef32_pk_fp4_f32 instruction with scale 1.0.  The range
 * must not run past 0xFFFFFFFF.  NaN inputs are outside the contract. */
nvfp4_status nvfp4v_e2m1_encode_sweep(uint32_t first_bits, int64_t count, int impl,
                                      uint8_t* codes_out, void* stream);

/* codes_out[i] = E4M3 byte of the fp32 value with bit pattern first_bits + i:
 * round to nearest even, saturating at 448, 0 for NaN and values <= 0.
 * impl 0: the kernels' encoder; impl 1: v_cvt_pk_fp8_f32 after clamping to
 * [0, 448]. */
nvfp4_status nvfp4v_e4m3_encode_sweep(uint32_t first_bits, int64_t count, int impl,
                                      uint8_t* codes_out, void* stream);

/* Decode tables: e2m1_out[16] = value of each 4-bit code, e4m3_out[128] =
 * value of scale bytes 0..127 and rcp_out[128] = their reciprocals (0 for
 * byte 0).  impl 0: the kernels' own decoders and IEEE division; impl 1:
 * v_cvt_scalef32_pk_f32_fp4 and v_rcp_f32. */
nvfp4_status nvfp4v_decode_tables(int impl, float* e2m1_out, float* e4m3_out, float* rcp_out,
                                  void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_VERIFY_H */
