/*
 * nvfp4_verify.h -- device codec sweeps exported for the test suite.
 *
 * They run the quantization kernels' own E2M1 / E4M3 encoders and decoders
 * (the same inline device functions) over fp32 bit patterns or scale bytes,
 * so that tests can compare them with the CPU reference on every input.  The
 * formats are those of NVFP4: E2M1 element codes on
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6} and FP8 E4M3 block scales ("Technical
 * summary: Four Over Six (4/6)", gist.science 2512.02010, "Problem
 * statement" and "Implementation details").  Not part of the quantization
 * path.  Same conventions as nvfp4.h: device pointers, stream as void*,
 * argument checks before any HIP call.
 */
#ifndef NVFP4_VERIFY_H
#define NVFP4_VERIFY_H

#include <stdint.h>

#include "nvfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* codes_out[i] (count bytes) = E2M1 code (sign in bit 3, magnitude index in
 * bits 0-2) of the fp32 value with bit pattern first_bits + i: round to
 * nearest even, saturating at 6.  first_bits + count must not exceed 2^32.
 * NaN inputs are outside the contract (the kernels never produce them). */
nvfp4_status nvfp4v_e2m1_encode_sweep(uint32_t first_bits, int64_t count, uint8_t* codes_out,
                                      void* stream);

/* codes_out[i] (count bytes) = E4M3 byte of the fp32 value with bit pattern
 * first_bits + i: round to nearest even, saturating at 448, 0 for NaN and
 * values <= 0. */
nvfp4_status nvfp4v_e4m3_encode_sweep(uint32_t first_bits, int64_t count, uint8_t* codes_out,
                                      void* stream);

/* Decode tables for a tensor scale g: e2m1_out[16] = value of each 4-bit
 * code; e4m3_out[128] = value of scale bytes 0..127; d_out[128] and
 * r_out[128] = the kernels' per-scale decode multiplier dec(S) * g and encode
 * multiplier min((1/g) * (1/dec(S)), FLT_MAX) (0 for S = 0). */
nvfp4_status nvfp4v_decode_tables(float g, float* e2m1_out, float* e4m3_out, float* d_out,
                                  float* r_out, void* stream);

/* The row-wise quantizer's memory traffic with none of its arithmetic, as
 * the attainable-bandwidth reference for that kernel: over nblocks blocks of
 * 16 bf16 values (in_bf16, 32 bytes each) it writes 8 bytes of packed_out
 * and 1 byte of scales_out per block, with the same launch shape, access
 * order and cache policies as nvfp4_quantize_ex with NVFP4_AXIS_COLS.  The
 * bytes are a fold of the input, not NVFP4 codes: for block b with 32-bit
 * words w0..w7, packed_out[8b..8b+7] = (w0^w1^w2^w3, w4^w5^w6^w7) as two
 * little-endian words, and scales_out[b] = the low byte of their XOR.
 * in_bf16 16-byte and packed_out 8-byte aligned; nblocks in [1, 2^42]. */
nvfp4_status nvfp4v_stream_pattern(const uint16_t* in_bf16, int64_t nblocks, uint8_t* packed_out,
                                   uint8_t* scales_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_VERIFY_H */
