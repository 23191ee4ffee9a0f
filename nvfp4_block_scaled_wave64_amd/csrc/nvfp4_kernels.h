// nvfp4_kernels.h -- kernel declarations and launch helpers shared by the
// host-side ABI (api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Threads per workgroup of the streaming kernels (4 waves of 64).
constexpr int kThreads = 256;
constexpr int kWavesPerGroup = kThreads / 64;

// Bits of the kernel variant selector.
enum : uint32_t {
  kVarFourOverSix = 1u,  // two candidates (max->6, max->4) instead of max->6 only
  kVarMae = 2u,          // MAE selection rule instead of MSE
  kVarSelmap = 4u,       // write the selection bitmap
  kVarErr = 8u,          // accumulate the per-tensor error sum
};

// ---- amax.hip ----
hipError_t launch_init(uint32_t* zero_u32, double* zero_f64, uint32_t* zero_words,
                       int64_t nwords, hipStream_t s);
hipError_t launch_amax(const uint16_t* in, int64_t numel, uint32_t* acc_bits, hipStream_t s);
hipError_t launch_global_scale(const float* amax, float six_m, float* gscale, hipStream_t s);

// ---- quantize_rows.hip: blocks of 16 contiguous elements ----
hipError_t launch_quantize_rows(const uint16_t* in, int64_t nblocks, const float* gscale,
                                uint32_t variant, uint8_t* packed, uint8_t* scales,
                                uint8_t* selmap, double* err_sum, hipStream_t s);

// ---- quantize_cols.hip: blocks of 16 rows within a column ----
hipError_t launch_quantize_cols(const uint16_t* in, int64_t rows, int64_t cols,
                                const float* gscale, uint32_t variant, uint8_t* packed,
                                uint8_t* scales, uint8_t* selmap, double* err_sum, hipStream_t s);

// ---- dequantize.hip ----
hipError_t launch_dequantize(const uint8_t* packed, const uint8_t* scales, const float* gscale,
                             int64_t rows, int64_t cols, int block_axis, int out_bf16, void* out,
                             hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace nvfp4
