// nvfp4_kernels.h -- kernel declarations and launch helpers shared by the
// host-side ABI (api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

namespace nvfp4 {

// Optional events bound to a launch: `start` takes the kernel's start
// timestamp and `stop` its end timestamp (hipExtLaunchKernel), so their
// elapsed time is the kernel's execution time alone.
struct Events {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launches `kernel` on stream s, binding ev.start / ev.stop (either may be
// null) to it; the arguments are converted to the kernel's parameter types.
template <typename... P, typename... A>
hipError_t launch_with_events(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t s,
                              Events ev, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  std::tuple<P...> vals(args...);
  void* ptrs[sizeof...(P)];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, s,
                            ev.start, ev.stop, 0);
}

// Threads per workgroup of the streaming kernels (4 waves of 64).
constexpr int kThreads = 256;
constexpr int kWavesPerGroup = kThreads / 64;

// Launch shape of the row-wise kernels (quantize_rows.hip, the byte-pattern
// kernel, the row-layout dequantizer): waves per compute unit, threads per
// workgroup, and how many steps the quantizer's waves take between
// workgroup barriers.
#ifndef NVFP4_ROWS_WAVES_PER_CU
#define NVFP4_ROWS_WAVES_PER_CU 16
#endif
#ifndef NVFP4_ROWS_THREADS
#define NVFP4_ROWS_THREADS 1024
#endif
#ifndef NVFP4_ROWS_SYNC_EVERY
#define NVFP4_ROWS_SYNC_EVERY 1
#endif
constexpr int kRowsSyncEvery = NVFP4_ROWS_SYNC_EVERY;
// One workgroup of 16 waves per compute unit: the 16 consecutive chunks a
// workgroup handles in one round write whole 128-byte lines of the bitmap
// (16 x 8 bytes) and of the scales from one XCD, and the error sum takes one
// atomic per compute unit.
constexpr int kRowsThreads = NVFP4_ROWS_THREADS;
constexpr int kRowsWaves = kRowsThreads / 64;
constexpr int kGroupsPerCu = NVFP4_ROWS_WAVES_PER_CU / kRowsWaves;

// Bits of the kernel variant selector.
enum : uint32_t {
  kVarFourOverSix = 1u,  // two candidates (max->6, max->4) instead of max->6 only
  kVarMae = 2u,          // MAE selection rule instead of MSE
  kVarMax = 16u,         // minimum-maximum-error selection rule instead of MSE
  kVarSelmap = 4u,       // write the selection bitmap
  kVarErr = 8u,          // accumulate the per-tensor error sum
  kVarAmax = 32u,        // also fold the tensor's max |x| into amax_out (row kernel)
};

// ---- amax.hip ----
hipError_t launch_init(uint32_t* zero_u32, double* zero_f64, uint32_t* zero_words,
                       int64_t nwords, hipStream_t s);
// Atomic max of A = max |x| into *acc_bits (fp32 bit pattern, zeroed by the
// caller), or of g = A / six_m when six_m > 0: division by a positive
// constant rounds monotonically, so the max over workgroups of A_wg / six_m
// is the rounded quotient of the tensor's A.
hipError_t launch_amax(const uint16_t* in, int64_t numel, float six_m, uint32_t* acc_bits,
                       hipStream_t s);
hipError_t launch_global_scale(const float* amax, float six_m, float* gscale, hipStream_t s);

// ---- quantize_rows.hip: blocks of 16 contiguous elements ----
// amax_out (nullable): receives, by atomic max on its fp32 bit pattern, the
// largest block max |x| of the tensor (the caller zeroes it first).
hipError_t launch_quantize_rows(const uint16_t* in, int64_t nblocks, const float* gscale,
                                uint32_t variant, uint8_t* packed, uint8_t* scales,
                                uint8_t* selmap, double* err_sum, uint32_t* amax_out,
                                hipStream_t s, Events ev);

// ---- quantize_cols.hip: blocks of 16 rows within a column ----
// Row-blocked outputs of a dual call (both block layouts from one read).
struct DualOut {
  uint8_t* packed_r;
  uint8_t* scales_r;
  uint8_t* selmap_r;  // nullable
  double* err_r;      // nullable (only with kVarErr)
};
hipError_t launch_quantize_cols(const uint16_t* in, int64_t rows, int64_t cols,
                                const float* gscale, uint32_t variant, uint8_t* packed,
                                uint8_t* scales, uint8_t* selmap, double* err_sum,
                                uint32_t* amax_out, const DualOut* dual, hipStream_t s,
                                Events ev);

// ---- dequantize.hip ----
hipError_t launch_dequantize(const uint8_t* packed, const uint8_t* scales, const float* gscale,
                             int64_t rows, int64_t cols, int block_axis, int out_bf16, void* out,
                             hipStream_t s);

// ---- residual.hip: outlier channels with a residual stage ----
// Atomic max of each column's max |x| into absmax_bits[c] (fp32 bit
// patterns; the caller zeroes them, or keeps earlier values to fold several
// tensors).
hipError_t launch_channel_absmax(const uint16_t* in, int64_t rows, int64_t cols,
                                 uint32_t* absmax_bits, hipStream_t s);
// *bad = the number of entries keeping perm from being a permutation of
// [0, cols) (cols - distinct in-range values); cols <= kResidualMaxCols.
hipError_t launch_check_order(const int32_t* perm, int64_t cols, uint32_t* bad, hipStream_t s);
// perm[k] = the channel of rank k (largest max first, ties by index).
hipError_t launch_channel_rank(const uint32_t* absmax_bits, int64_t cols, int32_t* perm,
                               hipStream_t s);
// Primary blocks of the reordered channels and residual blocks of the first
// nres of them (with dup: copies of their primary blocks); cols <=
// kResidualMaxCols (LDS holds a row and the order).
constexpr int64_t kResidualMaxCols = 32768;
hipError_t launch_quantize_residual(const uint16_t* in, int64_t rows, int64_t cols,
                                    const int32_t* perm, int64_t nres, const float* gscale,
                                    uint32_t variant, uint8_t* packed, uint8_t* scales, bool dup,
                                    hipStream_t s);

// RMSNorm in front of the residual path: y = bf16(x * rstd), then
// bf16(w * y) with a weight vector; amax_out (fp32 bits, nullable) receives
// max |y| by atomic max (the caller zeroes it).
struct RmsArgs {
  const uint16_t* weight;  // cols bf16 (16-byte aligned), or null
  float eps;
  uint32_t* amax_out;
};
constexpr int64_t kRmsMaxCols = 8192;       // one row per wave in LDS
constexpr int64_t kRmsWideMaxCols = 24576;  // rows shared by a workgroup, wider ones
hipError_t launch_rms_quantize_residual(const uint16_t* in, int64_t rows, int64_t cols,
                                        const int32_t* perm, int64_t nres, const float* gscale,
                                        uint32_t variant, uint8_t* packed, uint8_t* scales,
                                        const RmsArgs& ra, hipStream_t s);
// ---- gemm.hip: W4A4 product of two NVFP4 tensors blocked along K ----
// out [M][N] (fp32, or bf16 when out_bf16) = ga * gb * sum_k a(m,k) b(n,k).
hipError_t launch_gemm(const uint8_t* pa, const uint8_t* sa, const float* ga, const uint8_t* pb,
                       const uint8_t* sb, const float* gb, int64_t M, int64_t N, int64_t K,
                       int out_bf16, void* out, hipStream_t s, Events ev);
// The same with K split into `splits` (1 .. min(kGemmMaxSplits, K/128
// rounded up)) contiguous ranges: raw fp32 sums into ws [splits][M][N], then
// one pass adds the slices in order and scales them.
constexpr int kGemmMaxSplits = 64;
hipError_t launch_gemm_splitk(const uint8_t* pa, const uint8_t* sa, const float* ga,
                              const uint8_t* pb, const uint8_t* sb, const float* gb, int64_t M,
                              int64_t N, int64_t K, uint32_t splits, int out_bf16, void* out,
                              float* ws, hipStream_t s);
// Suggested split count for an M x N x K product on the current device.
int gemm_splits_hint(int64_t M, int64_t N, int64_t K);

// Atomic max of RN(max |y| / six_m) into *acc (fp32 bits; the caller zeroes it).
hipError_t launch_rms_amax(const uint16_t* in, int64_t rows, int64_t cols, const RmsArgs& ra,
                           float six_m, uint32_t* acc, hipStream_t s);

// ---- verify.hip: the row quantizer's memory traffic without its arithmetic ----
hipError_t launch_stream_pattern(const uint16_t* in, int64_t nblocks, uint8_t* packed,
                                 uint8_t* scales, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace nvfp4
