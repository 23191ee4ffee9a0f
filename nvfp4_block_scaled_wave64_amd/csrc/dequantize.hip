// dequantize.hip -- NVFP4 dequantization: x_hat = dec(code) * (dec(S) * g),
// each product one binary32 rounding, i.e. exactly the reconstruction the
// quantizer measured its error against ("Technical summary: Four Over Six
// (4/6)", "Adaptive block scaling algorithm": errors against the original
// values).
//
// A lane handles 8 consecutive stored elements: one dword of codes and the
// scale byte of their block.  E2M1 decode is exact bit placement: the 3-bit
// magnitude index at bit 22 of a binary32 word is value * 2^-126 (0.5 lands
// on a subnormal), so one multiply by 2^126 restores it, sign included.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

__device__ __forceinline__ float e2m1_value(uint32_t code) {
  return __uint_as_float(((code & 7u) << 22) | ((code & 8u) << 28)) * 0x1p126f;
}

__device__ __forceinline__ uint32_t to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool kBf16, bool kTransposed>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ gscale, int64_t n_rows, int64_t n_cols, void* __restrict__ out) {
  // The stored tensor is [n_rows][n_cols] in block order; for blocks along
  // the columns of x it is the transpose of the caller's [n_cols][n_rows].
  const float g = *gscale;
  const int64_t nunits = n_rows * n_cols / 8;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < nunits;
       u += (int64_t)gridDim.x * kThreads) {
    const uint32_t word = packed[u];
    const float d = e4m3_decode(scales[u >> 1]) * g;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = e2m1_value(word >> (4 * i)) * d;
    if (!kTransposed) {
      if (kBf16) {
        uint4 o;
        o.x = to_bf16_rne(v[0]) | (to_bf16_rne(v[1]) << 16);
        o.y = to_bf16_rne(v[2]) | (to_bf16_rne(v[3]) << 16);
        o.z = to_bf16_rne(v[4]) | (to_bf16_rne(v[5]) << 16);
        o.w = to_bf16_rne(v[6]) | (to_bf16_rne(v[7]) << 16);
        reinterpret_cast<uint4*>(out)[u] = o;
      } else {
        float4* o = reinterpret_cast<float4*>(out) + 2 * u;
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    } else {
      const int64_t e = u * 8;  // first stored element: row c of x^T, col r
      const int64_t c = e / n_cols, r = e % n_cols;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t o = (r + i) * n_rows + c;  // x is [n_cols][n_rows]
        if (kBf16)
          reinterpret_cast<uint16_t*>(out)[o] = (uint16_t)to_bf16_rne(v[i]);
        else
          reinterpret_cast<float*>(out)[o] = v[i];
      }
    }
  }
}

hipError_t launch_dequantize(const uint8_t* packed, const uint8_t* scales, const float* gscale,
                             int64_t rows, int64_t cols, int block_axis, int out_bf16, void* out,
                             hipStream_t s) {
  const bool tr = block_axis == 0;
  const int64_t n_rows = tr ? cols : rows, n_cols = tr ? rows : cols;
  const int64_t nunits = rows * cols / 8;
  int64_t groups = (nunits + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (groups > cap) groups = cap;
  if (groups < 1) groups = 1;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
  if (out_bf16) {
    if (tr)
      dequantize_kernel<true, true><<<(unsigned)groups, kThreads, 0, s>>>(p, scales, gscale, n_rows, n_cols, out);
    else
      dequantize_kernel<true, false><<<(unsigned)groups, kThreads, 0, s>>>(p, scales, gscale, n_rows, n_cols, out);
  } else {
    if (tr)
      dequantize_kernel<false, true><<<(unsigned)groups, kThreads, 0, s>>>(p, scales, gscale, n_rows, n_cols, out);
    else
      dequantize_kernel<false, false><<<(unsigned)groups, kThreads, 0, s>>>(p, scales, gscale, n_rows, n_cols, out);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
