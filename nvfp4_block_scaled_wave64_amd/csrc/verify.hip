// verify.hip -- device codec sweeps used by the test suite.
//
// These entry points run the kernels' own encoders (and, for comparison,
// gfx950's conversion instructions) over ranges of fp32 bit patterns so the
// tests can check them exhaustively against the CPU reference.  They are not
// part of the quantization path.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"
#include "../../include/nvfp4.h"
#include "../../include/nvfp4_verify.h"

namespace nvfp4 {

__global__ __launch_bounds__(kThreads) void e2m1_sweep_kernel(uint32_t first, int64_t count,
                                                              int impl, uint8_t* out) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kThreads) {
    const float a = __uint_as_float(first + (uint32_t)i);
    uint32_t code;
    if (impl == 0) {
      code = e2m1_index(e2m1_round(fabsf(a))) | ((__float_as_uint(a) >> 28) & 8u);
    } else {
      code = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, 0.0f, 1.0f, 0) & 0xFu;
    }
    out[i] = (uint8_t)code;
  }
}

__global__ __launch_bounds__(kThreads) void e4m3_sweep_kernel(uint32_t first, int64_t count,
                                                              int impl, uint8_t* out) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kThreads) {
    const float s = __uint_as_float(first + (uint32_t)i);
    uint32_t S;
    if (impl == 0) {
      S = e4m3_encode(s);
    } else {
      const float c = fminf(fmaxf(s, 0.0f), 448.0f);
      S = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false) & 0xFFu;
    }
    out[i] = (uint8_t)S;
  }
}

__global__ void decode_tables_kernel(int impl, float* e2m1, float* e4m3, float* rcp) {
  const uint32_t t = threadIdx.x;
  if (t < 16) {
    if (impl == 0) {
      e2m1[t] = __uint_as_float(((t & 7u) << 22) | ((t & 8u) << 28)) * 0x1p126f;
    } else {
      const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(t, 1.0f, 0);
      e2m1[t] = v[0];
    }
  }
  if (t < 128) {
    const float dec = e4m3_decode(t);
    e4m3[t] = dec;
    rcp[t] = (impl == 0) ? ((t == 0) ? 0.0f : 1.0f / dec) : __builtin_amdgcn_rcpf(dec);
  }
}

static int64_t sweep_groups(int64_t count) {
  int64_t g = (count + kThreads - 1) / kThreads;
  if (g > 16384) g = 16384;
  return g < 1 ? 1 : g;
}

}  // namespace nvfp4

extern "C" {

nvfp4_status nvfp4v_e2m1_encode_sweep(uint32_t first_bits, int64_t count, int impl,
                                      uint8_t* codes_out, void* stream) {
  if (!codes_out) return NVFP4_ERR_NULL;
  if (impl != 0 && impl != 1) return NVFP4_ERR_ENUM;
  if (count <= 0 || (uint64_t)first_bits + (uint64_t)count > (1ull << 32)) return NVFP4_ERR_SHAPE;
  nvfp4::e2m1_sweep_kernel<<<(unsigned)nvfp4::sweep_groups(count), nvfp4::kThreads, 0,
                             (hipStream_t)stream>>>(first_bits, count, impl, codes_out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4v_e4m3_encode_sweep(uint32_t first_bits, int64_t count, int impl,
                                      uint8_t* codes_out, void* stream) {
  if (!codes_out) return NVFP4_ERR_NULL;
  if (impl != 0 && impl != 1) return NVFP4_ERR_ENUM;
  if (count <= 0 || (uint64_t)first_bits + (uint64_t)count > (1ull << 32)) return NVFP4_ERR_SHAPE;
  nvfp4::e4m3_sweep_kernel<<<(unsigned)nvfp4::sweep_groups(count), nvfp4::kThreads, 0,
                             (hipStream_t)stream>>>(first_bits, count, impl, codes_out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4v_decode_tables(int impl, float* e2m1_out, float* e4m3_out, float* rcp_out,
                                  void* stream) {
  if (!e2m1_out || !e4m3_out || !rcp_out) return NVFP4_ERR_NULL;
  if (impl != 0 && impl != 1) return NVFP4_ERR_ENUM;
  nvfp4::decode_tables_kernel<<<1, 128, 0, (hipStream_t)stream>>>(impl, e2m1_out, e4m3_out,
                                                                  rcp_out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // extern "C"
