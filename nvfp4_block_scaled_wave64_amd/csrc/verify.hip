// verify.hip -- device codec sweeps used by the test suite.
//
// These entry points run the quantization kernels' own E2M1 / E4M3 encoders
// and decoders (the same inline functions the kernels call) over ranges of
// fp32 bit patterns, so the tests can compare them with the CPU reference on
// every input.  They are not part of the quantization path.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"
#include "nvfp4.h"
#include "nvfp4_verify.h"

namespace nvfp4 {

// Each thread encodes 8 consecutive patterns in one call of e2m1_encode8, so
// every byte position of the packed conversion is exercised.
__global__ __launch_bounds__(kThreads) void e2m1_sweep_kernel(uint32_t first, int64_t count,
                                                              uint8_t* out) {
  const int64_t ngroups = (count + 7) / 8;
  for (int64_t gidx = (int64_t)blockIdx.x * kThreads + threadIdx.x; gidx < ngroups;
       gidx += (int64_t)gridDim.x * kThreads) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t k = gidx * 8 + i;
      y[i] = __uint_as_float(first + (uint32_t)(k < count ? k : 0));
    }
    const uint32_t w = e2m1_encode8(y);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (gidx * 8 + i < count) out[gidx * 8 + i] = (uint8_t)((w >> (4 * i)) & 15u);
  }
}

__global__ __launch_bounds__(kThreads) void e4m3_sweep_kernel(uint32_t first, int64_t count,
                                                              uint8_t* out) {
  const int64_t npairs = (count + 1) / 2;
  for (int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x; p < npairs;
       p += (int64_t)gridDim.x * kThreads) {
    const int64_t k0 = 2 * p, k1 = 2 * p + 1;
    const float s0 = __uint_as_float(first + (uint32_t)k0);
    const float s1 = __uint_as_float(first + (uint32_t)(k1 < count ? k1 : k0));
    const uint32_t S2 = e4m3_encode2(s0, s1);
    out[k0] = (uint8_t)(S2 & 0xFFu);
    if (k1 < count) out[k1] = (uint8_t)(S2 >> 8);
  }
}

__global__ void decode_tables_kernel(float g, float* e2m1, float* e4m3, float* d, float* r) {
  const uint32_t t = threadIdx.x;
  if (t < 2) {
    float v[8];
    e2m1_decode8(t == 0 ? 0x76543210u : 0xFEDCBA98u, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) e2m1[8 * t + i] = v[i];
  }
  if (t < 128) {
    const TensorScales ts = tensor_scales(g);
    const float2 dr = scale_pair(t, ts);
    e4m3[t] = e4m3_decode(t);
    d[t] = dr.x;
    r[t] = dr.y;
  }
}

// The row quantizer's memory traffic with none of its arithmetic: the same
// launch shape, chunk order, non-temporal 2 x 16-byte loads per lane, lane
// pairing, 8-byte code stores and L2-merged scale-byte stores, writing a
// fold of the input instead of codes.  It moves exactly the quantizer's
// 32 + 8 + 1 bytes per block, so its time is the bandwidth ceiling for that
// pattern and its byte counters calibrate the profiler's.
__global__ __launch_bounds__(kRowsThreads) void stream_pattern_kernel(
    const uint16_t* __restrict__ in, int64_t nblocks, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales) {
  const uint32_t nb = (uint32_t)nblocks;  // <= 2^26 per launch
  const __amdgpu_buffer_rsrc_t r_in = make_rsrc(in, nb * 32u);
  const __amdgpu_buffer_rsrc_t r_packed = make_rsrc(packed, nb * 8u);
  const __amdgpu_buffer_rsrc_t r_scales = make_rsrc(scales, nb);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t off_in = (lane & 31u) * 32u + (lane >> 5) * 16u;
  const uint32_t nchunks = (nb + 63u) / 64u;
  const uint32_t nwaves = gridDim.x * kRowsWaves;
  for (uint32_t ch = blockIdx.x * kRowsWaves + (threadIdx.x >> 6); ch < nchunks; ch += nwaves) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r_in, ch * 2048u + off_in, 0, kStreamLoad);
    const u32x4 b =
        __builtin_amdgcn_raw_buffer_load_b128(r_in, ch * 2048u + 1024u + off_in, 0, kStreamLoad);
    uint32_t f = 0u, h = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto p = __builtin_amdgcn_permlane32_swap(a[j], b[j], false, false);
      f ^= p[0];
      h ^= p[1];
    }
    u32x2 o;
    o.x = f;
    o.y = h;
    __builtin_amdgcn_raw_buffer_store_b64(o, r_packed, ch * 512u + lane * 8u, 0, kStreamStore);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(f ^ h), r_scales, ch * 64u + lane, 0, kMergedStore);
  }
}

hipError_t launch_stream_pattern(const uint16_t* in, int64_t nblocks, uint8_t* packed,
                                 uint8_t* scales, hipStream_t s) {
  constexpr int64_t kSeg = int64_t(1) << 26;
  const int64_t cap = (int64_t)device_cu_count() * (kGroupsPerCu > 0 ? kGroupsPerCu : 1);
  for (int64_t b0 = 0; b0 < nblocks; b0 += kSeg) {
    const int64_t nb = nblocks - b0 < kSeg ? nblocks - b0 : kSeg;
    int64_t groups = ((nb + 63) / 64 + kRowsWaves - 1) / kRowsWaves;
    if (groups > cap) groups = cap;
    if (groups < 1) groups = 1;
    stream_pattern_kernel<<<(unsigned)groups, kRowsThreads, 0, s>>>(in + b0 * 16, nb,
                                                                   packed + b0 * 8, scales + b0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static int64_t sweep_groups(int64_t work) {
  int64_t g = (work + kThreads - 1) / kThreads;
  if (g > 16384) g = 16384;
  return g < 1 ? 1 : g;
}

}  // namespace nvfp4

extern "C" {

nvfp4_status nvfp4v_e2m1_encode_sweep(uint32_t first_bits, int64_t count, uint8_t* codes_out,
                                      void* stream) {
  if (!codes_out) return NVFP4_ERR_NULL;
  if (count <= 0 || (uint64_t)first_bits + (uint64_t)count > (1ull << 32)) return NVFP4_ERR_SHAPE;
  nvfp4::e2m1_sweep_kernel<<<(unsigned)nvfp4::sweep_groups((count + 7) / 8), nvfp4::kThreads, 0,
                             (hipStream_t)stream>>>(first_bits, count, codes_out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4v_e4m3_encode_sweep(uint32_t first_bits, int64_t count, uint8_t* codes_out,
                                      void* stream) {
  if (!codes_out) return NVFP4_ERR_NULL;
  if (count <= 0 || (uint64_t)first_bits + (uint64_t)count > (1ull << 32)) return NVFP4_ERR_SHAPE;
  nvfp4::e4m3_sweep_kernel<<<(unsigned)nvfp4::sweep_groups((count + 1) / 2), nvfp4::kThreads, 0,
                             (hipStream_t)stream>>>(first_bits, count, codes_out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4v_decode_tables(float g, float* e2m1_out, float* e4m3_out, float* d_out,
                                  float* r_out, void* stream) {
  if (!e2m1_out || !e4m3_out || !d_out || !r_out) return NVFP4_ERR_NULL;
  nvfp4::decode_tables_kernel<<<1, 128, 0, (hipStream_t)stream>>>(g, e2m1_out, e4m3_out, d_out,
                                                                  r_out);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4v_stream_pattern(const uint16_t* in_bf16, int64_t nblocks, uint8_t* packed_out,
                                   uint8_t* scales_out, void* stream) {
  if (!in_bf16 || !packed_out || !scales_out) return NVFP4_ERR_NULL;
  if (nblocks <= 0 || nblocks > (int64_t(1) << 42)) return NVFP4_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(in_bf16) & 15u) || (reinterpret_cast<uintptr_t>(packed_out) & 7u))
    return NVFP4_ERR_ALIGN;
  return nvfp4::launch_stream_pattern(in_bf16, nblocks, packed_out, scales_out,
                                      static_cast<hipStream_t>(stream)) == hipSuccess
             ? NVFP4_OK
             : NVFP4_ERR_HIP;
}

}  // extern "C"
