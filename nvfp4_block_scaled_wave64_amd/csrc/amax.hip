// amax.hip -- tensor amax (grid reduction), global scale and small set-up
// kernels.
//
// The per-tensor scale of NVFP4 is formed from the tensor's absolute maximum
// ("Technical summary: Four Over Six (4/6)", gist.science 2512.02010,
// "Implementation details": 6*448 for standard NVFP4, 6*256 under 4/6).
//
// amax is a pure 2-byte-per-element read.  Each lane reads 16 bytes (8 bf16)
// per step, clears the sign bits and keeps a packed pair of 16-bit maxima
// (non-negative bf16 bit patterns order like unsigned integers, so the max of
// the patterns is the pattern of the max).  Waves reduce with cross-lane
// shuffles, workgroups through LDS, and each workgroup issues one atomic max
// on the fp32 bit pattern of its result.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

__global__ void init_kernel(uint32_t* zero_u32, double* zero_f64, uint32_t* zero_words,
                            int64_t nwords) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    if (zero_u32) *zero_u32 = 0u;
    if (zero_f64) *zero_f64 = 0.0;
  }
  for (int64_t w = i; w < nwords; w += (int64_t)gridDim.x * blockDim.x) zero_words[w] = 0u;
}

// amax reads with 16-byte non-temporal buffer loads, kAmaxUnroll of them in
// flight per lane (grid-stride), from kAmaxGroupsPerCu workgroups of 4 waves
// per compute unit.  Measured on MI355X (32768 x 5120 bf16): 4 waves per CU
// with 8 loads each stream at about 7.3 TB/s, 8 waves with 4 loads at 7.1,
// while 32 waves with one load each reach about 5.4 TB/s -- fewer, deeper
// streams keep fewer DRAM pages open at once.  Loads past the end read 0
// (range-checked), which leaves the maximum unchanged.
constexpr int kAmaxUnroll = 8;
constexpr int kAmaxGroupsPerCu = 1;

__global__ __launch_bounds__(kThreads) void amax_kernel(const uint16_t* __restrict__ in,
                                                        uint32_t nvec,
                                                        const uint16_t* __restrict__ tail,
                                                        int ntail, float six_m,
                                                        uint32_t* __restrict__ acc) {
  __shared__ uint32_t part[kWavesPerGroup];
  const __amdgpu_buffer_rsrc_t r = make_rsrc(in, nvec * 16u);
  uint32_t m = 0u;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < nvec; i += kAmaxUnroll * stride) {
    u32x4 w[kAmaxUnroll];
#pragma unroll
    for (int k = 0; k < kAmaxUnroll; ++k)
      w[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (i + k * stride) * 16u, 0, kStreamLoad);
#pragma unroll
    for (int k = 0; k < kAmaxUnroll; ++k) {
      const uint32_t a = max_u16x2(w[k].x & 0x7FFF7FFFu, w[k].y & 0x7FFF7FFFu);
      const uint32_t b = max_u16x2(w[k].z & 0x7FFF7FFFu, w[k].w & 0x7FFF7FFFu);
      m = max_u16x2(m, max_u16x2(a, b));
    }
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) m = max_u16x2(m, tail[threadIdx.x] & 0x7FFFu);
  uint32_t v = max(m & 0xFFFFu, m >> 16) << 16;  // fp32 bit pattern of |x|max
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t rr = part[0];
    for (int k = 1; k < kWavesPerGroup; ++k) rr = max(rr, part[k]);
    // Non-negative fp32 values order like their bit patterns, and so do
    // their quotients by six_m > 0 (one rounded division, monotone in A).
    if (six_m > 0.0f) rr = __float_as_uint(__uint_as_float(rr) / six_m);
    atomicMax(acc, rr);
  }
}

__global__ void global_scale_kernel(const float* amax, float six_m, float* gscale) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *gscale = *amax / six_m;
}

hipError_t launch_init(uint32_t* zero_u32, double* zero_f64, uint32_t* zero_words, int64_t nwords,
                       hipStream_t s) {
  int64_t blocks = (nwords + kThreads - 1) / kThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  init_kernel<<<(unsigned)blocks, kThreads, 0, s>>>(zero_u32, zero_f64, zero_words, nwords);
  return hipGetLastError();
}

hipError_t launch_amax(const uint16_t* in, int64_t numel, float six_m, uint32_t* acc_bits,
                       hipStream_t s) {
  // Segments of at most 2^27 vectors (2 GiB) keep buffer offsets in 32 bits
  // (the furthest offset is below 2^31 + kAmaxUnroll * grid * 16 bytes);
  // every segment folds into the same accumulator.
  constexpr int64_t kSegVec = int64_t(1) << 27;
  const int64_t nvec = numel / 8;
  const int ntail = (int)(numel % 8);
  const int64_t cap = (int64_t)device_cu_count() * kAmaxGroupsPerCu;
  int64_t v0 = 0;
  do {
    const int64_t nv = nvec - v0 < kSegVec ? nvec - v0 : kSegVec;
    const bool last = v0 + nv >= nvec;
    int64_t groups = (nv + kThreads - 1) / kThreads;
    if (groups > cap) groups = cap;
    if (groups < 1) groups = 1;
    amax_kernel<<<(unsigned)groups, kThreads, 0, s>>>(in + v0 * 8, (uint32_t)nv, in + nvec * 8,
                                                      last ? ntail : 0, six_m, acc_bits);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    v0 += nv;
  } while (v0 < nvec);
  return hipSuccess;
}

hipError_t launch_global_scale(const float* amax, float six_m, float* gscale, hipStream_t s) {
  global_scale_kernel<<<1, 64, 0, s>>>(amax, six_m, gscale);
  return hipGetLastError();
}

}  // namespace nvfp4
