// dequantize.hip -- NVFP4 dequantization: x_hat = dec(code) * (dec(S) * g),
// each product one binary32 rounding, i.e. exactly the reconstruction the
// quantizer measured its error against ("Technical summary: Four Over Six
// (4/6)", "Adaptive block scaling algorithm": errors against the original
// values).
//
// Blocks along the row (the stored layout is the caller's layout): the same
// work layout as the row-wise quantizer, reversed.  A wave step is a chunk
// of 64 blocks; lane l owns block l of the chunk: one 8-byte code load and
// one scale byte (range-checked buffer loads, issued a chunk ahead), E2M1
// decode with gfx950's packed FP4 conversion, one multiply by d per element
// and, for bf16 output, gfx950's round-to-nearest-even v_cvt_pk_bf16_f32.
// Four v_permlane32_swap moves then give each lane pair one block's two
// 16-byte halves in the order of the output, so each store instruction
// writes 1 KiB contiguously (the inverse of the quantizer's load pairing).
//
// Blocks along the column (stored as the transpose): a lane handles 8
// consecutive stored elements and writes them with strided stores.  E2M1
// decode there is exact bit placement: the 3-bit magnitude index at bit 22
// of a binary32 word is value * 2^-126 (0.5 lands on a subnormal), so one
// multiply by 2^126 restores it, sign included.
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

// Blocks along the column: the stored tensor is [n_rows][n_cols] in block
// order, the transpose of the caller's [n_cols][n_rows].
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void dequantize_transposed_kernel(
    const uint32_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ gscale, int64_t n_rows, int64_t n_cols, void* __restrict__ out) {
  const float g = *gscale;
  const int64_t nunits = n_rows * n_cols / 8;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < nunits;
       u += (int64_t)gridDim.x * kThreads) {
    const uint32_t word = packed[u];
    const float d = e4m3_decode(scales[u >> 1]) * g;
    const int64_t e = u * 8;  // first stored element: row c of x^T, col r
    const int64_t c = e / n_cols, r = e % n_cols;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = e2m1_value(word >> (4 * i)) * d;
      const int64_t o = (r + i) * n_rows + c;  // x is [n_cols][n_rows]
      if (kBf16)
        reinterpret_cast<uint16_t*>(out)[o] = (uint16_t)to_bf16_rne(v);
      else
        reinterpret_cast<float*>(out)[o] = v;
    }
  }
}

#ifndef NVFP4_DEQ_STORE_AUX
#define NVFP4_DEQ_STORE_AUX 16
#endif
// Cache policy of the output stores.
constexpr int kDeqStore = NVFP4_DEQ_STORE_AUX;

template <bool kBf16>
__global__ __launch_bounds__(kRowsThreads) void dequantize_rows_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ gscale, int64_t nblocks, void* __restrict__ out) {
  constexpr uint32_t kOutBlock = kBf16 ? 32u : 64u;  // output bytes per block
  const float g = *gscale;
  const uint32_t nb = (uint32_t)nblocks;  // <= 2^25 per launch
  const __amdgpu_buffer_rsrc_t r_codes = make_rsrc(packed, nb * 8u);
  const __amdgpu_buffer_rsrc_t r_scales = make_rsrc(scales, nb);
  const __amdgpu_buffer_rsrc_t r_out = make_rsrc(out, nb * kOutBlock);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t nchunks = (nb + 63u) / 64u;
  const uint32_t nwaves = gridDim.x * kRowsWaves;
  const uint32_t first = blockIdx.x * kRowsWaves + (threadIdx.x >> 6);
  const uint32_t off_pair = (lane & 31u) * 32u + (lane >> 5) * 16u;  // bf16 output pairing

  struct In {
    u32x2 c;
    uint32_t s;
  };
  // Chunks past the end read zeros; ch stays below nchunks + 2 * nwaves.
  auto load = [&](uint32_t ch) -> In {
    In t;
    t.c = __builtin_amdgcn_raw_buffer_load_b64(r_codes, ch * 512u + lane * 8u, 0, kStreamLoad);
    t.s = __builtin_amdgcn_raw_buffer_load_b8(r_scales, ch * 64u + lane, 0, kStreamLoad);
    return t;
  };
  In nxt = load(first);
  for (uint32_t ch = first; ch < nchunks; ch += nwaves) {
    const In cur = nxt;
    nxt = load(ch + nwaves);
    const float d = e4m3_decode(cur.s & 0xFFu) * g;
    float v[16];
    e2m1_decode8(cur.c.x, v);
    e2m1_decode8(cur.c.y, v + 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= d;
    if (kBf16) {
      uint32_t h[8];  // bf16 pairs: elements 2j (low half) and 2j+1
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x2 p = {v[2 * j], v[2 * j + 1]};
        h[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
      }
      u32x4 a, b;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const auto p = __builtin_amdgcn_permlane32_swap(h[j], h[4 + j], false, false);
        a[j] = p[0];
        b[j] = p[1];
      }
      __builtin_amdgcn_raw_buffer_store_b128(a, r_out, ch * 2048u + off_pair, 0, kDeqStore);
      __builtin_amdgcn_raw_buffer_store_b128(b, r_out, ch * 2048u + 1024u + off_pair, 0,
                                             kDeqStore);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 o;
        o.x = __float_as_uint(v[4 * q]);
        o.y = __float_as_uint(v[4 * q + 1]);
        o.z = __float_as_uint(v[4 * q + 2]);
        o.w = __float_as_uint(v[4 * q + 3]);
        __builtin_amdgcn_raw_buffer_store_b128(o, r_out, ch * 4096u + lane * 64u + q * 16u, 0,
                                               kDeqStore);
      }
    }
  }
}

hipError_t launch_dequantize(const uint8_t* packed, const uint8_t* scales, const float* gscale,
                             int64_t rows, int64_t cols, int block_axis, int out_bf16, void* out,
                             hipStream_t s) {
  const bool tr = block_axis == 0;
  if (!tr) {
    // Segments of at most 2^25 blocks keep every buffer offset (up to 64
    // output bytes per block) within 32 bits.
    constexpr int64_t kSeg = int64_t(1) << 25;
    const int64_t nblocks = rows * cols / 16;
    const int64_t cap = (int64_t)device_cu_count() * (kGroupsPerCu > 0 ? kGroupsPerCu : 1);
    for (int64_t b0 = 0; b0 < nblocks; b0 += kSeg) {
      const int64_t nb = nblocks - b0 < kSeg ? nblocks - b0 : kSeg;
      int64_t groups = ((nb + 63) / 64 + kRowsWaves - 1) / kRowsWaves;
      if (groups > cap) groups = cap;
      if (groups < 1) groups = 1;
      if (out_bf16)
        dequantize_rows_kernel<true><<<(unsigned)groups, kRowsThreads, 0, s>>>(
            packed + b0 * 8, scales + b0, gscale, nb, static_cast<uint8_t*>(out) + b0 * 32);
      else
        dequantize_rows_kernel<false><<<(unsigned)groups, kRowsThreads, 0, s>>>(
            packed + b0 * 8, scales + b0, gscale, nb, static_cast<uint8_t*>(out) + b0 * 64);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int64_t n_rows = cols, n_cols = rows;
  const int64_t nunits = rows * cols / 8;
  int64_t groups = (nunits + kThreads - 1) / kThreads;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (groups > cap) groups = cap;
  if (groups < 1) groups = 1;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
  if (out_bf16)
    dequantize_transposed_kernel<true><<<(unsigned)groups, kThreads, 0, s>>>(p, scales, gscale,
                                                                             n_rows, n_cols, out);
  else
    dequantize_transposed_kernel<false><<<(unsigned)groups, kThreads, 0, s>>>(p, scales, gscale,
                                                                              n_rows, n_cols, out);
  return hipGetLastError();
}

}  // namespace nvfp4
