// residual.hip -- outlier channels with a residual NVFP4 stage.
//
// Method ("ARCQuant" summary, gist.science 2601.07475, "Methodology"): the
// channels (columns of an activation tensor [tokens][channels], the
// reduction dimension of the GEMM it feeds) are ranked by their absolute
// maximum; the top channels get a second quantization stage over what the
// first stage left, x - x_hat, and those residual blocks are appended along
// the reduction dimension, so that one NVFP4 GEMM over cols + nres channels
// adds the compensation by itself.
//
// Three kernels:
//   channel_absmax_kernel  absmax[c] = max_r |x[r][c]|: a pure 2-byte-per-
//       element read.  A workgroup owns a tile of 512 columns (64 lanes x 8
//       bf16 per 16-byte load) and a range of rows; its 8 waves interleave
//       the rows, keep packed 16-bit maxima (non-negative bf16 patterns order
//       like integers), meet in LDS, and issue one atomic max per column on
//       the fp32 bit pattern (which orders the same way).
//   channel_rank_kernel    perm[rank(c)] = c with rank(c) = the number of
//       channels with a larger maximum, or an equal one and a lower index
//       (largest first, stable).  O(cols^2) comparisons against LDS tiles of
//       the maxima; a few microseconds at transformer widths, and run once
//       per calibration, not per step.
//   quantize_residual_kernel  the per-step pass.  A workgroup stages R whole
//       rows in LDS with coalesced 16-byte loads (the next rows' loads are in
//       flight while it works on the current ones), keeps the channel order
//       in LDS as 16-bit indices, and gives each thread one output block: it
//       gathers the block's 16 channels from LDS, quantizes them (the same
//       block quantizer as the row-wise path), stores the codes and the
//       scale byte, and for the first nres/16 blocks forms the residual
//       x - v*d of the kept codes (one fused multiply-add per element, so an
//       exact reconstruction leaves +0) and quantizes it as a second block
//       with the same tensor scale, stored after the row's primary blocks.
#include <algorithm>

#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

typedef unsigned short ushort2_r __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t max_u16x2_r(uint32_t a, uint32_t b) {
  ushort2_r va = __builtin_bit_cast(ushort2_r, a), vb = __builtin_bit_cast(ushort2_r, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(va, vb));
}

// ---------------------------------------------------------------- absmax --

constexpr int kAbsThreads = 512;
constexpr int kAbsWaves = kAbsThreads / 64;
constexpr int kAbsUnroll = 4;

// Workgroup g owns column tile g % ctiles and row range g / ctiles.
__global__ __launch_bounds__(kAbsThreads) void channel_absmax_kernel(
    const uint16_t* __restrict__ in, int64_t rows, uint32_t cols, uint32_t ctiles,
    int64_t rows_per_group, uint32_t* __restrict__ absmax_bits) {
  __shared__ u32x4 part[kAbsWaves][64];
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
  const uint32_t tile = blockIdx.x % ctiles, split = blockIdx.x / ctiles;
  const uint32_t nvc = cols / 8u;              // 16-byte vectors per row
  const uint32_t cv = tile * 64u + lane;       // this lane's vector column
  const int64_t r0 = (int64_t)split * rows_per_group;
  const int64_t r1 = std::min<int64_t>(rows, r0 + rows_per_group);
  const uint32_t nrows = (uint32_t)(r1 - r0);
  const uint32_t pitch = cols * 2u;
  // The group's rows are below 2^31 bytes (host), so an out-of-tile lane's
  // offset 2^31 + row offset is past the range and reads 0.
  const __amdgpu_buffer_rsrc_t r = make_rsrc(in + r0 * cols, nrows * pitch);
  const uint32_t voff = cv < nvc ? cv * 16u : 0x80000000u;
  u32x4 m = {0u, 0u, 0u, 0u};
  for (uint32_t i = wave; i < nrows; i += kAbsWaves * kAbsUnroll) {
    u32x4 w[kAbsUnroll];
#pragma unroll
    for (int k = 0; k < kAbsUnroll; ++k) {
      const uint32_t row = i + k * kAbsWaves;  // rows past the group's read 0
      w[k] = __builtin_amdgcn_raw_buffer_load_b128(r, voff + row * pitch, 0, kStreamLoad);
    }
#pragma unroll
    for (int k = 0; k < kAbsUnroll; ++k) {
      m.x = max_u16x2_r(m.x, w[k].x & 0x7FFF7FFFu);
      m.y = max_u16x2_r(m.y, w[k].y & 0x7FFF7FFFu);
      m.z = max_u16x2_r(m.z, w[k].z & 0x7FFF7FFFu);
      m.w = max_u16x2_r(m.w, w[k].w & 0x7FFF7FFFu);
    }
  }
  part[wave][lane] = m;
  __syncthreads();
  // Thread t folds word t & 3 (two columns) of lane t >> 2 over the waves.
  if (threadIdx.x < 256u) {
    const uint32_t l = threadIdx.x >> 2, word = threadIdx.x & 3u;
    uint32_t v = 0u;
    for (int k = 0; k < kAbsWaves; ++k) v = max_u16x2_r(v, part[k][l][word]);
    const uint32_t c = (tile * 64u + l) * 8u + word * 2u;
    if (c < cols) {
      if (v & 0xFFFFu) atomicMax(absmax_bits + c, (v & 0xFFFFu) << 16);
      if (v >> 16) atomicMax(absmax_bits + c + 1, v & 0xFFFF0000u);
    }
  }
}

// ------------------------------------------------------------------ rank --

constexpr int kRankThreads = 64;
constexpr uint32_t kRankTile = 1024;

__global__ __launch_bounds__(kRankThreads) void channel_rank_kernel(
    const uint32_t* __restrict__ absmax_bits, uint32_t cols, int32_t* __restrict__ perm) {
  __shared__ uint32_t tile[kRankTile];
  const uint32_t i = blockIdx.x * kRankThreads + threadIdx.x;
  const uint32_t ai = i < cols ? absmax_bits[i] : 0u;
  uint32_t rank = 0u;
  for (uint32_t j0 = 0; j0 < cols; j0 += kRankTile) {
    const uint32_t n = std::min(kRankTile, cols - j0);
    __syncthreads();
    for (uint32_t t = threadIdx.x; t < n; t += kRankThreads) tile[t] = absmax_bits[j0 + t];
    __syncthreads();
    // Non-negative fp32 maxima order like their bit patterns.  Channel j
    // precedes i if larger, or equal with a lower index.
    for (uint32_t t = 0; t < n; ++t) {
      const uint32_t a = tile[t];
      rank += (a > ai) | ((a == ai) & (j0 + t < i));
    }
  }
  if (i < cols) perm[rank] = (int32_t)i;
}

// -------------------------------------------------------------- quantize --

constexpr int kResVec = 4;  // 16-byte staging loads per thread and iteration

template <uint32_t V, int T>
__global__ __launch_bounds__(T) void quantize_residual_kernel(
    const uint16_t* __restrict__ in, int64_t rows, uint32_t cols, const int32_t* __restrict__ perm,
    uint32_t nres, const float* __restrict__ gscale, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales, uint32_t R) {
  constexpr bool k46 = (V & kVarFourOverSix) != 0;
  constexpr int kRule = !k46 ? kRuleMse
                        : (V & kVarMax) ? kRuleMax
                        : (V & kVarMae) ? kRuleMae
                                        : kRuleMse;
  constexpr bool kNeedErr = k46;

  // LDS: scale table (1 KiB), channel order (cols 16-bit indices), R rows.
  extern __shared__ __align__(16) uint8_t lds[];
  float2* tab = reinterpret_cast<float2*>(lds);
  uint16_t* pm = reinterpret_cast<uint16_t*>(lds + 1024);
  uint16_t* xs = pm + cols;  // cols * 2 bytes is a multiple of 32
  u32x4* xs4 = reinterpret_cast<u32x4*>(xs);

  const TensorScales ts = tensor_scales(*gscale);
  build_scale_table(tab, ts);
  // Indices are clamped into the row, so no entry can read outside it.
  for (uint32_t c = threadIdx.x; c < cols; c += T)
    pm[c] = (uint16_t)std::min((uint32_t)perm[c], cols - 1u);

  const uint32_t nb = cols >> 4, nrb = nres >> 4, bout = nb + nrb;
  const uint32_t vrow = cols >> 3;
  const int64_t niter = (rows + R - 1) / R;

  auto rows_at = [&](int64_t it) -> uint32_t {
    return (uint32_t)std::min<int64_t>((int64_t)R, rows - it * R);
  };
  // Rows of one iteration are contiguous: R * cols * 2 bytes from row it*R.
  auto load = [&](int64_t it, u32x4 (&buf)[kResVec]) {
    const uint32_t nv = rows_at(it) * vrow;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(in + it * R * cols, nv * 16u);
#pragma unroll
    for (int k = 0; k < kResVec; ++k)
      buf[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (threadIdx.x + k * T) * 16u, 0,
                                                     kStreamLoad);
  };

  u32x4 buf[kResVec];
  if ((int64_t)blockIdx.x < niter) load(blockIdx.x, buf);
  for (int64_t it = blockIdx.x; it < niter; it += gridDim.x) {
    const uint32_t nr = rows_at(it);
    __syncthreads();  // the previous rows are consumed (and pm, tab written)
#pragma unroll
    for (int k = 0; k < kResVec; ++k) {
      const uint32_t v = threadIdx.x + k * T;
      if (v < nr * vrow) xs4[v] = buf[k];
    }
    __syncthreads();
    if (it + gridDim.x < niter) {
      __builtin_amdgcn_s_setprio(3);
      load(it + gridDim.x, buf);
      __builtin_amdgcn_s_setprio(0);
    }

    const int64_t r0 = it * R;
    const __amdgpu_buffer_rsrc_t r_packed = make_rsrc(packed + r0 * bout * 8, nr * bout * 8u);
    const __amdgpu_buffer_rsrc_t r_scales = make_rsrc(scales + r0 * bout, nr * bout);
    const uint32_t nitems = nr * nb;
    for (uint32_t item = threadIdx.x; item < nitems; item += T) {
      const uint32_t rr = item / nb, j = item - rr * nb;
      const uint16_t* xr = xs + rr * cols;
      const u32x4* p4 = reinterpret_cast<const u32x4*>(pm + j * 16u);
      const u32x4 i0 = p4[0], i1 = p4[1];
      const uint32_t ix[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
      uint32_t wd[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        wd[k] = (uint32_t)xr[ix[k] & 0xFFFFu] | ((uint32_t)xr[ix[k] >> 16] << 16);
      const Block16 q = quantize_block16<k46, kRule, kNeedErr>(wd, ts.k6, ts.k4, tab);
      const uint32_t ob = rr * bout + j;
      u32x2 codes;
      codes.x = q.lo;
      codes.y = q.hi;
      __builtin_amdgcn_raw_buffer_store_b64(codes, r_packed, ob * 8u, 0, kStreamStore);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)q.S, r_scales, ob, 0, kMergedStore);
      if (j < nrb) {
        // Residual of the kept candidate, x - v*d rounded once.
        float v[16], res[16];
        e2m1_decode8(q.lo, v);
        e2m1_decode8(q.hi, v + 8);
        const float d = tab[q.S].x;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          res[2 * k] = __builtin_fmaf(-v[2 * k], d, bf16_lo(wd[k]));
          res[2 * k + 1] = __builtin_fmaf(-v[2 * k + 1], d, bf16_hi(wd[k]));
        }
        const Block16 qr = quantize_block16f<k46, kRule, kNeedErr>(res, ts.k6, ts.k4, tab);
        u32x2 rc;
        rc.x = qr.lo;
        rc.y = qr.hi;
        __builtin_amdgcn_raw_buffer_store_b64(rc, r_packed, (ob + nb) * 8u, 0, kStreamStore);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)qr.S, r_scales, ob + nb, 0, kMergedStore);
      }
    }
  }
}

// ------------------------------------------------------------- launchers --

hipError_t launch_channel_absmax(const uint16_t* in, int64_t rows, int64_t cols,
                                 uint32_t* absmax_bits, hipStream_t s) {
  const int64_t ctiles = (cols / 8 + 63) / 64;
  // About two workgroups per compute unit in total; each group's rows stay
  // below 2^31 bytes so that buffer offsets fit 32 bits.
  const int64_t target = 2 * (int64_t)device_cu_count();
  int64_t splits = std::max<int64_t>(1, target / ctiles);
  int64_t per = (rows + splits - 1) / splits;
  const int64_t cap = ((int64_t(1) << 31) - 1) / (cols * 2) - kAbsWaves * kAbsUnroll;
  if (per > cap) per = cap;
  if (per < 1) per = 1;
  splits = (rows + per - 1) / per;
  channel_absmax_kernel<<<(unsigned)(ctiles * splits), kAbsThreads, 0, s>>>(
      in, rows, (uint32_t)cols, (uint32_t)ctiles, per, absmax_bits);
  return hipGetLastError();
}

hipError_t launch_channel_rank(const uint32_t* absmax_bits, int64_t cols, int32_t* perm,
                               hipStream_t s) {
  const unsigned groups = (unsigned)((cols + kRankThreads - 1) / kRankThreads);
  channel_rank_kernel<<<groups, kRankThreads, 0, s>>>(absmax_bits, (uint32_t)cols, perm);
  return hipGetLastError();
}

template <uint32_t V, int T>
static hipError_t launch_residual_vt(const uint16_t* in, int64_t rows, int64_t cols,
                                     const int32_t* perm, int64_t nres, const float* gscale,
                                     uint8_t* packed, uint8_t* scales, hipStream_t s) {
  // Rows per iteration: enough output blocks for every thread, within the
  // staging capacity of T * kResVec 16-byte vectors.
  const int64_t nb = cols / 16;
  const int64_t cap_rows = (int64_t)T * kResVec * 8 / cols;
  int64_t R = (T + nb - 1) / nb;
  if (R > cap_rows) R = cap_rows;
  if (R < 1) R = 1;
  const size_t lds = 1024 + (size_t)cols * 2 + (size_t)R * cols * 2;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&quantize_residual_kernel<V, T>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t per_cu =
      std::max<int64_t>(1, std::min<int64_t>(163840 / (int64_t)lds, 2048 / T));
  const int64_t niter = (rows + R - 1) / R;
  const int64_t groups = std::max<int64_t>(1, std::min<int64_t>(niter, per_cu * device_cu_count()));
  quantize_residual_kernel<V, T><<<(unsigned)groups, T, lds, s>>>(
      in, rows, (uint32_t)cols, perm, (uint32_t)nres, gscale, packed, scales, (uint32_t)R);
  return hipGetLastError();
}

template <uint32_t V>
static hipError_t launch_residual_v(const uint16_t* in, int64_t rows, int64_t cols,
                                    const int32_t* perm, int64_t nres, const float* gscale,
                                    uint8_t* packed, uint8_t* scales, hipStream_t s) {
  if (cols <= 8192)
    return launch_residual_vt<V, 256>(in, rows, cols, perm, nres, gscale, packed, scales, s);
  return launch_residual_vt<V, 1024>(in, rows, cols, perm, nres, gscale, packed, scales, s);
}

hipError_t launch_quantize_residual(const uint16_t* in, int64_t rows, int64_t cols,
                                    const int32_t* perm, int64_t nres, const float* gscale,
                                    uint32_t variant, uint8_t* packed, uint8_t* scales,
                                    hipStream_t s) {
  switch (variant) {
    case 0: return launch_residual_v<0>(in, rows, cols, perm, nres, gscale, packed, scales, s);
    case 1: return launch_residual_v<1>(in, rows, cols, perm, nres, gscale, packed, scales, s);
    case 3: return launch_residual_v<3>(in, rows, cols, perm, nres, gscale, packed, scales, s);
    case 17: return launch_residual_v<17>(in, rows, cols, perm, nres, gscale, packed, scales, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4
