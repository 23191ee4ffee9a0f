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
// Kernels:
//   channel_absmax_kernel  absmax[c] = max_r |x[r][c]|: a pure 2-byte-per-
//       element read.  A workgroup owns a tile of 512 columns (64 lanes x 8
//       bf16 per 16-byte load) and a range of rows; its 8 waves interleave
//       the rows, keep packed 16-bit maxima (non-negative bf16 patterns order
//       like integers), meet in LDS, and issue one atomic max per column on
//       the fp32 bit pattern (which orders the same way).
//   channel_rank_kernel    perm[rank(c)] = c with rank(c) = the number of
//       channels with a larger maximum, or an equal one and a lower index
//       (largest first, stable): O(cols^2) comparisons, one 64-bit compare
//       each, split over 16 waves per 64 channels; run once per calibration,
//       not per step.
//   the per-step pass, in two shapes.  Both keep the channel order in LDS
//       as 16-bit byte offsets into a row and stage whole rows in LDS with
//       coalesced 16-byte loads (the next rows' loads in flight while the
//       current ones are quantized); each output block is then one thread's
//       work: gather the block's 16 channels from LDS, quantize them (the
//       row-wise path's block quantizer), store codes and scale byte, and for
//       the first nres/16 blocks form the residual x - v*d of the kept codes
//       (one fused multiply-add per element, so an exact reconstruction
//       leaves +0) and quantize it as a second block with the same tensor
//       scale, stored after the row's primary blocks.
//     quantize_residual_wave_kernel (cols <= 8192): every wave owns a row
//       buffer and streams its own rows, with no workgroup barrier.  With
//       kRms it applies RMSNorm to each staged row first (the fused kernel
//       of the same section).
//     quantize_residual_kernel (wider rows): a 1024-thread workgroup shares
//       R staged rows per step between two barriers.
//   rms_amax_kernel  the fused path's first pass when the tensor scale is
//       not given: max |RMSNorm(x)| folded into g.
#include <algorithm>
#include <atomic>

#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

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
      m.x = max_u16x2(m.x, w[k].x & 0x7FFF7FFFu);
      m.y = max_u16x2(m.y, w[k].y & 0x7FFF7FFFu);
      m.z = max_u16x2(m.z, w[k].z & 0x7FFF7FFFu);
      m.w = max_u16x2(m.w, w[k].w & 0x7FFF7FFFu);
    }
  }
  part[wave][lane] = m;
  __syncthreads();
  // Thread t folds word t & 3 (two columns) of lane t >> 2 over the waves.
  if (threadIdx.x < 256u) {
    const uint32_t l = threadIdx.x >> 2, word = threadIdx.x & 3u;
    uint32_t v = 0u;
    for (int k = 0; k < kAbsWaves; ++k) v = max_u16x2(v, part[k][l][word]);
    const uint32_t c = (tile * 64u + l) * 8u + word * 2u;
    if (c < cols) {
      if (v & 0xFFFFu) atomicMax(absmax_bits + c, (v & 0xFFFFu) << 16);
      if (v >> 16) atomicMax(absmax_bits + c + 1, v & 0xFFFF0000u);
    }
  }
}

// ------------------------------------------------------------------ rank --

// A workgroup ranks 64 channels (one per lane); its 16 waves split the
// channels compared against, and the partial counts meet in LDS.  Channel
// j precedes i iff key_j > key_i with key = (max bits, ~index): a larger
// maximum, or an equal one and a lower index -- one 64-bit compare per
// pair.  The compared maxima are wave-uniform loads (scalar cache).
constexpr int kRankThreads = 1024;
constexpr int kRankWaves = kRankThreads / 64;

__global__ __launch_bounds__(kRankThreads) void channel_rank_kernel(
    const uint32_t* __restrict__ absmax_bits, uint32_t cols, int32_t* __restrict__ perm) {
  __shared__ uint32_t part[kRankWaves][64];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t i = blockIdx.x * 64u + lane;
  const uint64_t key_i = ((uint64_t)(i < cols ? absmax_bits[i] : 0u) << 32) | (uint32_t)~i;
  const uint32_t per = (cols + kRankWaves - 1) / kRankWaves;
  const uint32_t j0 = std::min(cols, wave * per), j1 = std::min(cols, j0 + per);
  uint32_t rank = 0u;
#pragma unroll 8
  for (uint32_t j = j0; j < j1; ++j) {
    const uint64_t key_j = ((uint64_t)absmax_bits[j] << 32) | (uint32_t)~j;
    rank += key_j > key_i ? 1u : 0u;
  }
  part[wave][lane] = rank;
  __syncthreads();
  if (threadIdx.x < 64u) {
    uint32_t r = 0u;
    for (int k = 0; k < kRankWaves; ++k) r += part[k][lane];
    if (i < cols) perm[r] = (int32_t)i;
  }
}

// -------------------------------------------------------------- quantize --

// Output block j of one staged row xr (bf16 in LDS): gathers the channels
// pm[16j .. 16j+15], quantizes them, stores codes and scale as block ob of
// the output, and with `res` also block ob + nb: the residual block, or with
// `dup` (the weight side of the augmented product) a copy of block ob.
template <bool k46, int kRule>
__device__ __forceinline__ void residual_block(const uint16_t* xr, const uint16_t* pm,
                                               uint32_t j, uint32_t ob, uint32_t nb, bool res,
                                               bool dup,
                                               __amdgpu_buffer_rsrc_t r_packed,
                                               __amdgpu_buffer_rsrc_t r_scales,
                                               const TensorScales& ts, const float2* tab) {
  constexpr bool kNeedErr = k46;
  // pm holds byte offsets into the row, two per dword; each gathered bf16
  // becomes its fp32 value by a 16-bit shift.
  const u32x4* p4 = reinterpret_cast<const u32x4*>(pm + j * 16u);
  const u32x4 i0 = p4[0], i1 = p4[1];
  const uint32_t ix[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(xr);
  float x[16];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x[2 * k] = __uint_as_float(
        (uint32_t)*reinterpret_cast<const uint16_t*>(xb + (ix[k] & 0xFFFFu)) << 16);
    x[2 * k + 1] =
        __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(xb + (ix[k] >> 16)) << 16);
  }
  const Block16 q = quantize_block16f<k46, kRule, kNeedErr>(x, ts.k6, ts.k4, tab);
  u32x2 codes;
  codes.x = q.lo;
  codes.y = q.hi;
  __builtin_amdgcn_raw_buffer_store_b64(codes, r_packed, ob * 8u, 0, kStreamStore);
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)q.S, r_scales, ob, 0, kMergedStore);
  if (res && dup) {
    __builtin_amdgcn_raw_buffer_store_b64(codes, r_packed, (ob + nb) * 8u, 0, kStreamStore);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)q.S, r_scales, ob + nb, 0, kMergedStore);
  } else if (res) {
    // Residual of the kept candidate, x - v*d rounded once.
    float v[16], rx[16];
    e2m1_decode8(q.lo, v);
    e2m1_decode8(q.hi, v + 8);
    const float d = tab[q.S].x;
#pragma unroll
    for (int k = 0; k < 16; ++k) rx[k] = __builtin_fmaf(-v[k], d, x[k]);
    const Block16 qr = quantize_block16f<k46, kRule, kNeedErr>(rx, ts.k6, ts.k4, tab);
    u32x2 rc;
    rc.x = qr.lo;
    rc.y = qr.hi;
    __builtin_amdgcn_raw_buffer_store_b64(rc, r_packed, (ob + nb) * 8u, 0, kStreamStore);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)qr.S, r_scales, ob + nb, 0, kMergedStore);
  }
}

// Wide rows (cols > 8192): a workgroup of 1024 threads stages R rows in LDS
// per step (coalesced 16-byte loads; the group's next rows are in flight
// while it quantizes the current ones) and gives each thread one output
// block at a time.
constexpr int kResThreads = 1024;
constexpr int kResVec = 8;    // 16-byte staging loads per thread and step
constexpr int kResItems = 2;  // output blocks per thread and step, at least

template <uint32_t V>
__global__ __launch_bounds__(kResThreads) void quantize_residual_kernel(
    const uint16_t* __restrict__ in, int64_t rows, uint32_t cols, const int32_t* __restrict__ perm,
    uint32_t nres, const float* __restrict__ gscale, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales, uint32_t R, uint32_t dup) {
  constexpr bool k46 = (V & kVarFourOverSix) != 0;
  constexpr int kRule = !k46 ? kRuleMse
                        : (V & kVarMax) ? kRuleMax
                        : (V & kVarMae) ? kRuleMae
                                        : kRuleMse;

  // LDS: scale table (1 KiB), channel order (cols 16-bit byte offsets), R
  // rows.
  extern __shared__ __align__(16) uint8_t lds[];
  float2* tab = reinterpret_cast<float2*>(lds);
  uint16_t* pm = reinterpret_cast<uint16_t*>(lds + 1024);
  uint16_t* xs = pm + cols;  // cols * 2 bytes is a multiple of 32
  u32x4* xs4 = reinterpret_cast<u32x4*>(xs);

  const TensorScales ts = tensor_scales(*gscale);
  build_scale_table(tab, ts);
  // Byte offsets of the channels in a row; indices are clamped into the
  // row, so no entry can read outside it.
  for (uint32_t c = threadIdx.x; c < cols; c += kResThreads)
    pm[c] = (uint16_t)(2u * std::min((uint32_t)perm[c], cols - 1u));

  const uint32_t nb = cols >> 4, nrb = nres >> 4, bout = nb + nrb;
  const uint32_t vrow = cols >> 3;
  const int64_t niter = (rows + R - 1) / R;

  auto rows_at = [&](int64_t it) -> uint32_t {
    return (uint32_t)std::min<int64_t>((int64_t)R, rows - it * R);
  };
  // Rows of one step are contiguous: R * cols * 2 bytes from row it*R.
  auto load = [&](int64_t it, u32x4 (&buf)[kResVec]) {
    const uint32_t nv = rows_at(it) * vrow;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(in + it * R * cols, nv * 16u);
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int k = 0; k < kResVec; ++k)
      buf[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (threadIdx.x + k * kResThreads) * 16u, 0,
                                                     kStreamLoad);
    __builtin_amdgcn_s_setprio(0);
  };

  // The waves take turns at the extra items (blocks past a multiple of the
  // thread count, residual blocks): the first item rotates one wave per step.
  u32x4 buf[kResVec];
  if ((int64_t)blockIdx.x < niter) load(blockIdx.x, buf);
  uint32_t rot = 0u;
  for (int64_t it = blockIdx.x; it < niter; it += gridDim.x) {
    const uint32_t nr = rows_at(it);
    __syncthreads();  // the previous rows are consumed (and pm, tab written)
#pragma unroll
    for (int k = 0; k < kResVec; ++k) {
      const uint32_t v = threadIdx.x + k * kResThreads;
      if (v < nr * vrow) xs4[v] = buf[k];
    }
    __syncthreads();
    if (it + gridDim.x < niter) load(it + gridDim.x, buf);

    const int64_t r0 = it * R;
    const __amdgpu_buffer_rsrc_t r_packed = make_rsrc(packed + r0 * bout * 8, nr * bout * 8u);
    const __amdgpu_buffer_rsrc_t r_scales = make_rsrc(scales + r0 * bout, nr * bout);
    const uint32_t nitems = nr * nb;
#pragma unroll 1
    for (uint32_t item = (threadIdx.x + rot) & (kResThreads - 1u); item < nitems;
         item += kResThreads) {
      const uint32_t rr = item / nb, j = item - rr * nb;
      residual_block<k46, kRule>(xs + rr * cols, pm, j, rr * bout + j, nb, j < nrb, dup != 0u,
                                 r_packed, r_scales, ts, tab);
    }
    rot = (rot + 64u) & (kResThreads - 1u);
  }
}

// ------------------------------------------------------------ RMSNorm --

// RMSNorm applied in front of the two stages (the fused kernel of the
// "ARCQuant" summary, "Methodology").  The operation order is fixed so that
// any implementation reproduces it bit for bit: per 8 consecutive elements a
// sequential fma sum of squares, those sums added pairwise (a zero-padded
// power-of-two tree), then rstd = 1 / sqrt(ss / cols + eps) with IEEE sqrt
// and division, y = bf16(x * rstd) and, with a weight, bf16(w * y).

constexpr int pow2_at_least(int n) { return n <= 1 ? 1 : 2 * pow2_at_least((n + 1) / 2); }

// Pairwise sum over the 64 lanes, levels in the order of the lane index
// bits (lane l and l ^ 2^k at level k): ds_swizzle exchanges within 32
// lanes, then the two halves' (uniform) values.  Every lane gets the sum.
__device__ __forceinline__ float wave_pair_sum(float t) {
  t = t + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(t), 0x1F | (1 << 10)));
  t = t + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(t), 0x1F | (2 << 10)));
  t = t + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(t), 0x1F | (4 << 10)));
  t = t + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(t), 0x1F | (8 << 10)));
  t = t + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(t), 0x1F | (16 << 10)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 32));
}

// Sum of squares of the row a wave holds as kVpl 16-byte vectors per lane
// (vector v = lane + 64 m covers elements 8v .. 8v+7; vectors past the row
// were loaded as zeros).  Lane xor-shuffles add the pairs of the tree's
// first six levels, the vectors of one lane the rest; every lane ends with
// the same value.
template <int kVpl>
__device__ __forceinline__ float row_sumsq(const u32x4 (&buf)[kVpl]) {
  constexpr int kM = pow2_at_least(kVpl);
  float a[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    a[m] = 0.0f;
    if (m < kVpl) {
      float t = 0.0f;
      t = __builtin_fmaf(bf16_lo(buf[m].x), bf16_lo(buf[m].x), t);
      t = __builtin_fmaf(bf16_hi(buf[m].x), bf16_hi(buf[m].x), t);
      t = __builtin_fmaf(bf16_lo(buf[m].y), bf16_lo(buf[m].y), t);
      t = __builtin_fmaf(bf16_hi(buf[m].y), bf16_hi(buf[m].y), t);
      t = __builtin_fmaf(bf16_lo(buf[m].z), bf16_lo(buf[m].z), t);
      t = __builtin_fmaf(bf16_hi(buf[m].z), bf16_hi(buf[m].z), t);
      t = __builtin_fmaf(bf16_lo(buf[m].w), bf16_lo(buf[m].w), t);
      t = __builtin_fmaf(bf16_hi(buf[m].w), bf16_hi(buf[m].w), t);
      a[m] = wave_pair_sum(t);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int n = kM; n > 1; n >>= 1) {
#pragma unroll
    for (int i = 0; i < n / 2; ++i) a[i] = a[2 * i] + a[2 * i + 1];
  }
  return a[0];
}

__device__ __forceinline__ float rms_rstd(float ss, uint32_t cols, float eps) {
  const float ms = ss / (float)cols;
  const float var = ms + eps;
  const float sd = __builtin_sqrtf(var);
  return 1.0f / sd;
}

// bf16 pair (round to nearest even) of two fp32 values.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 p;
  p.x = lo;
  p.y = hi;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}

// One bf16 pair of y: bf16(x * rstd), then bf16(w * y).  Without a weight
// vector w is 1, which leaves y unchanged (the product is exact).
// ymax keeps the two halves' running max |y| as bf16 bit patterns
// (non-negative bf16 values order like their patterns).
__device__ __forceinline__ uint32_t rms_pair(uint32_t x, uint32_t w, float rstd, uint32_t& ymax) {
  uint32_t y = pack_bf16(bf16_lo(x) * rstd, bf16_hi(x) * rstd);
  y = pack_bf16(bf16_lo(w) * bf16_lo(y), bf16_hi(w) * bf16_hi(y));
  ymax = max_u16x2(ymax, y & 0x7FFF7FFFu);
  return y;
}

// fp32 value of the larger half of a packed bf16 maximum.
__device__ __forceinline__ float bf16_pair_max(uint32_t m) {
  return __uint_as_float(max(m & 0xFFFFu, m >> 16) << 16);
}

// Replaces the row held in buf by y = RMSNorm(x) (bf16) and folds max |y|
// into ymax.  w4: the weight vector in LDS (ones without one), zero-padded
// to 64 * kVpl 16-byte vectors.  Vectors past the row hold zeros and stay
// zero.
template <int kVpl>
__device__ __forceinline__ void rms_apply(u32x4 (&buf)[kVpl], const u32x4* w4, uint32_t lane,
                                          float rstd, uint32_t& ymax) {
  // The widened values of the sum of squares are not reused here: an empty
  // register constraint makes the compiler re-read the packed words, rather
  // than keep 8 fp32 values per vector alive across the reduction.
#pragma unroll
  for (int m = 0; m < kVpl; ++m)
    asm volatile("" : "+v"(buf[m].x), "+v"(buf[m].y), "+v"(buf[m].z), "+v"(buf[m].w));
#pragma unroll
  for (int m = 0; m < kVpl; ++m) {
    const u32x4 w = w4[lane + 64u * m];
    buf[m].x = rms_pair(buf[m].x, w.x, rstd, ymax);
    buf[m].y = rms_pair(buf[m].y, w.y, rstd, ymax);
    buf[m].z = rms_pair(buf[m].z, w.z, rstd, ymax);
    buf[m].w = rms_pair(buf[m].w, w.w, rstd, ymax);
  }
}

// Stages the weight vector in LDS as 64 * kVpl 16-byte vectors: the weights
// (bf16 ones without a weight vector), then zeros.
template <int kVpl>
__device__ __forceinline__ void stage_weight(u32x4* w4, const uint16_t* weight, uint32_t vrow) {
  const u32x4* wg = reinterpret_cast<const u32x4*>(weight);
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  for (uint32_t v = threadIdx.x; v < 64u * kVpl; v += blockDim.x)
    w4[v] = v < vrow ? (weight ? wg[v] : ones) : u32x4{0u, 0u, 0u, 0u};
}

// Wave maximum of a non-negative float, then one atomic max per wave on its
// bit pattern (of m / six_m when six_m > 0: the tensor scale's quotient,
// monotone in m).
__device__ __forceinline__ void wave_max_to(uint32_t* dst, float m, float six_m) {
  uint32_t v = __float_as_uint(m);
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  if ((threadIdx.x & 63u) == 0u) {
    if (six_m > 0.0f) v = __float_as_uint(__uint_as_float(v) / six_m);
    atomicMax(dst, v);
  }
}

// First pass of the fused path when g is not given: max |y| over the
// normalized tensor, folded into *acc as RN(max / six_m) = g.  One row per
// wave, the weight vector in LDS.
// Workgroup size of the kernels that normalize rows of kVpl >= 12 vectors
// per lane: 12 waves, which leaves each wave room for its row, the
// normalization and (fused) the block quantizer in registers.
constexpr int rms_threads(int kVpl) { return kVpl >= 12 ? 768 : 1024; }

template <int kVpl>
__global__ __launch_bounds__(rms_threads(kVpl)) void rms_amax_kernel(const uint16_t* __restrict__ in,
                                                        int64_t rows, uint32_t cols,
                                                        RmsArgs ra, float six_m,
                                                        uint32_t* __restrict__ acc) {
  extern __shared__ __align__(16) uint8_t lds[];
  u32x4* w4 = reinterpret_cast<u32x4*>(lds);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t vrow = cols >> 3;
  stage_weight<kVpl>(w4, ra.weight, vrow);
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x >> 6);
  uint32_t ymax = 0u;
  auto load = [&](int64_t row, u32x4 (&buf)[kVpl]) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(in + row * cols, vrow * 16u);
#pragma unroll
    for (int m = 0; m < kVpl; ++m)
      buf[m] = __builtin_amdgcn_raw_buffer_load_b128(r, (lane + 64u * m) * 16u, 0, kStreamLoad);
  };
  // The next row's loads are in flight while the current row is reduced.
  const int64_t first = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  u32x4 nxt[kVpl];
  if (first < rows) load(first, nxt);
  for (int64_t row = first; row < rows; row += stride) {
    u32x4 buf[kVpl];
#pragma unroll
    for (int m = 0; m < kVpl; ++m) buf[m] = nxt[m];
    if (row + stride < rows) load(row + stride, nxt);
    const float rstd = rms_rstd(row_sumsq<kVpl>(buf), cols, ra.eps);
    rms_apply<kVpl>(buf, w4, lane, rstd, ymax);
  }
  wave_max_to(acc, bf16_pair_max(ymax), six_m);
}

// Narrow rows (cols <= 8192): every wave owns one LDS row buffer and
// streams its own rows with no workgroup barrier.  The next row's loads
// (kVpl 16-byte vectors per lane) are in flight while the wave quantizes the
// current one; lane l handles the row's blocks l, l + 64, ...  The workgroup
// shares the scale table, the channel order and (kRms) the weight vector.
// With kRms the staged row is normalized in LDS (RMSNorm above; its sum of
// squares comes from the row's registers), so the gathers, both stages and
// the residual see y.
template <uint32_t V, int kVpl, bool kRms>
__global__ __launch_bounds__(kRms ? rms_threads(kVpl) : 1024) void quantize_residual_wave_kernel(
    const uint16_t* __restrict__ in, int64_t rows, uint32_t cols, const int32_t* __restrict__ perm,
    uint32_t nres, const float* __restrict__ gscale, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales, RmsArgs ra, uint32_t dup) {
  constexpr bool k46 = (V & kVarFourOverSix) != 0;
  constexpr int kRule = !k46 ? kRuleMse
                        : (V & kVarMax) ? kRuleMax
                        : (V & kVarMae) ? kRuleMae
                                        : kRuleMse;
  // LDS: scale table (1 KiB), channel order (cols 16-bit byte offsets),
  // with kRms the zero-padded weight vector, one row per wave.
  extern __shared__ __align__(16) uint8_t lds[];
  float2* tab = reinterpret_cast<float2*>(lds);
  uint16_t* pm = reinterpret_cast<uint16_t*>(lds + 1024);
  u32x4* w4 = reinterpret_cast<u32x4*>(pm + cols);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t nwaves_g = blockDim.x >> 6;
  // cols * 2 bytes is a multiple of 32; the weight area is 64 * kVpl
  // 16-byte vectors.
  uint16_t* xr = pm + cols + (kRms ? 512u * kVpl : 0u) + cols * wave;
  u32x4* xr4 = reinterpret_cast<u32x4*>(xr);

  const TensorScales ts = tensor_scales(*gscale);
  build_scale_table(tab, ts);
  for (uint32_t c = threadIdx.x; c < cols; c += blockDim.x)
    pm[c] = (uint16_t)(2u * std::min((uint32_t)perm[c], cols - 1u));
  const uint32_t vrow = cols >> 3;
  if constexpr (kRms) stage_weight<kVpl>(w4, ra.weight, vrow);
  __syncthreads();

  const uint32_t nb = cols >> 4, nrb = nres >> 4, bout = nb + nrb;
  const int64_t first = (int64_t)blockIdx.x * nwaves_g + wave;
  const int64_t stride = (int64_t)gridDim.x * nwaves_g;
  uint32_t ymax = 0u;  // packed bf16 max |y| (kRms)

  auto load = [&](int64_t row, u32x4 (&buf)[kVpl]) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(in + row * cols, vrow * 16u);
#pragma unroll
    for (int m = 0; m < kVpl; ++m)
      buf[m] = __builtin_amdgcn_raw_buffer_load_b128(r, (lane + 64u * m) * 16u, 0, kStreamLoad);
  };

  u32x4 buf[kVpl];
  if (first < rows) load(first, buf);
  for (int64_t row = first; row < rows; row += stride) {
    float rstd = 0.0f;
    if constexpr (kRms) rstd = rms_rstd(row_sumsq<kVpl>(buf), cols, ra.eps);
    // LDS operations of one wave complete in order: the previous row's
    // gathers are done before these writes, and the writes before the
    // gathers below.
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int m = 0; m < kVpl; ++m) {
      const uint32_t v = lane + 64u * m;
      if (v < vrow) xr4[v] = buf[m];
    }
    __builtin_amdgcn_wave_barrier();
    if (row + stride < rows) {
      __builtin_amdgcn_s_setprio(3);
      load(row + stride, buf);
      __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (kRms) {
      // Normalize the staged row in place, each lane its own vectors, while
      // the next row's loads are in flight (its registers are taken).
#pragma unroll 1
      for (uint32_t v = lane; v < vrow; v += 64u) {
        const u32x4 x = xr4[v], w = w4[v];
        xr4[v] = u32x4{rms_pair(x.x, w.x, rstd, ymax), rms_pair(x.y, w.y, rstd, ymax),
                       rms_pair(x.z, w.z, rstd, ymax), rms_pair(x.w, w.w, rstd, ymax)};
      }
      __builtin_amdgcn_wave_barrier();
    }
    const __amdgpu_buffer_rsrc_t r_packed = make_rsrc(packed + row * bout * 8, bout * 8u);
    const __amdgpu_buffer_rsrc_t r_scales = make_rsrc(scales + row * bout, bout);
#pragma unroll 1
    for (uint32_t j = lane; j < nb; j += 64u)
      residual_block<k46, kRule>(xr, pm, j, j, nb, j < nrb, dup != 0u, r_packed, r_scales, ts,
                                 tab);
  }
  if (kRms && ra.amax_out) wave_max_to(ra.amax_out, bf16_pair_max(ymax), 0.0f);
}

// ------------------------------------------------------------- launchers --

// Raises a kernel's dynamic-LDS limit above 64 KiB once per size it needs
// (hipFuncSetAttribute), not on every launch.
template <auto Kernel>
static hipError_t allow_lds(size_t bytes) {
  static std::atomic<size_t> allowed{65536};
  size_t cur = allowed.load(std::memory_order_relaxed);
  if (bytes <= cur) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  while (cur < bytes && !allowed.compare_exchange_weak(cur, bytes, std::memory_order_relaxed)) {
  }
  return hipSuccess;
}

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
  const unsigned groups = (unsigned)((cols + 63) / 64);
  channel_rank_kernel<<<groups, kRankThreads, 0, s>>>(absmax_bits, (uint32_t)cols, perm);
  return hipGetLastError();
}

template <uint32_t V>
static hipError_t launch_residual_group(const uint16_t* in, int64_t rows, int64_t cols,
                                        const int32_t* perm, int64_t nres, const float* gscale,
                                        uint8_t* packed, uint8_t* scales, bool dup,
                                        hipStream_t s) {
  // Rows per step: at least kResItems output blocks per thread, within the
  // staging capacity of kResThreads * kResVec 16-byte vectors and the
  // compute unit's 160 KiB of LDS.
  const int64_t nb = cols / 16;
  int64_t R = ((int64_t)kResItems * kResThreads + nb - 1) / nb;
  R = std::min<int64_t>(R, (int64_t)kResThreads * kResVec * 8 / cols);
  R = std::min<int64_t>(R, (163840 - 1024 - cols * 2) / (cols * 2));
  if (R < 1) R = 1;
  const size_t lds = 1024 + (size_t)cols * 2 + (size_t)R * cols * 2;
  const hipError_t e = allow_lds<&quantize_residual_kernel<V>>(lds);
  if (e != hipSuccess) return e;
  // One workgroup per compute unit, persistent over steps.
  const int64_t niter = (rows + R - 1) / R;
  const int64_t groups = std::max<int64_t>(1, std::min<int64_t>(niter, device_cu_count()));
  quantize_residual_kernel<V><<<(unsigned)groups, kResThreads, lds, s>>>(
      in, rows, (uint32_t)cols, perm, (uint32_t)nres, gscale, packed, scales, (uint32_t)R,
      (uint32_t)dup);
  return hipGetLastError();
}

template <uint32_t V, int kVpl, bool kRms>
static hipError_t launch_residual_wave(const uint16_t* in, int64_t rows, int64_t cols,
                                       const int32_t* perm, int64_t nres, const float* gscale,
                                       uint8_t* packed, uint8_t* scales, const RmsArgs& ra,
                                       bool dup, hipStream_t s) {
  // As many waves per compute unit as their row buffers fit in LDS (at most
  // 16), one workgroup per compute unit.
  const int64_t row_bytes = cols * 2;
  const int64_t shared = 1024 + row_bytes + (kRms ? 1024 * kVpl : 0);
  int64_t waves = (163840 - shared) / row_bytes;
  const int64_t max_waves = (kRms ? rms_threads(kVpl) : 1024) / 64;
  if (waves > max_waves) waves = max_waves;
  if (waves < 1) waves = 1;
  int64_t groups = (rows + waves - 1) / waves;
  if (groups > device_cu_count()) groups = device_cu_count();
  const size_t lds = (size_t)shared + (size_t)row_bytes * waves;
  const hipError_t e = allow_lds<&quantize_residual_wave_kernel<V, kVpl, kRms>>(lds);
  if (e != hipSuccess) return e;
  quantize_residual_wave_kernel<V, kVpl, kRms>
      <<<(unsigned)groups, (unsigned)(waves * 64), lds, s>>>(
          in, rows, (uint32_t)cols, perm, (uint32_t)nres, gscale, packed, scales, ra,
          (uint32_t)dup);
  return hipGetLastError();
}

template <uint32_t V>
static hipError_t launch_residual_v(const uint16_t* in, int64_t rows, int64_t cols,
                                    const int32_t* perm, int64_t nres, const float* gscale,
                                    uint8_t* packed, uint8_t* scales, bool dup, hipStream_t s) {
  // Rows of up to 8192 channels: one row per wave (kVpl = cols / 512 vectors
  // per lane, rounded up to the next instantiated size); wider rows: rows
  // shared by a workgroup.
  if (cols <= 2048)
    return launch_residual_wave<V, 4, false>(in, rows, cols, perm, nres, gscale, packed, scales,
                                           RmsArgs{}, dup, s);
  if (cols <= 4096)
    return launch_residual_wave<V, 8, false>(in, rows, cols, perm, nres, gscale, packed, scales,
                                           RmsArgs{}, dup, s);
  if (cols <= 6144)
    return launch_residual_wave<V, 12, false>(in, rows, cols, perm, nres, gscale, packed, scales,
                                           RmsArgs{}, dup, s);
  if (cols <= 8192)
    return launch_residual_wave<V, 16, false>(in, rows, cols, perm, nres, gscale, packed, scales,
                                           RmsArgs{}, dup, s);
  return launch_residual_group<V>(in, rows, cols, perm, nres, gscale, packed, scales, dup, s);
}

template <uint32_t V>
static hipError_t launch_rms_residual_v(const uint16_t* in, int64_t rows, int64_t cols,
                                        const int32_t* perm, int64_t nres, const float* gscale,
                                        uint8_t* packed, uint8_t* scales, const RmsArgs& ra,
                                        hipStream_t s) {
  if (cols <= 2048)
    return launch_residual_wave<V, 4, true>(in, rows, cols, perm, nres, gscale, packed, scales,
                                            ra, false, s);
  if (cols <= 4096)
    return launch_residual_wave<V, 8, true>(in, rows, cols, perm, nres, gscale, packed, scales,
                                            ra, false, s);
  if (cols <= 6144)
    return launch_residual_wave<V, 12, true>(in, rows, cols, perm, nres, gscale, packed, scales,
                                             ra, false, s);
  return launch_residual_wave<V, 16, true>(in, rows, cols, perm, nres, gscale, packed, scales,
                                           ra, false, s);
}

hipError_t launch_rms_quantize_residual(const uint16_t* in, int64_t rows, int64_t cols,
                                        const int32_t* perm, int64_t nres, const float* gscale,
                                        uint32_t variant, uint8_t* packed, uint8_t* scales,
                                        const RmsArgs& ra, hipStream_t s) {
  switch (variant) {
    case 0: return launch_rms_residual_v<0>(in, rows, cols, perm, nres, gscale, packed, scales, ra, s);
    case 1: return launch_rms_residual_v<1>(in, rows, cols, perm, nres, gscale, packed, scales, ra, s);
    case 3: return launch_rms_residual_v<3>(in, rows, cols, perm, nres, gscale, packed, scales, ra, s);
    case 17: return launch_rms_residual_v<17>(in, rows, cols, perm, nres, gscale, packed, scales, ra, s);
    default: return hipErrorInvalidValue;
  }
}

template <int kVpl>
static hipError_t launch_rms_amax_v(const uint16_t* in, int64_t rows, int64_t cols,
                                    const RmsArgs& ra, float six_m, uint32_t* acc, hipStream_t s) {
  // One workgroup per compute unit; LDS holds the weight vector.
  const int64_t waves = rms_threads(kVpl) / 64;
  int64_t groups = (rows + waves - 1) / waves;
  if (groups > device_cu_count()) groups = device_cu_count();
  const size_t lds = (size_t)1024 * kVpl;
  rms_amax_kernel<kVpl><<<(unsigned)groups, (unsigned)(waves * 64), lds, s>>>(
      in, rows, (uint32_t)cols, ra, six_m, acc);
  return hipGetLastError();
}

hipError_t launch_rms_amax(const uint16_t* in, int64_t rows, int64_t cols, const RmsArgs& ra,
                           float six_m, uint32_t* acc, hipStream_t s) {
  if (cols <= 2048) return launch_rms_amax_v<4>(in, rows, cols, ra, six_m, acc, s);
  if (cols <= 4096) return launch_rms_amax_v<8>(in, rows, cols, ra, six_m, acc, s);
  if (cols <= 6144) return launch_rms_amax_v<12>(in, rows, cols, ra, six_m, acc, s);
  return launch_rms_amax_v<16>(in, rows, cols, ra, six_m, acc, s);
}

hipError_t launch_quantize_residual(const uint16_t* in, int64_t rows, int64_t cols,
                                    const int32_t* perm, int64_t nres, const float* gscale,
                                    uint32_t variant, uint8_t* packed, uint8_t* scales,
                                    bool dup, hipStream_t s) {
  switch (variant) {
    case 0: return launch_residual_v<0>(in, rows, cols, perm, nres, gscale, packed, scales, dup, s);
    case 1: return launch_residual_v<1>(in, rows, cols, perm, nres, gscale, packed, scales, dup, s);
    case 3: return launch_residual_v<3>(in, rows, cols, perm, nres, gscale, packed, scales, dup, s);
    case 17:
      return launch_residual_v<17>(in, rows, cols, perm, nres, gscale, packed, scales, dup, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nvfp4
