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

// Cache policy of the code stores (8 bytes per block, scattered over the
// rows of a batch): non-temporal.  Measured on 32768 x 5120, nres 256: 1.6 us
// of 93 faster than sc1 (the row-wise quantizer's choice), 3 us faster than
// the default policy.
constexpr int kResCodeStore = 2;

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

// ----------------------------------------------------------- check order --

// *bad = cols - (number of distinct values of perm inside [0, cols)): 0
// exactly when perm is a permutation of the channels.  One workgroup; an LDS
// bitmap marks the values seen.
constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_order_kernel(
    const int32_t* __restrict__ perm, uint32_t cols, uint32_t* __restrict__ bad) {
  __shared__ uint32_t seen[32768 / 32];
  __shared__ uint32_t part[kCheckThreads / 64];
  const uint32_t words = (cols + 31u) / 32u;
  for (uint32_t w = threadIdx.x; w < words; w += kCheckThreads) seen[w] = 0u;
  __syncthreads();
  for (uint32_t c = threadIdx.x; c < cols; c += kCheckThreads) {
    const uint32_t v = (uint32_t)perm[c];
    if (v < cols) atomicOr(&seen[v >> 5], 1u << (v & 31u));
  }
  __syncthreads();
  uint32_t n = 0u;
  for (uint32_t w = threadIdx.x; w < words; w += kCheckThreads) n += __popc(seen[w]);
  for (int off = 32; off > 0; off >>= 1) n += (uint32_t)__shfl_xor((int)n, off);
  if ((threadIdx.x & 63u) == 0u) part[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0u;
    for (int k = 0; k < kCheckThreads / 64; ++k) t += part[k];
    *bad = cols - t;
  }
}

// Output rows of a call whose order has an entry outside [0, cols): every
// scale byte is 0x7F (the E4M3 NaN code) and every code 0, so that
// dequantizing the result, or a product over it, gives NaN instead of
// plausible numbers.  Rows row0, row0 + stride, ... of bout blocks; the
// threads of `team` (tid = 0 .. team - 1) share each row.
__device__ void poison_rows(int64_t row0, int64_t stride, int64_t rows, uint32_t bout,
                            uint32_t tid, uint32_t team, uint8_t* packed, uint8_t* scales) {
  for (int64_t r = row0; r < rows; r += stride) {
    for (uint32_t b = tid; b < bout; b += team) {
      scales[r * bout + b] = 0x7Fu;
      *reinterpret_cast<u32x2*>(packed + (r * bout + b) * 8) = u32x2{0u, 0u};
    }
  }
}

// -------------------------------------------------------------- quantize --

// Channel offsets of output block j: pm[16j .. 16j+15], byte offsets into
// a staged row, two per dword.
struct BlockIdx {
  u32x4 a, b;
};
__device__ __forceinline__ BlockIdx read_block_idx(const uint16_t* pm, uint32_t j) {
  const u32x4* p4 = reinterpret_cast<const u32x4*>(pm + j * 16u);
  return BlockIdx{p4[0], p4[1]};
}

// Gathers the 16 channels of a block from the staged row xr (bf16 in LDS):
// w[k] = the bf16 pattern of element k in the low 16 bits.
__device__ __forceinline__ void gather_block(const uint16_t* xr, const BlockIdx& ix,
                                             uint32_t (&w)[16]) {
  const uint32_t o[8] = {ix.a.x, ix.a.y, ix.a.z, ix.a.w, ix.b.x, ix.b.y, ix.b.z, ix.b.w};
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(xr);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    w[2 * k] = *reinterpret_cast<const uint16_t*>(xb + (o[k] & 0xFFFFu));
    w[2 * k + 1] = *reinterpret_cast<const uint16_t*>(xb + (o[k] >> 16));
  }
}

// Output block ob from its gathered channels w (gather_block): quantizes
// them, stores codes and scale as block ob of the output, and with `res`
// also block ob + nb: the residual block, or with `dup` (the weight side of
// the augmented product) a copy of block ob.
//   stash (nullable): instead of quantizing the residual block here, store
//   its 16 values x - v*d to stash[q * plane] (q = 0..3, float4 each) for a
//   later pass that quantizes up to 64 of them at once (stash_quantize).
//   The stash is four planes of float4 (values 4q .. 4q+3 of every block in
//   plane q), so that consecutive lanes access consecutive 16-byte slots.
//   mid: run inside the block quantizer once its scale-table reads are
//   issued (quantize_block16_with).
// Returns the primary block (codes and scale of block ob).
template <bool k46, int kRule, typename Mid = NoMid>
__device__ __forceinline__ Block16 residual_tail(const uint32_t (&w)[16], uint32_t ob,
                                                 uint32_t nb, bool res, bool dup,
                                                 __amdgpu_buffer_rsrc_t r_packed,
                                                 __amdgpu_buffer_rsrc_t r_scales,
                                                 const TensorScales& ts, const float2* tab,
                                                 float4* stash = nullptr, uint32_t plane = 0,
                                                 const Mid& mid = Mid{}) {
  constexpr bool kNeedErr = k46;
  float x[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = bf16_lo(w[k]);
  const Block16 q = quantize_block16f<k46, kRule, kNeedErr>(x, ts.k6, ts.k4, tab, mid);
  u32x2 codes;
  codes.x = q.lo;
  codes.y = q.hi;
  __builtin_amdgcn_raw_buffer_store_b64(codes, r_packed, ob * 8u, 0, kResCodeStore);
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)q.S, r_scales, ob, 0, kMergedStore);
  if (res && dup) {
    __builtin_amdgcn_raw_buffer_store_b64(codes, r_packed, (ob + nb) * 8u, 0, kResCodeStore);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)q.S, r_scales, ob + nb, 0, kMergedStore);
  } else if (res) {
    // Residual of the kept candidate, x - v*d rounded once.
    float v[16], rx[16];
    e2m1_decode8(q.lo, v);
    e2m1_decode8(q.hi, v + 8);
    const float d = tab[q.S].x;
#pragma unroll
    for (int k = 0; k < 16; ++k) rx[k] = __builtin_fmaf(-v[k], d, x[k]);
    if (stash) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        stash[plane * k] = float4{rx[4 * k], rx[4 * k + 1], rx[4 * k + 2], rx[4 * k + 3]};
      return q;
    }
    const Block16 qr = quantize_block16f<k46, kRule, kNeedErr>(rx, ts.k6, ts.k4, tab);
    u32x2 rc;
    rc.x = qr.lo;
    rc.y = qr.hi;
    __builtin_amdgcn_raw_buffer_store_b64(rc, r_packed, (ob + nb) * 8u, 0, kResCodeStore);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)qr.S, r_scales, ob + nb, 0, kMergedStore);
  }
  return q;
}

// Output block j of one staged row xr: gather_block, then residual_tail.
template <bool k46, int kRule>
__device__ __forceinline__ void residual_block(const uint16_t* xr, const uint16_t* pm,
                                               uint32_t j, uint32_t ob, uint32_t nb, bool res,
                                               bool dup, __amdgpu_buffer_rsrc_t r_packed,
                                               __amdgpu_buffer_rsrc_t r_scales,
                                               const TensorScales& ts, const float2* tab) {
  uint32_t w[16];
  gather_block(xr, read_block_idx(pm, j), w);
  residual_tail<k46, kRule>(w, ob, nb, res, dup, r_packed, r_scales, ts, tab);
}

// Quantizes one stashed residual block (its 16 values at stash[q * plane],
// q = 0..3) and stores it as block ob of `packed` / `scales` (global
// pointers: the stashed blocks of one pass belong to several rows).
template <bool k46, int kRule>
__device__ __forceinline__ void stash_quantize(const float4* stash, uint32_t plane, int64_t ob,
                                               uint8_t* packed, uint8_t* scales,
                                               const TensorScales& ts, const float2* tab) {
  float rx[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 t = stash[plane * k];
    rx[4 * k] = t.x;
    rx[4 * k + 1] = t.y;
    rx[4 * k + 2] = t.z;
    rx[4 * k + 3] = t.w;
  }
  const Block16 qr = quantize_block16f<k46, kRule, k46>(rx, ts.k6, ts.k4, tab);
  *reinterpret_cast<u32x2*>(packed + ob * 8) = u32x2{qr.lo, qr.hi};
  scales[ob] = (uint8_t)qr.S;
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
  // row, so no entry can read outside it, and an order with an entry
  // outside [0, cols) poisons the whole output (poison_rows).
  int bad = 0;
  for (uint32_t c = threadIdx.x; c < cols; c += kResThreads) {
    const uint32_t v = (uint32_t)perm[c];
    bad |= v >= cols;
    pm[c] = (uint16_t)(2u * std::min(v, cols - 1u));
  }

  const uint32_t nb = cols >> 4, nrb = nres >> 4, bout = nb + nrb;
  const uint32_t vrow = cols >> 3;
  const int64_t niter = (rows + R - 1) / R;
  if (__syncthreads_or(bad)) {
    for (int64_t it = blockIdx.x; it < niter; it += gridDim.x)
      poison_rows(it * R, 1, std::min<int64_t>(rows, it * R + R), bout, threadIdx.x,
                  kResThreads, packed, scales);
    return;
  }

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
// bits: level k adds the values of lanes l and l ^ 2^k.  DPP moves within the
// VALU (no LDS round trips): quad permutations for partners l ^ 1 and l ^ 2,
// row shifts by 4 and 8 (lane l takes l - 4 or l - 8 in its row of 16), then
// the row broadcasts of lanes 15 and 31.  A shift reaches the partner only
// in lanes whose bit k is set, so only some lanes carry the tree's pairs;
// lane 63, whose bits are all set, does at every level (its partners 62, 61,
// 59, 55, 47 and 31 did too at the levels before), and every pair is added in
// some order of its two operands (the same value).  Returns lane 63's sum.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_tree_sum(float t) {
  t = t + dpp_f32<0xB1>(t);   // quad_perm [1,0,3,2]: lane l ^ 1
  t = t + dpp_f32<0x4E>(t);   // quad_perm [2,3,0,1]: lane l ^ 2
  t = t + dpp_f32<0x114>(t);  // row_shr:4
  t = t + dpp_f32<0x118>(t);  // row_shr:8
  t = t + dpp_f32<0x142>(t);  // row_bcast:15 (lane 15 of each row to the next row)
  t = t + dpp_f32<0x143>(t);  // row_bcast:31 (lane 31 to rows 2 and 3)
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 63));
}

// One block held by a lane pair: lane 2b + h holds elements 8h .. 8h+7 of
// block b.  The steps and roundings are those of quantize_block16_with: the
// block max is the larger of the two halves' maxima (a maximum in any order),
// each lane encodes its half under both candidates and sums its half's error
// sequentially, and the block error joins the two halves (a sum or a
// maximum: both commute, so the two lanes hold the same value and keep the
// same candidate).  Returns this lane's 32-bit code word (its 8 codes) and
// the kept scale byte.  Both lanes of every pair must be active.
struct Half8 {
  uint32_t w;
  uint32_t S;
};
template <bool k46, int kRule>
__device__ __forceinline__ Half8 quantize_half8(const float x[8], float k6, float k4,
                                                const float2* tab) {
  const float bh = __builtin_elementwise_maximum(
      absmax3(x[0], x[1], x[2]), absmax3(absmax3(x[3], x[4], x[5]), x[6], x[7]));
  const float b = __builtin_elementwise_maximum(bh, dpp_f32<0xB1>(bh));  // lane l ^ 1
  const uint32_t S2 = e4m3_encode2(b * k6, k46 ? b * k4 : 0.0f);
  const uint32_t S6 = S2 & 0xFFu, S4 = (S2 >> 8) & 0xFFu;
  const float2 t6 = tab[S6];
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[i] * t6.y;
  const uint32_t c6 = e2m1_encode8(y);
  if constexpr (!k46) return Half8{c6, S6};
  const float2 t4 = tab[S4];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[i] * t4.y;
  const uint32_t c4 = e2m1_encode8(y);
  const float h6 = half_error<kRule>(x, c6, t6.x);
  const float h4 = half_error<kRule>(x, c4, t4.x);
  const float e6 = block_error<kRule>(h6, dpp_f32<0xB1>(h6));
  const float e4 = block_error<kRule>(h4, dpp_f32<0xB1>(h4));
  const bool pick4 = e4 < e6;  // ties and NaN keep max->6
  return Half8{pick4 ? c4 : c6, pick4 ? S4 : S6};
}

// Sum of squares of the row a wave holds as kVpl 16-byte vectors per lane
// (vector v = lane + 64 m covers elements 8v .. 8v+7; vectors past the row
// were loaded as zeros).  The chunk sums of one vector index m go through
// the lane tree (the first six levels of the pairwise tree over v), the
// per-m sums through the rest.  Vector indices m with no vector of the row
// (64 m >= vrow) hold zeros only: their sums are exactly 0 and are not
// computed.
template <int kVpl>
__device__ __forceinline__ float row_sumsq(const u32x4 (&buf)[kVpl], uint32_t vrow) {
  constexpr int kM = pow2_at_least(kVpl);
  float a[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    a[m] = 0.0f;
    if (m < kVpl && 64u * m < vrow) {
      float t = 0.0f;
      t = __builtin_fmaf(bf16_lo(buf[m].x), bf16_lo(buf[m].x), t);
      t = __builtin_fmaf(bf16_hi(buf[m].x), bf16_hi(buf[m].x), t);
      t = __builtin_fmaf(bf16_lo(buf[m].y), bf16_lo(buf[m].y), t);
      t = __builtin_fmaf(bf16_hi(buf[m].y), bf16_hi(buf[m].y), t);
      t = __builtin_fmaf(bf16_lo(buf[m].z), bf16_lo(buf[m].z), t);
      t = __builtin_fmaf(bf16_hi(buf[m].z), bf16_hi(buf[m].z), t);
      t = __builtin_fmaf(bf16_lo(buf[m].w), bf16_lo(buf[m].w), t);
      t = __builtin_fmaf(bf16_hi(buf[m].w), bf16_hi(buf[m].w), t);
      a[m] = wave_tree_sum(t);
    }
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

// One bf16 pair of y: bf16(x * rstd), then bf16(w * y) with the weights
// (wl, wh) as fp32 values (1 without a weight vector, which leaves y
// unchanged: the product of two bf16 values is exact).  With kMax, ymax
// keeps the two halves' running max |y| as bf16 bit patterns (non-negative
// bf16 values order like their patterns).
template <bool kMax>
__device__ __forceinline__ uint32_t rms_pair(uint32_t x, float wl, float wh, float rstd,
                                             uint32_t& ymax) {
  // bf16(x * rstd) of each half straight as an fp32 value: converting the
  // pair (0, v) puts bf16(v) in the high half over a zero low half.
  const float yl = __uint_as_float(pack_bf16(0.0f, bf16_lo(x) * rstd));
  const float yh = __uint_as_float(pack_bf16(0.0f, bf16_hi(x) * rstd));
  const uint32_t y = pack_bf16(wl * yl, wh * yh);
  if (kMax) ymax = max_u16x2(ymax, y & 0x7FFF7FFFu);
  return y;
}

// fp32 value of the larger half of a packed bf16 maximum.
__device__ __forceinline__ float bf16_pair_max(uint32_t m) {
  return __uint_as_float(max(m & 0xFFFFu, m >> 16) << 16);
}

// Replaces the row held in buf (kVpl 16-byte vectors per lane, vector
// lane + 64 m) by y = RMSNorm(x), bf16 pairs.  wf: the weights in LDS as
// fp32 in two planes of vrow float4 (the first and the last four weights of
// every row vector), so that consecutive lanes read consecutive 16-byte
// slots.  Vectors past the row are loaded as zeros and are left unchanged
// (they are never stored); vector indices m past the row are skipped.
template <int kVpl, bool kMax>
__device__ __forceinline__ void rms_apply(u32x4 (&buf)[kVpl], const float* wf, uint32_t lane,
                                          uint32_t vrow, float rstd, uint32_t& ymax) {
#pragma unroll
  for (int m = 0; m < kVpl; ++m) {
    const uint32_t v = lane + 64u * m;
    if (64u * m < vrow && v < vrow) {
      const float4 w0 = reinterpret_cast<const float4*>(wf)[v];
      const float4 w1 = reinterpret_cast<const float4*>(wf)[vrow + v];
      buf[m].x = rms_pair<kMax>(buf[m].x, w0.x, w0.y, rstd, ymax);
      buf[m].y = rms_pair<kMax>(buf[m].y, w0.z, w0.w, rstd, ymax);
      buf[m].z = rms_pair<kMax>(buf[m].z, w1.x, w1.y, rstd, ymax);
      buf[m].w = rms_pair<kMax>(buf[m].w, w1.z, w1.w, rstd, ymax);
    }
  }
}

// Stages the weight vector in LDS as fp32 in the two planes rms_apply
// reads: weight c (row vector v = c / 8, place i = c % 8) at plane i / 4,
// slot v, element i % 4; the weights widened exactly, or ones without a
// weight vector.
__device__ __forceinline__ void stage_weight(float* wf, const uint16_t* weight, uint32_t cols) {
  const uint32_t vrow = cols >> 3;
  for (uint32_t c = threadIdx.x; c < cols; c += blockDim.x) {
    const uint32_t v = c >> 3, i = c & 7u;
    wf[((i >> 2) * vrow + v) * 4u + (i & 3u)] =
        weight ? __uint_as_float((uint32_t)weight[c] << 16) : 1.0f;
  }
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
// Workgroup size of the kernels that normalize rows of kVpl >= 10 vectors
// per lane: 12 waves, which leaves each wave room for its row (two, in the
// first pass), the normalization and (fused) the block quantizer in
// registers.
constexpr int rms_threads(int kVpl) { return kVpl >= 10 ? 768 : 1024; }

template <int kVpl>
__global__ __launch_bounds__(rms_threads(kVpl)) void rms_amax_kernel(const uint16_t* __restrict__ in,
                                                        int64_t rows, uint32_t cols,
                                                        RmsArgs ra, float six_m,
                                                        uint32_t* __restrict__ acc) {
  extern __shared__ __align__(16) uint8_t lds[];
  float* wf = reinterpret_cast<float*>(lds);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t vrow = cols >> 3;
  stage_weight(wf, ra.weight, cols);
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * (blockDim.x >> 6);
  uint32_t ymax = 0u;
  auto load = [&](int64_t row, u32x4 (&buf)[kVpl]) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(uniform_ptr(in + row * cols), vrow * 16u);
#pragma unroll
    for (int m = 0; m < kVpl; ++m)
      buf[m] = __builtin_amdgcn_raw_buffer_load_b128(r, (lane + 64u * m) * 16u, 0, kStreamLoad);
  };
  // The next row's loads are in flight while the current row is reduced,
  // where two rows fit in registers (up to 10 vectors per lane); wider rows
  // load one row at a time and rely on the other waves.
  const int64_t first = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  constexpr bool kAhead = kVpl <= 10;
  u32x4 nxt[kVpl];
  if constexpr (kAhead) {
    if (first < rows) load(first, nxt);
  }
  for (int64_t row = first; row < rows; row += stride) {
    u32x4 buf[kVpl];
    if constexpr (kAhead) {
#pragma unroll
      for (int m = 0; m < kVpl; ++m) buf[m] = nxt[m];
      if (row + stride < rows) load(row + stride, nxt);
    } else {
      load(row, buf);
    }
    const float rstd = rms_rstd(row_sumsq<kVpl>(buf, vrow), cols, ra.eps);
    rms_apply<kVpl, true>(buf, wf, lane, vrow, rstd, ymax);
  }
  wave_max_to(acc, bf16_pair_max(ymax), six_m);
}

// Wide rows with RMSNorm in front (kRmsMaxCols < cols <= kRmsWideMaxCols):
// a 1024-thread workgroup per compute unit stages R rows per step, as
// quantize_residual_kernel does, and normalizes them in LDS before the
// gathers.  The sum of squares keeps the order above: chunk v of a row (its
// elements 8v .. 8v+7, one 16-byte LDS read) is summed by lane v % 64 of a
// wave that holds the 64 chunks of an aligned group, wave_tree_sum adds them
// (the first six levels of the zero-padded pairwise tree), and one wave per
// row adds the group sums with the same tree, the groups past the row's
// padded length being zeros, which leave the pairwise sums unchanged.
//   kOnlyAmax: the first pass of the fused path: normalize, fold
//   RN(max |y| / six_m) into *acc, quantize nothing.
//   V & kVarAmax: also fold max |y| into ra.amax_out while quantizing.
// LDS: scale table (1 KiB), channel order (cols 16-bit byte offsets), the
// weights as bf16 (cols), 64 group sums and one rstd per staged row, then
// the R staged rows.
template <uint32_t V, bool kOnlyAmax>
__global__ __launch_bounds__(kResThreads) void rms_residual_wide_kernel(
    const uint16_t* __restrict__ in, int64_t rows, uint32_t cols, const int32_t* __restrict__ perm,
    uint32_t nres, const float* __restrict__ gscale, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales, RmsArgs ra, uint32_t R, float six_m, uint32_t* __restrict__ acc) {
  constexpr bool k46 = (V & kVarFourOverSix) != 0;
  constexpr int kRule = !k46 ? kRuleMse
                        : (V & kVarMax) ? kRuleMax
                        : (V & kVarMae) ? kRuleMae
                                        : kRuleMse;
  constexpr bool kTrack = kOnlyAmax || (V & kVarAmax) != 0;
  extern __shared__ __align__(16) uint8_t lds[];
  float2* tab = reinterpret_cast<float2*>(lds);
  uint16_t* pm = reinterpret_cast<uint16_t*>(lds + 1024);
  uint16_t* wb = pm + cols;                                   // weights, bf16
  float* gsum = reinterpret_cast<float*>(wb + cols);          // [R][64]
  float* rstd_s = gsum + 64u * R;                             // [R], padded to 16 bytes
  uint16_t* xs = reinterpret_cast<uint16_t*>(rstd_s + ((R + 3u) & ~3u));
  u32x4* xs4 = reinterpret_cast<u32x4*>(xs);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr uint32_t kWaves = kResThreads / 64;

  const TensorScales ts = tensor_scales(kOnlyAmax ? 1.0f : *gscale);
  if constexpr (!kOnlyAmax) build_scale_table(tab, ts);
  int bad = 0;
  for (uint32_t c = threadIdx.x; c < cols; c += kResThreads) {
    if constexpr (!kOnlyAmax) {
      const uint32_t v = (uint32_t)perm[c];
      bad |= v >= cols;
      pm[c] = (uint16_t)(2u * std::min(v, cols - 1u));
    }
    wb[c] = ra.weight ? ra.weight[c] : (uint16_t)0x3F80u;  // 1.0 without a weight vector
  }
  const uint32_t nb = cols >> 4, nrb = nres >> 4, bout = nb + nrb;
  const uint32_t vrow = cols >> 3;
  // Groups of 64 chunks per row in the zero-padded tree: its padded length
  // is a power of two of at least 64, and vrow > 1024 here.
  uint32_t ngroups = 1u;
  while (64u * ngroups < vrow) ngroups *= 2u;
  const int64_t niter = (rows + R - 1) / R;
  if (__syncthreads_or(bad)) {
    for (int64_t it = blockIdx.x; it < niter; it += gridDim.x)
      poison_rows(it * R, 1, std::min<int64_t>(rows, it * R + R), bout, threadIdx.x,
                  kResThreads, packed, scales);
    return;
  }

  auto rows_at = [&](int64_t it) -> uint32_t {
    return (uint32_t)std::min<int64_t>((int64_t)R, rows - it * R);
  };
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

  uint32_t ymax = 0u;  // packed bf16 max |y| (kTrack)
  u32x4 buf[kResVec];
  if ((int64_t)blockIdx.x < niter) load(blockIdx.x, buf);
  uint32_t rot = 0u;
  for (int64_t it = blockIdx.x; it < niter; it += gridDim.x) {
    const uint32_t nr = rows_at(it);
    __syncthreads();  // the previous rows are consumed (and pm, wb, tab written)
#pragma unroll
    for (int k = 0; k < kResVec; ++k) {
      const uint32_t v = threadIdx.x + k * kResThreads;
      if (v < nr * vrow) xs4[v] = buf[k];
    }
    __syncthreads();
    if (it + gridDim.x < niter) load(it + gridDim.x, buf);

    // Sum of squares: group sums (every lane of a wave takes part in the
    // tree; chunks past the row read as zeros).
    for (uint32_t g = wave; g < nr * ngroups; g += kWaves) {
      const uint32_t rr = g / ngroups, chunk = (g - rr * ngroups) * 64u + lane;
      float t = 0.0f;
      if (chunk < vrow) {
        const u32x4 q = xs4[rr * vrow + chunk];
        t = __builtin_fmaf(bf16_lo(q.x), bf16_lo(q.x), t);
        t = __builtin_fmaf(bf16_hi(q.x), bf16_hi(q.x), t);
        t = __builtin_fmaf(bf16_lo(q.y), bf16_lo(q.y), t);
        t = __builtin_fmaf(bf16_hi(q.y), bf16_hi(q.y), t);
        t = __builtin_fmaf(bf16_lo(q.z), bf16_lo(q.z), t);
        t = __builtin_fmaf(bf16_hi(q.z), bf16_hi(q.z), t);
        t = __builtin_fmaf(bf16_lo(q.w), bf16_lo(q.w), t);
        t = __builtin_fmaf(bf16_hi(q.w), bf16_hi(q.w), t);
      }
      const float gs = wave_tree_sum(t);
      if (lane == 0u) gsum[rr * 64u + (g - rr * ngroups)] = gs;
    }
    __syncthreads();
    if (wave < nr) {
      const float t = lane < ngroups ? gsum[wave * 64u + lane] : 0.0f;
      const float rstd = rms_rstd(wave_tree_sum(t), cols, ra.eps);
      if (lane == 0u) rstd_s[wave] = rstd;
    }
    __syncthreads();
    // Normalize the staged rows in place (8 elements per 16-byte slot).
    const u32x4* w4 = reinterpret_cast<const u32x4*>(wb);
    for (uint32_t v = threadIdx.x; v < nr * vrow; v += kResThreads) {
      const uint32_t rr = v / vrow, c8 = v - rr * vrow;
      const float rstd = rstd_s[rr];
      const u32x4 w = w4[c8];
      u32x4 q = xs4[v];
      q.x = rms_pair<kTrack>(q.x, bf16_lo(w.x), bf16_hi(w.x), rstd, ymax);
      q.y = rms_pair<kTrack>(q.y, bf16_lo(w.y), bf16_hi(w.y), rstd, ymax);
      q.z = rms_pair<kTrack>(q.z, bf16_lo(w.z), bf16_hi(w.z), rstd, ymax);
      q.w = rms_pair<kTrack>(q.w, bf16_lo(w.w), bf16_hi(w.w), rstd, ymax);
      if constexpr (!kOnlyAmax) xs4[v] = q;
    }
    if constexpr (!kOnlyAmax) {
      __syncthreads();
      const int64_t r0 = it * R;
      const __amdgpu_buffer_rsrc_t r_packed = make_rsrc(packed + r0 * bout * 8, nr * bout * 8u);
      const __amdgpu_buffer_rsrc_t r_scales = make_rsrc(scales + r0 * bout, nr * bout);
      const uint32_t nitems = nr * nb;
#pragma unroll 1
      for (uint32_t item = (threadIdx.x + rot) & (kResThreads - 1u); item < nitems;
           item += kResThreads) {
        const uint32_t rr = item / nb, j = item - rr * nb;
        residual_block<k46, kRule>(xs + rr * cols, pm, j, rr * bout + j, nb, j < nrb, false,
                                   r_packed, r_scales, ts, tab);
      }
      rot = (rot + 64u) & (kResThreads - 1u);
    }
  }
  if constexpr (kOnlyAmax)
    wave_max_to(acc, bf16_pair_max(ymax), six_m);
  else if constexpr (kTrack)
    wave_max_to(ra.amax_out, bf16_pair_max(ymax), 0.0f);
}

// Workgroup size bound of the narrow-row kernel: 12 waves where the row (in
// registers), the normalization and two blocks in flight need more than 128
// VGPRs.  Rows of 12 or more vectors per lane fit at most 12 waves per
// compute unit in LDS anyway.
constexpr int wave_threads(bool kRms, int kVpl) {
  return (kVpl >= 10 || (kRms && kVpl >= 8)) ? 768 : 1024;
}

// Instantiations that hold the two-lanes-per-block residual pass: the
// plain kernels of 8 and 16 vectors per lane are at their register limit
// already (the pass would spill there) and keep the stash.
constexpr bool pair_res_fits(bool kRms, int kVpl) { return kRms || (kVpl != 8 && kVpl != 16); }

// Narrow rows (cols <= 8192): every wave owns one LDS row buffer and
// streams its own rows with no workgroup barrier.  The next row's loads
// (kVpl 16-byte vectors per lane) are in flight while the wave quantizes the
// current one; lane l handles the row's blocks l, l + 64, ...  The workgroup
// shares the scale table, the channel order and (kRms) the weight vector.
// With kRms the row is normalized in its registers before it is staged
// (RMSNorm above), so the gathers, both stages and the residual see y; with
// kVarAmax in V the kernel also folds max |y| into ra.amax_out.
template <uint32_t V, int kVpl, bool kRms>
__global__ __launch_bounds__(wave_threads(kRms, kVpl)) void quantize_residual_wave_kernel(
    const uint16_t* __restrict__ in, int64_t rows, uint32_t cols, const int32_t* __restrict__ perm,
    uint32_t nres, const float* __restrict__ gscale, uint8_t* __restrict__ packed,
    uint8_t* __restrict__ scales, RmsArgs ra, uint32_t dup, uint32_t stash_items,
    uint32_t pair_res) {
  constexpr bool k46 = (V & kVarFourOverSix) != 0;
  constexpr int kRule = !k46 ? kRuleMse
                        : (V & kVarMax) ? kRuleMax
                        : (V & kVarMae) ? kRuleMae
                                        : kRuleMse;
  constexpr bool kMax = kRms && (V & kVarAmax) != 0;
  // LDS: scale table (1 KiB), channel order (cols 16-bit byte offsets),
  // with kRms the weights as fp32 (cols * 4 bytes), one row per wave.
  extern __shared__ __align__(16) uint8_t lds[];
  float2* tab = reinterpret_cast<float2*>(lds);
  uint16_t* pm = reinterpret_cast<uint16_t*>(lds + 1024);
  float* wf = reinterpret_cast<float*>(pm + cols);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t nwaves_g = blockDim.x >> 6;
  // cols * 2 bytes is a multiple of 32, so every row buffer is 16-byte
  // aligned.
  // Residual blocks (nres > 0, not dup): when the launch gives a stash of
  // stash_items (32 or 64) blocks per wave and a row has at most that many,
  // each row's are stashed (x - v*d, 64 bytes each) and quantized in passes
  // of batch = stash_items / nrb rows, so that the second stage runs on
  // (nearly) full waves instead of a few lanes per row.
  const uint32_t nrb_ = nres >> 4;
  const uint32_t batch = stash_items ? stash_items / nrb_ : 0u;
  const uint32_t stash_bytes = stash_items * 64u;
  uint8_t* wave_area = reinterpret_cast<uint8_t*>(pm + cols + (kRms ? 2u * cols : 0u)) +
                       (size_t)(cols * 2u + stash_bytes) * wave;
  uint16_t* xr = reinterpret_cast<uint16_t*>(wave_area);
  float4* stash = reinterpret_cast<float4*>(wave_area + cols * 2u);
  u32x4* xr4 = reinterpret_cast<u32x4*>(xr);

  const TensorScales ts = tensor_scales(*gscale);
  build_scale_table(tab, ts);
  // Clamped byte offsets; an entry outside [0, cols) poisons the output.
  int bad = 0;
  for (uint32_t c = threadIdx.x; c < cols; c += blockDim.x) {
    const uint32_t v = (uint32_t)perm[c];
    bad |= v >= cols;
    pm[c] = (uint16_t)(2u * std::min(v, cols - 1u));
  }
  const uint32_t vrow = cols >> 3;
  if constexpr (kRms) stage_weight(wf, ra.weight, cols);

  const uint32_t nb = cols >> 4, nrb = nres >> 4, bout = nb + nrb;
  const int64_t first = (int64_t)blockIdx.x * nwaves_g + wave;
  const int64_t stride = (int64_t)gridDim.x * nwaves_g;
  if (__syncthreads_or(bad)) {
    poison_rows(first, stride, rows, bout, lane, 64u, packed, scales);
    return;
  }
  uint32_t ymax = 0u;  // packed bf16 max |y| (kRms)

  auto load = [&](int64_t row, u32x4 (&buf)[kVpl]) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(in + row * cols, vrow * 16u);
#pragma unroll
    for (int m = 0; m < kVpl; ++m)
      buf[m] = __builtin_amdgcn_raw_buffer_load_b128(r, (lane + 64u * m) * 16u, 0, kStreamLoad);
  };

  // The staged row's blocks j = lane, lane + 64, ... < nb, two in flight:
  // the next block's channels are gathered (and the offsets of the one
  // after it read) while the current block is quantized, right behind its
  // scale-table reads, so that their LDS latency hides behind that work.
  // Indices past the row are clamped to its last block (gathered and never
  // used).
  auto each_block = [&](auto&& tail) {
    if (lane >= nb) return;
    if constexpr (kRms && kVpl >= 16) {
      // Rows of 16 vectors per lane with the normalization leave no
      // registers for a second block: one at a time.
#pragma unroll 1
      for (uint32_t j = lane; j < nb; j += 64u) {
        uint32_t w[16];
        gather_block(xr, read_block_idx(pm, j), w);
        tail(w, j, NoMid{});
      }
      return;
    }
    const uint32_t last = nb - 1u;
    uint32_t wa[16], wb[16];
    gather_block(xr, read_block_idx(pm, lane), wa);
    BlockIdx ib = read_block_idx(pm, std::min(lane + 64u, last));
    BlockIdx ia;
#pragma unroll 1
    for (uint32_t j = lane;; j += 128u) {
      tail(wa, j, [&] {
        gather_block(xr, ib, wb);
        ia = read_block_idx(pm, std::min(j + 128u, last));
      });
      if (j + 64u >= nb) break;
      tail(wb, j + 64u, [&] {
        gather_block(xr, ia, wa);
        ib = read_block_idx(pm, std::min(j + 192u, last));
      });
      if (j + 128u >= nb) break;
    }
  };

  // Stashed block i = slot * nrb + j (slot = the row's place in its batch)
  // is lane i's in the pass: its row and block are fixed per lane.
  const uint32_t my_slot = batch ? lane / nrb_ : 0u, my_j = batch ? lane % nrb_ : 0u;
  // pair_res (only where pair_res_fits): lane j < nrb keeps its primary
  // block's codes and scale byte for the residual pass (pair_res implies
  // nrb <= 32).
  uint32_t keep_lo = 0u, keep_hi = 0u, keep_s = 0u;
  u32x4 buf[kVpl];
  if (first < rows) load(first, buf);
  uint32_t slot = 0;
  int64_t batch_row0 = first;
  for (int64_t row = first; row < rows; row += stride) {
    if constexpr (kRms) {
      // Normalize the row in its registers (each lane its own vectors).
      const float rstd = rms_rstd(row_sumsq<kVpl>(buf, vrow), cols, ra.eps);
      rms_apply<kVpl, kMax>(buf, wf, lane, vrow, rstd, ymax);
    }
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
    const __amdgpu_buffer_rsrc_t r_packed = make_rsrc(packed + row * bout * 8, bout * 8u);
    const __amdgpu_buffer_rsrc_t r_scales = make_rsrc(scales + row * bout, bout);
    if (pair_res_fits(kRms, kVpl) && pair_res) {
      each_block([&](const uint32_t(&w)[16], uint32_t j, const auto& mid) {
        const Block16 q = residual_tail<k46, kRule>(w, j, nb, false, false, r_packed, r_scales,
                                                    ts, tab, nullptr, 0u, mid);
        if (j < nrb) {
          keep_lo = q.lo;
          keep_hi = q.hi;
          keep_s = q.S;
        }
      });
      // Residual blocks, two lanes each (quantize_half8): lane 2b + h
      // gathers elements 8h .. 8h+7 of block b again from the staged row,
      // takes block b's codes and scale byte from lane b, and quantizes
      // x - v*d (one fused multiply-add per element, as residual_tail).
      // The exchanges run with every lane active.
      const uint32_t src = lane >> 1;
      const uint32_t p_lo = (uint32_t)__shfl((int)keep_lo, (int)src);
      const uint32_t p_hi = (uint32_t)__shfl((int)keep_hi, (int)src);
      const uint32_t p_s = (uint32_t)__shfl((int)keep_s, (int)src);
      if (lane < 2u * nrb) {
        const uint32_t b = lane >> 1, h = lane & 1u;
        const u32x4 o = *reinterpret_cast<const u32x4*>(pm + 16u * b + 8u * h);
        const uint32_t oo[4] = {o.x, o.y, o.z, o.w};
        const uint8_t* xb = reinterpret_cast<const uint8_t*>(xr);
        float x[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[2 * k] = bf16_lo(*reinterpret_cast<const uint16_t*>(xb + (oo[k] & 0xFFFFu)));
          x[2 * k + 1] = bf16_lo(*reinterpret_cast<const uint16_t*>(xb + (oo[k] >> 16)));
        }
        float v[8], rx[8];
        e2m1_decode8(h ? p_hi : p_lo, v);
        const float d = tab[p_s].x;
#pragma unroll
        for (int k = 0; k < 8; ++k) rx[k] = __builtin_fmaf(-v[k], d, x[k]);
        const Half8 qr = quantize_half8<k46, kRule>(rx, ts.k6, ts.k4, tab);
        __builtin_amdgcn_raw_buffer_store_b32(qr.w, r_packed, (nb + b) * 8u + 4u * h, 0,
                                              kResCodeStore);
        if (h == 0u)
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)qr.S, r_scales, nb + b, 0, kMergedStore);
      }
    } else if (batch) {
      each_block([&](const uint32_t(&w)[16], uint32_t j, const auto& mid) {
        residual_tail<k46, kRule>(w, j, nb, j < nrb, false, r_packed, r_scales, ts, tab,
                                  stash + slot * nrb + j, stash_items, mid);
      });
      // A full batch, or the wave's last row: quantize the stashed blocks
      // (LDS operations of one wave complete in order).
      if (++slot == batch || row + stride >= rows) {
        __builtin_amdgcn_wave_barrier();
        if (lane < slot * nrb) {
          const int64_t r = batch_row0 + (int64_t)my_slot * stride;
          stash_quantize<k46, kRule>(stash + lane, stash_items, r * bout + nb + my_j, packed,
                                     scales, ts, tab);
        }
        __builtin_amdgcn_wave_barrier();
        slot = 0;
        batch_row0 = row + stride;
      }
    } else {
      each_block([&](const uint32_t(&w)[16], uint32_t j, const auto& mid) {
        residual_tail<k46, kRule>(w, j, nb, j < nrb, dup != 0u, r_packed, r_scales, ts, tab,
                                  nullptr, 0u, mid);
      });
    }
  }
  if (kMax) wave_max_to(ra.amax_out, bf16_pair_max(ymax), 0.0f);
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

hipError_t launch_check_order(const int32_t* perm, int64_t cols, uint32_t* bad, hipStream_t s) {
  check_order_kernel<<<1, kCheckThreads, 0, s>>>(perm, (uint32_t)cols, bad);
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
  // Stash capacity (blocks per wave; 0 = the residual blocks are quantized
  // where they are formed).  The stash shares LDS with the row buffers, and
  // these kernels slow down sharply below about 12 waves per compute unit
  // (measured on 32768 x 5120, nres = 256: the plain kernel 105 us without a
  // stash at 14 waves, 95 us with 32 blocks at 12 waves, 99 us with 64 at
  // 10; the fused RMSNorm kernel 130 us without at 12 waves, 148 and 161 us
  // with 32 and 64 at 10 and 9), so the smallest capacity that holds a
  // row's residual blocks is taken only if it leaves at least
  // min(12, the waves without a stash).
  const int64_t nrb = nres / 16;
  const int64_t fixed = 1024 + cols * 2 + (kRms ? cols * 4 : 0);
  const int64_t max_waves = wave_threads(kRms, kVpl) / 64;
  auto waves_with = [&](int64_t items) {
    return std::min<int64_t>(max_waves, (163840 - fixed) / (cols * 2 + items * 64));
  };
  // Rows of at most 32 residual blocks take the two-lanes-per-block
  // residual pass after each row (no stash) where the instantiation holds
  // it; otherwise the stash or, failing that, the in-place second stage.
  const bool pair_res = pair_res_fits(kRms, kVpl) && !dup && nrb > 0 && nrb <= 32;
  int64_t stash_items = 0;
  if (!dup && nrb > 0 && !pair_res) {
    const int64_t need = std::min<int64_t>(12, waves_with(0));
    for (int64_t cap : {32, 64})
      if (nrb <= cap && waves_with(cap) >= need) {
        stash_items = cap;
        break;
      }
  }
  // As many waves per compute unit as their row buffers (and stashes) fit
  // in LDS, at most max_waves; one workgroup per compute unit.
  const int64_t row_bytes = cols * 2 + stash_items * 64;
  const int64_t shared = fixed;
  int64_t waves = (163840 - shared) / row_bytes;
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
          (uint32_t)dup, (uint32_t)stash_items, (uint32_t)pair_res);
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
  if (cols <= 5120)
    return launch_residual_wave<V, 10, false>(in, rows, cols, perm, nres, gscale, packed, scales,
                                           RmsArgs{}, dup, s);
  if (cols <= 6144)
    return launch_residual_wave<V, 12, false>(in, rows, cols, perm, nres, gscale, packed, scales,
                                           RmsArgs{}, dup, s);
  if (cols <= 8192)
    return launch_residual_wave<V, 16, false>(in, rows, cols, perm, nres, gscale, packed, scales,
                                           RmsArgs{}, dup, s);
  return launch_residual_group<V>(in, rows, cols, perm, nres, gscale, packed, scales, dup, s);
}

template <uint32_t V, bool kOnlyAmax>
static hipError_t launch_rms_wide(const uint16_t* in, int64_t rows, int64_t cols,
                                  const int32_t* perm, int64_t nres, const float* gscale,
                                  uint8_t* packed, uint8_t* scales, const RmsArgs& ra,
                                  float six_m, uint32_t* acc, hipStream_t s) {
  // Rows per step: at least kResItems output blocks per thread, within the
  // staging capacity of kResThreads * kResVec 16-byte vectors and the
  // compute unit's 160 KiB of LDS (rms_residual_wide_kernel's layout).
  const int64_t nb = cols / 16;
  auto lds_for = [&](int64_t r) {
    return 1024 + 4 * cols + 256 * r + 4 * ((r + 3) & ~int64_t(3)) + 2 * cols * r;
  };
  int64_t R = ((int64_t)kResItems * kResThreads + nb - 1) / nb;
  R = std::min<int64_t>(R, (int64_t)kResThreads * kResVec * 8 / cols);
  while (R > 1 && lds_for(R) > 163840) --R;
  if (R < 1 || lds_for(R) > 163840) return hipErrorInvalidValue;
  const size_t lds = (size_t)lds_for(R);
  const hipError_t e = allow_lds<&rms_residual_wide_kernel<V, kOnlyAmax>>(lds);
  if (e != hipSuccess) return e;
  // One workgroup per compute unit, persistent over steps.
  const int64_t niter = (rows + R - 1) / R;
  const int64_t groups = std::max<int64_t>(1, std::min<int64_t>(niter, device_cu_count()));
  rms_residual_wide_kernel<V, kOnlyAmax><<<(unsigned)groups, kResThreads, lds, s>>>(
      in, rows, (uint32_t)cols, perm, (uint32_t)nres, gscale, packed, scales, ra, (uint32_t)R,
      six_m, acc);
  return hipGetLastError();
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
  if (cols <= 5120)
    return launch_residual_wave<V, 10, true>(in, rows, cols, perm, nres, gscale, packed, scales,
                                            ra, false, s);
  if (cols <= 6144)
    return launch_residual_wave<V, 12, true>(in, rows, cols, perm, nres, gscale, packed, scales,
                                             ra, false, s);
  if (cols <= kRmsMaxCols)
    return launch_residual_wave<V, 16, true>(in, rows, cols, perm, nres, gscale, packed, scales,
                                             ra, false, s);
  return launch_rms_wide<V, false>(in, rows, cols, perm, nres, gscale, packed, scales, ra, 0.0f,
                                   nullptr, s);
}

hipError_t launch_rms_quantize_residual(const uint16_t* in, int64_t rows, int64_t cols,
                                        const int32_t* perm, int64_t nres, const float* gscale,
                                        uint32_t variant, uint8_t* packed, uint8_t* scales,
                                        const RmsArgs& ra, hipStream_t s) {
  // max |y| is tracked only when asked for (kVarAmax).
  if (ra.amax_out) variant |= kVarAmax;
#define NVFP4_RMS_CASE(v) \
  case v:                 \
    return launch_rms_residual_v<v>(in, rows, cols, perm, nres, gscale, packed, scales, ra, s);
  switch (variant) {
    NVFP4_RMS_CASE(0)
    NVFP4_RMS_CASE(1)
    NVFP4_RMS_CASE(3)
    NVFP4_RMS_CASE(17)
    NVFP4_RMS_CASE(0 | kVarAmax)
    NVFP4_RMS_CASE(1 | kVarAmax)
    NVFP4_RMS_CASE(3 | kVarAmax)
    NVFP4_RMS_CASE(17 | kVarAmax)
    default: return hipErrorInvalidValue;
  }
#undef NVFP4_RMS_CASE
}

template <int kVpl>
static hipError_t launch_rms_amax_v(const uint16_t* in, int64_t rows, int64_t cols,
                                    const RmsArgs& ra, float six_m, uint32_t* acc, hipStream_t s) {
  // One workgroup per compute unit; LDS holds the weight vector.
  const int64_t waves = rms_threads(kVpl) / 64;
  int64_t groups = (rows + waves - 1) / waves;
  if (groups > device_cu_count()) groups = device_cu_count();
  const size_t lds = (size_t)cols * 4;
  rms_amax_kernel<kVpl><<<(unsigned)groups, (unsigned)(waves * 64), lds, s>>>(
      in, rows, (uint32_t)cols, ra, six_m, acc);
  return hipGetLastError();
}

hipError_t launch_rms_amax(const uint16_t* in, int64_t rows, int64_t cols, const RmsArgs& ra,
                           float six_m, uint32_t* acc, hipStream_t s) {
  if (cols <= 2048) return launch_rms_amax_v<4>(in, rows, cols, ra, six_m, acc, s);
  if (cols <= 4096) return launch_rms_amax_v<8>(in, rows, cols, ra, six_m, acc, s);
  if (cols <= 5120) return launch_rms_amax_v<10>(in, rows, cols, ra, six_m, acc, s);
  if (cols <= 6144) return launch_rms_amax_v<12>(in, rows, cols, ra, six_m, acc, s);
  if (cols <= kRmsMaxCols) return launch_rms_amax_v<16>(in, rows, cols, ra, six_m, acc, s);
  return launch_rms_wide<0u, true>(in, rows, cols, nullptr, 0, nullptr, nullptr, nullptr, ra,
                                   six_m, acc, s);
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
