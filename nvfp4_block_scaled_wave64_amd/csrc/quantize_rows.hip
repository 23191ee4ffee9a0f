// quantize_rows.hip -- NVFP4 / Four-Over-Six quantization of blocks of 16
// contiguous bf16 elements (the block runs along the row).
//
// Method ("Technical summary: Four Over Six (4/6)", gist.science 2512.02010):
//   "Problem statement"       the standard scale maps each block max to 6;
//   "Core mechanism"          the alternative maps it to 4;
//   "Adaptive block scaling"  quantize both ways, measure each error against
//                             the original values, keep the lower one (MSE or
//                             MAE rule);
//   "Implementation details"  E4M3 block scales; all candidates and their
//                             errors stay in registers.
//
// Work layout (wave64).  The tensor is a flat sequence of 16-element blocks
// (the packed codes, the scale bytes and the bitmap are in the same order).
// One wave step covers a chunk of 32 blocks = 512 elements = 1 KiB of input:
// lane l loads the 16 bytes at offset 16*l, so a lane pair (2p, 2p+1) holds
// block p, the even lane the first 8 elements.  Loads are fully coalesced
// 1 KiB wave accesses; each lane stores its 8 codes as one dword (256 B per
// wave), even lanes store the block's scale byte, and the 32 selection bits
// of a chunk are one dword of the bitmap.
//
// Per block, the lane pair shares the work that is per block: each lane
// encodes one candidate's E4M3 scale (even lane max->6, odd lane max->4) and
// the pair swaps them with one DPP move; decode / encode multipliers of all
// 127 scale bytes sit in a per-workgroup LDS table built at start-up.  Each
// lane then evaluates both candidates on its 8 elements (scaled value, E2M1
// rounding, reconstruction, error) and the pair adds its two half-block
// errors with one more DPP move, so both lanes hold e_6 and e_4 and take the
// same decision.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

template <uint32_t V>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(
    const uint4* __restrict__ in, int64_t nblocks, const float* __restrict__ gscale,
    uint32_t* __restrict__ packed, uint8_t* __restrict__ scales, uint8_t* __restrict__ selmap,
    double* __restrict__ err_sum) {
  constexpr bool k46 = (V & kVarFourOverSix) != 0;
  constexpr bool kMae = k46 && (V & kVarMae) != 0;
  constexpr bool kSel = (V & kVarSelmap) != 0;
  constexpr bool kErr = (V & kVarErr) != 0;
  constexpr bool kNeedErr = k46 || kErr;

  __shared__ float2 tab[128];
  __shared__ double wsum[kWavesPerGroup];

  const TensorScales ts = tensor_scales(*gscale);
  build_scale_table(tab, ts);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const bool odd = (lane & 1) != 0;
  const float k_mine = (k46 && odd) ? ts.k4 : ts.k6;
  const int64_t nchunks = (nblocks + 31) / 32;
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerGroup;
  double acc = 0.0;

  for (int64_t ch = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6); ch < nchunks;
       ch += nwaves) {
    const int64_t blk = ch * 32 + (lane >> 1);
    const bool valid = blk < nblocks;
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (valid) w = load_stream16(&in[ch * 64 + lane]);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    const HalfBlock hb = quantize_half_block<k46, kMae, kNeedErr>(wd, odd, k_mine, tab);
    const bool pick4 = hb.pick4;
    if (valid) {
      packed[ch * 64 + lane] = hb.word;
      if (!odd) scales[blk] = (uint8_t)hb.S;
    }
    if (kSel) {
      // Both lanes of a pair vote the same bit; keep the even-lane bits.
      uint64_t x = __ballot(pick4) & 0x5555555555555555ull;
      x = (x | (x >> 1)) & 0x3333333333333333ull;
      x = (x | (x >> 2)) & 0x0F0F0F0F0F0F0F0Full;
      x = (x | (x >> 4)) & 0x00FF00FF00FF00FFull;
      x = (x | (x >> 8)) & 0x0000FFFF0000FFFFull;
      x = (x | (x >> 16)) & 0x00000000FFFFFFFFull;
      const int64_t nvalid = nblocks - ch * 32;
      if (nvalid >= 32) {
        if (lane == 0) reinterpret_cast<uint32_t*>(selmap)[ch] = (uint32_t)x;
      } else if (lane < (int)((nvalid + 7) / 8)) {
        selmap[ch * 4 + lane] = (uint8_t)(x >> (8 * lane));
      }
    }
    if (kErr && valid && !odd) acc += (double)hb.err;
  }

  if (kErr) {
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) wsum[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = wsum[0];
      for (int k = 1; k < kWavesPerGroup; ++k) t += wsum[k];
      unsafeAtomicAdd(err_sum, t);
    }
  }
}

template <uint32_t V>
static hipError_t launch_rows_v(const uint16_t* in, int64_t nblocks, const float* gscale,
                                uint8_t* packed, uint8_t* scales, uint8_t* selmap,
                                double* err_sum, hipStream_t s) {
  const int64_t nchunks = (nblocks + 31) / 32;
  int64_t groups = (nchunks + kWavesPerGroup - 1) / kWavesPerGroup;
  const int64_t cap = (int64_t)device_cu_count() * 8;  // 8 groups (32 waves) per CU
  if (groups > cap) groups = cap;
  quantize_rows_kernel<V><<<(unsigned)groups, kThreads, 0, s>>>(
      reinterpret_cast<const uint4*>(in), nblocks, gscale, reinterpret_cast<uint32_t*>(packed),
      scales, selmap, err_sum);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* in, int64_t nblocks, const float* gscale,
                                uint32_t variant, uint8_t* packed, uint8_t* scales,
                                uint8_t* selmap, double* err_sum, hipStream_t s) {
#define NVFP4_ROWS_CASE(v) \
  case v:                  \
    return launch_rows_v<v>(in, nblocks, gscale, packed, scales, selmap, err_sum, s);
  switch (variant) {
    NVFP4_ROWS_CASE(0)
    NVFP4_ROWS_CASE(1)
    NVFP4_ROWS_CASE(3)
    NVFP4_ROWS_CASE(4)
    NVFP4_ROWS_CASE(5)
    NVFP4_ROWS_CASE(7)
    NVFP4_ROWS_CASE(8)
    NVFP4_ROWS_CASE(9)
    NVFP4_ROWS_CASE(11)
    NVFP4_ROWS_CASE(12)
    NVFP4_ROWS_CASE(13)
    NVFP4_ROWS_CASE(15)
    default:
      return hipErrorInvalidValue;
  }
#undef NVFP4_ROWS_CASE
}

}  // namespace nvfp4
