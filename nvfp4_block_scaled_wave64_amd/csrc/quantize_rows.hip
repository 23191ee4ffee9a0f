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
// and the packed codes, scale bytes and bitmap follow the same order.  A wave
// step covers a chunk of 32 blocks = 512 elements = 1 KiB of input: lane l
// (l < 32) holds the first 8 elements of block l and lane l + 32 the last 8,
// so one 16-byte load per lane reads the whole KiB, and the 32 selection
// bits of the chunk are the low half of one wave ballot.  The two lanes of a
// block exchange their partial maximum and partial errors with one
// v_permlane32_swap each.  Each lane converts both candidate scales with one
// packed E4M3 conversion, reads their decode / encode multipliers from a
// per-workgroup LDS table of all 128 scale bytes, and evaluates both
// candidates on its 8 elements with packed E2M1 conversions (encode and
// decode), keeping every intermediate in registers.
//
// Memory: all global accesses are raw buffer operations with hardware range
// checks (loads past the end read 0, stores past the end are dropped), so the
// ragged last chunk needs no branches, and the per-lane offsets are fixed.
// Each wave keeps the loads of its next chunks in flight while it works on
// the current ones.  One launch covers at most 2^30 elements (buffer offsets
// are 32-bit); the host splits larger tensors at chunk boundaries.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

// Chunks in flight per wave: the next round's loads are issued before the
// current round is processed.
constexpr int kDepth = 2;

template <uint32_t V>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(
    const uint16_t* __restrict__ in, int64_t nblocks, const float* __restrict__ gscale,
    uint8_t* __restrict__ packed, uint8_t* __restrict__ scales, uint8_t* __restrict__ selmap,
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

  const uint32_t nb = (uint32_t)nblocks;  // <= 2^26 per launch
  const __amdgpu_buffer_rsrc_t r_in = make_rsrc(in, nb * 32u);
  const __amdgpu_buffer_rsrc_t r_packed = make_rsrc(packed, nb * 8u);
  const __amdgpu_buffer_rsrc_t r_scales = make_rsrc(scales, nb);
  const __amdgpu_buffer_rsrc_t r_sel = make_rsrc(selmap, (nb + 7u) / 8u);

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t blk_in_chunk = lane & 31u, half = lane >> 5;
  const uint32_t off_in = blk_in_chunk * 32u + half * 16u;    // bytes within a 1 KiB chunk
  const uint32_t off_packed = blk_in_chunk * 8u + half * 4u;  // within 256 B
  const uint32_t off_scale = half ? 0x80000000u : blk_in_chunk;  // upper lanes: out of range
  const uint32_t off_sel = lane < 4u ? lane : 0x80000000u;
  const uint32_t nchunks = (nb + 31u) / 32u;
  const uint32_t nwaves = gridDim.x * kWavesPerGroup;
  const uint32_t first = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  double acc = 0.0;

  // Chunks past the end read as zeros (range-checked buffer load); ch stays
  // below nchunks + kDepth * nwaves, so ch * 1024 cannot wrap.
  auto load = [&](uint32_t ch) -> u32x4 {
    return __builtin_amdgcn_raw_buffer_load_b128(r_in, ch * 1024u + off_in, 0, kStreamLoad);
  };

  u32x4 buf[kDepth];
#pragma unroll
  for (int k = 0; k < kDepth; ++k) buf[k] = load(first + k * nwaves);

  for (uint32_t base = first; base < nchunks; base += kDepth * nwaves) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const uint32_t ch = base + k * nwaves;
      const u32x4 w = buf[k];
      buf[k] = load(ch + kDepth * nwaves);
      if (ch >= nchunks) break;  // wave-uniform
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
      const HalfBlock hb = quantize_half_block<k46, kMae, kNeedErr>(wd, ts.k6, ts.k4, tab);
      __builtin_amdgcn_raw_buffer_store_b32(hb.word, r_packed, ch * 256u + off_packed, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)hb.S, r_scales, ch * 32u + off_scale, 0, 0);
      if (kSel) {
        // Lane l < 32 decides block l: the low half of the ballot is the
        // chunk's 32 selection bits; lanes 0-3 store its 4 bytes.
        const uint32_t bits = (uint32_t)__ballot(hb.pick4);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(bits >> (8u * (lane & 3u))), r_sel,
                                             ch * 4u + off_sel, 0, 0);
      }
      // Both lanes of a pair hold the block error (blocks past the end
      // contribute 0); the wave total is halved at the end.
      if (kErr) acc += (double)hb.err;
    }
  }

  if (kErr) {
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) wsum[threadIdx.x >> 6] = 0.5 * acc;
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
  // Segments of at most 2^26 blocks (2^30 elements, 2 GiB of input) keep
  // every buffer offset within 32 bits; a multiple of 32 blocks, so each
  // segment's bitmap starts on a byte (indeed a dword) boundary.
  constexpr int64_t kSeg = int64_t(1) << 26;
  const int64_t cap = (int64_t)device_cu_count() * 8;  // 8 groups (32 waves) per CU
  for (int64_t b0 = 0; b0 < nblocks; b0 += kSeg) {
    const int64_t nb = nblocks - b0 < kSeg ? nblocks - b0 : kSeg;
    const int64_t nchunks = (nb + 31) / 32;
    int64_t groups = (nchunks + kWavesPerGroup - 1) / kWavesPerGroup;
    if (groups > cap) groups = cap;
    quantize_rows_kernel<V><<<(unsigned)groups, kThreads, 0, s>>>(
        in + b0 * 16, nb, gscale, packed + b0 * 8, scales + b0,
        selmap ? selmap + b0 / 8 : nullptr, err_sum);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
