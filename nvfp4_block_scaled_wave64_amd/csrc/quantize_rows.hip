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
// step covers a chunk of 64 blocks = 1024 elements = 2 KiB of input, read as
// two fully coalesced 1 KiB loads in which lane l (l < 32) holds the first
// half of block l of that KiB and lane l + 32 its second half.  Four
// v_permlane32_swap moves (one per dword) then leave every lane with one
// whole block: lane l owns block l of the chunk.  Per-block work (max, the
// two E4M3 scales, the selection) is thus done once per 16 elements, the 64
// selection bits of a chunk are one wave ballot, and each lane stores its 16
// codes as one 8-byte write (512 contiguous bytes per wave) and its scale
// byte (64 contiguous bytes).  Both candidates are evaluated in registers
// with packed E2M1 conversions (encode and decode); decode / encode
// multipliers of all 128 scale bytes come from a per-workgroup LDS table.
//
// Memory: all global accesses are raw buffer operations with hardware range
// checks (loads past the end read 0, stores past the end are dropped), so the
// ragged last chunk needs no branches.  Loads and the code stores are
// non-temporal (nothing is re-read); the small scale and bitmap stores go
// through the L2 so that partial lines merge before they reach HBM.  Each wave keeps the loads of its next chunk in
// flight while it works on the current one.  One launch covers at most 2^30
// elements (buffer offsets are 32-bit); the host splits larger tensors at
// chunk boundaries.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

template <uint32_t V>
__global__ __launch_bounds__(kRowsThreads) void quantize_rows_kernel(
    const uint16_t* __restrict__ in, int64_t nblocks, const float* __restrict__ gscale,
    uint8_t* __restrict__ packed, uint8_t* __restrict__ scales, uint8_t* __restrict__ selmap,
    double* __restrict__ err_sum, uint32_t* __restrict__ amax_out) {
  constexpr bool k46 = (V & kVarFourOverSix) != 0;
  constexpr int kRule = !k46 ? kRuleMse
                        : (V & kVarMax) ? kRuleMax
                        : (V & kVarMae) ? kRuleMae
                                        : kRuleMse;
  constexpr bool kSel = (V & kVarSelmap) != 0;
  constexpr bool kErr = (V & kVarErr) != 0;
  constexpr bool kAmax = (V & kVarAmax) != 0;
  constexpr bool kNeedErr = k46 || kErr;

  __shared__ float2 tab[128];
  __shared__ double wsum[kRowsWaves];
  __shared__ uint32_t wmax[kRowsWaves];

  const TensorScales ts = tensor_scales(*gscale);
  build_scale_table(tab, ts);
  __syncthreads();

  const uint32_t nb = (uint32_t)nblocks;  // <= 2^26 per launch
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t off_in = (lane & 31u) * 32u + (lane >> 5) * 16u;  // within a 1 KiB half
  const uint32_t off_sel = lane < 8u ? lane : 0x80000000u;          // lanes 0-7 store
  const uint32_t nchunks = (nb + 63u) / 64u;
  const uint32_t nwaves = gridDim.x * kRowsWaves;
  // The chunk a wave works on is wave-uniform: it lives in scalar registers,
  // and so do the per-chunk buffer resources below (no per-lane address
  // arithmetic in the loop).
  const uint32_t first =
      blockIdx.x * kRowsWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  double acc = 0.0;
  float bmax = 0.0f;  // running block max for amax_out (blocks past the end are 0)

  // Resource over the bytes [off, total) of chunk ch's part of a stream p,
  // based at p + off; empty for a chunk past the end (the prefetch of a
  // wave's last step).  For a chunk that exists, off < total holds for every
  // stream (its first input byte, code byte, scale byte and bitmap byte all
  // lie inside the tensor's), so the count needs no clamp; selecting it on
  // ch < nchunks keeps it scalar arithmetic (the compiler turns a clamp on
  // off < total into a vector instruction, and the resource would then look
  // divergent).  Range-checked accesses past the end read 0 or are dropped,
  // so the ragged last chunk needs no branches either.
  auto part = [&](const void* p, uint32_t ch, uint32_t off, uint32_t total) {
    return make_rsrc(static_cast<const uint8_t*>(p) + off, ch < nchunks ? total - off : 0u);
  };
  struct Two {
    u32x4 a, b;
  };
  auto load = [&](uint32_t ch) -> Two {
    const __amdgpu_buffer_rsrc_t r = part(in, ch, ch * 2048u, nb * 32u);
    Two t;
    t.a = __builtin_amdgcn_raw_buffer_load_b128(r, off_in, 0, kStreamLoad);
    t.b = __builtin_amdgcn_raw_buffer_load_b128(r, off_in + 1024u, 0, kStreamLoad);
    return t;
  };
  // The next chunk's loads are issued at raised wave priority so that they
  // leave as soon as the wave is scheduled, ahead of other waves' arithmetic.
  auto prefetch = [&](uint32_t ch) -> Two {
    __builtin_amdgcn_s_setprio(3);
    const Two t = load(ch);
    __builtin_amdgcn_s_setprio(0);
    return t;
  };

  auto process = [&](uint32_t ch, const Two& w) {
    // Lane l < 32 keeps its half of block l and takes the other half from
    // lane l + 32; lane l >= 32 takes block l (second KiB) the same way.
    uint32_t wd[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto p = __builtin_amdgcn_permlane32_swap(w.a[j], w.b[j], false, false);
      wd[j] = p[0];
      wd[4 + j] = p[1];
    }
    const Block16 q = quantize_block16<k46, kRule, kNeedErr>(wd, ts.k6, ts.k4, tab);
    if (kAmax) bmax = __builtin_elementwise_maximum(bmax, q.b);
    u32x2 codes;
    codes.x = q.lo;
    codes.y = q.hi;
    __builtin_amdgcn_raw_buffer_store_b64(codes, part(packed, ch, ch * 512u, nb * 8u), lane * 8u, 0,
                                          kStreamStore);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)q.S, part(scales, ch, ch * 64u, nb), lane, 0,
                                         kMergedStore);
    if (kSel) {
      // Lane l decides block l: the ballot is the chunk's 64 selection bits;
      // lanes 0-7 store its 8 bytes.
      const uint64_t bits = __ballot(q.pick4);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(bits >> (8u * (lane & 7u))),
                                           part(selmap, ch, ch * 8u, (nb + 7u) / 8u), off_sel, 0,
                                           kMergedStore);
    }
    if (kErr) acc += (double)q.err;  // blocks past the end contribute 0
  };

  // Every wave runs the same number of steps (a chunk index past the end is
  // skipped, wave-uniformly), so the workgroup can meet at a barrier every
  // kRowsSyncEvery steps.  Measured on MI355X: without it the 16 waves of a
  // compute unit drift apart over the tensor and their loads spread over
  // more DRAM pages; with a barrier every 2 steps the kernel runs about 10%
  // faster, and with one every step (the default) another 3% (32768 x 5120,
  // 4/6 MSE with bitmap and error sum: 71.6 -> 69.2 us), while every 4 steps
  // is slower (74.6 us).
  // The loop is unrolled twice with two load buffers used in turn, so the
  // prefetched registers are never copied.
  auto after_step = [&](uint32_t k) {
    if constexpr (kRowsSyncEvery > 0) {
      if (k % kRowsSyncEvery == kRowsSyncEvery - 1) __syncthreads();
    }
  };
  const uint32_t steps = (nchunks + nwaves - 1) / nwaves;
  Two bufa = load(first);
  uint32_t k = 0;
  for (; k + 1 < steps; k += 2) {
    const uint32_t ch = first + k * nwaves;
    const Two bufb = prefetch(ch + nwaves);
    if (ch < nchunks) process(ch, bufa);
    after_step(k);
    bufa = prefetch(ch + 2u * nwaves);
    if (ch + nwaves < nchunks) process(ch + nwaves, bufb);
    after_step(k + 1);
  }
  if (k < steps) {
    const uint32_t ch = first + k * nwaves;
    if (ch < nchunks) process(ch, bufa);
    after_step(k);
  }

  if (kAmax) group_max_to<kRowsWaves>(amax_out, bmax, wmax);
  if (kErr) {
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) wsum[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = wsum[0];
      for (int k2 = 1; k2 < kRowsWaves; ++k2) t += wsum[k2];
      unsafeAtomicAdd(err_sum, t);
    }
  }
}

template <uint32_t V>
static hipError_t launch_rows_v(const uint16_t* in, int64_t nblocks, const float* gscale,
                                uint8_t* packed, uint8_t* scales, uint8_t* selmap,
                                double* err_sum, uint32_t* amax_out, hipStream_t s,
                                Events ev) {
  // Segments of at most 2^26 blocks (2^30 elements, 2 GiB of input) keep
  // every buffer offset within 32 bits; a multiple of 64 blocks, so each
  // segment's bitmap starts on a byte boundary.
  constexpr int64_t kSeg = int64_t(1) << 26;
  const int64_t cap = (int64_t)device_cu_count() * (kGroupsPerCu > 0 ? kGroupsPerCu : 1);
  for (int64_t b0 = 0; b0 < nblocks; b0 += kSeg) {
    const int64_t nb = nblocks - b0 < kSeg ? nblocks - b0 : kSeg;
    const int64_t nchunks = (nb + 63) / 64;
    int64_t groups = (nchunks + kRowsWaves - 1) / kRowsWaves;
    if (groups > cap) groups = cap;
    if (groups < 1) groups = 1;
    Events seg;  // the first segment starts the bracket, the last one ends it
    if (b0 == 0) seg.start = ev.start;
    if (b0 + nb >= nblocks) seg.stop = ev.stop;
    const hipError_t e = launch_with_events(
        quantize_rows_kernel<V>, dim3((unsigned)groups), dim3(kRowsThreads), s, seg,
        in + b0 * 16, nb, gscale, packed + b0 * 8, scales + b0,
        selmap ? selmap + b0 / 8 : nullptr, err_sum, amax_out);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quantize_rows(const uint16_t* in, int64_t nblocks, const float* gscale,
                                uint32_t variant, uint8_t* packed, uint8_t* scales,
                                uint8_t* selmap, double* err_sum, uint32_t* amax_out,
                                hipStream_t s, Events ev) {
  if (amax_out) variant |= kVarAmax;
#define NVFP4_ROWS_CASE(v)                                                                       \
  case v:                                                                                        \
    return launch_rows_v<v>(in, nblocks, gscale, packed, scales, selmap, err_sum, amax_out, s,  \
                            ev);                                                                 \
  case v | kVarAmax:                                                                             \
    return launch_rows_v<v | kVarAmax>(in, nblocks, gscale, packed, scales, selmap, err_sum,     \
                                       amax_out, s, ev);
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
    NVFP4_ROWS_CASE(17)
    NVFP4_ROWS_CASE(21)
    NVFP4_ROWS_CASE(25)
    NVFP4_ROWS_CASE(29)
    default:
      return hipErrorInvalidValue;
  }
#undef NVFP4_ROWS_CASE
}

}  // namespace nvfp4
