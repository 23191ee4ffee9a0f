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
// Blocks along the column (stored as the transpose): tiles of 64 columns x
// 256 rows are decoded into a row-major LDS tile and leave as 16-byte row
// segments (see dequantize_cols_kernel).
#include <type_traits>

#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

#ifndef NVFP4_DEQ_STORE_AUX
#define NVFP4_DEQ_STORE_AUX 16
#endif
// Cache policy of the output stores (each store instruction writes 1 KiB
// contiguously): sc1.
constexpr int kDeqStore = NVFP4_DEQ_STORE_AUX;

template <bool kBf16>
__global__ __launch_bounds__(kRowsThreads) void dequantize_rows_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ gscale, int64_t nblocks, void* __restrict__ out) {
  constexpr uint32_t kOutBlock = kBf16 ? 32u : 64u;  // output bytes per block
  constexpr uint32_t kStageBytes = 16u * 272u;        // fp32 staging per wave
  __shared__ __attribute__((aligned(16))) uint8_t stage[kBf16 ? 16u : kRowsWaves * kStageBytes];
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
  // Every wave runs the same number of steps (a chunk past the end is
  // skipped after the barrier), so the workgroup meets at a barrier every
  // step: its 16 waves then stream neighbouring chunks together.  Measured
  // on MI355X (32768 x 5120): bf16 output 77.3 -> 72.5 us, fp32 150 -> 131 us.
  In nxt = load(first);
  const uint32_t steps = (nchunks + nwaves - 1) / nwaves;
  for (uint32_t k = 0; k < steps; ++k) {
    const uint32_t ch = first + k * nwaves;
    const In cur = nxt;
    nxt = load(ch + nwaves);
    __syncthreads();
    if (ch >= nchunks) continue;
    const float d = block_decode_scale(cur.s & 0xFFu, g);
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
      // fp32: a block is 64 output bytes, so lane l's 4 quarters would land
      // 64 bytes apart.  The wave passes them through its own LDS region
      // (groups of 4 blocks padded to 272 bytes, so the 16 lanes of each
      // write pass hit distinct banks) and reads them back in output order:
      // store q then writes bytes 1024q .. 1024q + 1023 of the chunk.
      uint8_t* st = stage + (threadIdx.x >> 6) * kStageBytes;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 o = {__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                         __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])};
        *reinterpret_cast<u32x4*>(st + (lane >> 2) * 272u + (lane & 3u) * 64u + q * 16u) = o;
      }
      __builtin_amdgcn_wave_barrier();  // LDS operations of one wave complete in order
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t blk = 16u * q + (lane >> 2);  // block of output bytes 1024q + 16 lane
        const u32x4 o = *reinterpret_cast<const u32x4*>(st + (blk >> 2) * 272u + (blk & 3u) * 64u +
                                                        (lane & 3u) * 16u);
        __builtin_amdgcn_raw_buffer_store_b128(o, r_out, ch * 4096u + q * 1024u + lane * 16u, 0,
                                               kDeqStore);
      }
      __builtin_amdgcn_wave_barrier();  // the next step rewrites the region
    }
  }
}

// Blocks along the column: the stored codes are [n_rows = cols][rows/2]
// (the layout of the transpose).  A workgroup of 512 threads takes a tile of
// 64 stored rows (= columns of x) by 256 stored columns (= rows of x):
//   1. each lane loads 16 bytes of codes (two blocks) of one column; lanes
//      t < 64 load that tile column's 16 scale bytes into LDS;
//   2. each lane decodes a column pair's block (two columns, 16 rows) and
//      writes the 16 row pairs into a row-major LDS tile;
//   3. the tile leaves as 16-byte row segments (128 contiguous bytes per row
//      and tile for bf16, 256 for fp32).
constexpr int kDtCols = 64;    // columns of x per tile
constexpr int kDtRows = 256;   // rows of x per tile
constexpr int kDtThreads = 512;

template <bool kBf16>
__global__ __launch_bounds__(kDtThreads) void dequantize_cols_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ scales,
    const float* __restrict__ gscale, int64_t rows, int64_t cols, void* __restrict__ out) {
  constexpr int kEl = kBf16 ? 2 : 4;                 // output bytes per element
  constexpr int kPitch = kDtCols * kEl + 16;         // LDS bytes per tile row
  __shared__ __attribute__((aligned(16))) uint8_t tile[kDtRows * kPitch];
  __shared__ __attribute__((aligned(16))) uint32_t sc[kDtCols][4];  // 16 scale bytes per column
  __shared__ __attribute__((aligned(16))) uint32_t cw[kDtCols][33];  // 128 code bytes + pad

  const float g = *gscale;
  const int t = threadIdx.x;
  const int64_t nstrips = (cols + kDtCols - 1) / kDtCols;
  const int64_t nrt = (rows + kDtRows - 1) / kDtRows;
  const int64_t ntiles = nstrips * nrt;
  const int64_t rb_col = rows / 16;
  const bool scales16 = (reinterpret_cast<uintptr_t>(scales) % 16 == 0) && (rb_col % 16 == 0);

  // Waves split by role: the first half loads the next tile's codes and
  // scale bytes, the second half stores the output rows, and all decode.  A
  // wave's memory counter then covers only its own kind of access, so the
  // loading waves wait for their loads alone (issued a tile ahead) and never
  // for the previous tile's stores, which drain while the next tile is
  // staged and decoded.
  // Consecutive tiles on one XCD (workgroups are dispatched round-robin over
  // the 8 XCDs): the 8 row tiles of a strip share each 128-byte line of a
  // column's scale bytes, which one L2 then fetches once.
  const uint32_t nwg = gridDim.x;
  const uint32_t wg =
      (nwg % 8u == 0u) ? (blockIdx.x % 8u) * (nwg / 8u) + blockIdx.x / 8u : blockIdx.x;
  constexpr int kHalf = kDtThreads / 2;
  const bool loader_wave = __builtin_amdgcn_readfirstlane(t) < kHalf;  // wave-uniform

  // A tile's inputs in registers of the loading waves: lane u holds blocks
  // u + 256 h (h = 0..3) of the 64 x 16 (column, block) grid (8 code bytes
  // each); lanes u < 64 also hold column u's 16 scale bytes.  Loaded one tile
  // ahead.
  constexpr int kLoadH = kDtCols * 16 / kHalf;
  struct In {
    uint32_t c[2 * kLoadH];
    uint32_t s[4];
  };
  // Each role runs its own copy of the tile loop (the same barriers in the
  // same order), so that neither copy holds the other's memory operations.
  auto run = [&](auto role) {
    constexpr bool loader = decltype(role)::value;
    const int u = loader ? t : t - kHalf;  // index within the role
    auto load = [&](int64_t tt) -> In {
      In in;
#pragma unroll
      for (int i = 0; i < 2 * kLoadH; ++i) in.c[i] = 0u;
      in.s[0] = in.s[1] = in.s[2] = in.s[3] = 0u;
      if (tt >= ntiles || !loader) return in;  // the storing waves load nothing
      const int64_t strip = tt / nrt, rt = tt % nrt;
      const int64_t c0 = strip * kDtCols, r0 = rt * kDtRows;
      const int nrb = (int)((rows - r0) / 16 < 16 ? (rows - r0) / 16 : 16);
      const int ncol = (int)(cols - c0 < kDtCols ? cols - c0 : kDtCols);
#pragma unroll
      for (int h = 0; h < kLoadH; ++h) {
        const int k = u + h * kHalf, c = k >> 4, b = k & 15;
        if (c < ncol && b < nrb) {
          const uint32_t* src = reinterpret_cast<const uint32_t*>(
              packed + (c0 + c) * (rows / 2) + (r0 / 16 + b) * 8);
          // Default cache policy: the two halves of a block share a line,
          // which non-temporal loads fetched twice (1.78x the code bytes).
          in.c[2 * h] = src[0];
          in.c[2 * h + 1] = src[1];
        }
      }
      if (u < ncol) {
        const uint8_t* src = scales + (c0 + u) * rb_col + r0 / 16;
        if (scales16 && nrb == 16) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(src);
          in.s[0] = w.x; in.s[1] = w.y; in.s[2] = w.z; in.s[3] = w.w;
        } else {
          // Unrolled with constant word indices, so that in.s stays in registers.
#pragma unroll
          for (int b = 0; b < 16; ++b)
            if (b < nrb) in.s[b >> 2] |= (uint32_t)src[b] << (8 * (b & 3));
        }
      }
      return in;
    };

    In nxt = load(wg);
    for (int64_t tt = wg; tt < ntiles; tt += gridDim.x) {
      const int64_t strip = tt / nrt, rt = tt % nrt;
      const int64_t c0 = strip * kDtCols, r0 = rt * kDtRows;
      const int nrb = (int)((rows - r0) / 16 < 16 ? (rows - r0) / 16 : 16);
      __syncthreads();  // the previous tile's LDS contents have been read
      // 1. stage the codes and scale bytes in LDS (loading waves).
      if (loader) {
        const In cur = nxt;
#pragma unroll
        for (int h = 0; h < kLoadH; ++h) {
          const int k = u + h * kHalf, c = k >> 4, b = k & 15;
          cw[c][2 * b] = cur.c[2 * h];
          cw[c][2 * b + 1] = cur.c[2 * h + 1];
        }
        if (u < kDtCols) {
          sc[u][0] = cur.s[0];
          sc[u][1] = cur.s[1];
          sc[u][2] = cur.s[2];
          sc[u][3] = cur.s[3];
        }
      }
      __syncthreads();
      nxt = load(tt + gridDim.x);  // in flight during the decode and the stores
      // 2. lane t decodes block b = t / 32 of the column pair cp = t % 32.
      {
        const int cp = t & 31, b = t >> 5;
        float v0[16], v1[16];
        const int ca = 2 * cp, cb = 2 * cp + 1;
        const float da = block_decode_scale((sc[ca][b >> 2] >> (8 * (b & 3))) & 0xFFu, g);
        const float db = block_decode_scale((sc[cb][b >> 2] >> (8 * (b & 3))) & 0xFFu, g);
        e2m1_decode8(cw[ca][2 * b], v0);
        e2m1_decode8(cw[ca][2 * b + 1], v0 + 8);
        e2m1_decode8(cw[cb][2 * b], v1);
        e2m1_decode8(cw[cb][2 * b + 1], v1 + 8);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float xa = v0[i] * da, xb = v1[i] * db;
          uint8_t* dst = &tile[(b * 16 + i) * kPitch + ca * kEl];
          if (kBf16) {
            const f32x2 p = {xa, xb};
            *reinterpret_cast<uint32_t*>(dst) =
                __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
          } else {
            *reinterpret_cast<u32x2*>(dst) = u32x2{__float_as_uint(xa), __float_as_uint(xb)};
          }
        }
      }
      __syncthreads();
      // 3. rows of x (storing waves): 256 rows x (64 * kEl) bytes, 16 bytes per
      // lane and step.
      constexpr int kSegs = kDtCols * kEl / 16;  // 8 (bf16) or 16 (fp32) per row
      if (!loader) {
        for (int k = u; k < kDtRows * kSegs; k += kHalf) {
          const int r = k / kSegs, sg = k % kSegs;
          const int64_t gr = r0 + r;
          const int64_t gc = c0 + sg * (16 / kEl);
          if (gr < r0 + nrb * 16 && gc < cols) {
            const uint8_t* src = &tile[r * kPitch + sg * 16];
            const u32x2 a = *reinterpret_cast<const u32x2*>(src);
            const u32x2 b = *reinterpret_cast<const u32x2*>(src + 8);
            uint8_t* dst = static_cast<uint8_t*>(out) + (gr * cols + gc) * kEl;
            if (gc + 16 / kEl <= cols && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
              // Measured: non-temporal stores are faster for the bf16 rows
              // (128 bytes per row and tile), the default policy for fp32 (256).
              if (kBf16)
                __builtin_nontemporal_store(u32x4{a.x, a.y, b.x, b.y},
                                            reinterpret_cast<u32x4*>(dst));
              else
                *reinterpret_cast<u32x4*>(dst) = u32x4{a.x, a.y, b.x, b.y};
            } else {
              const uint32_t w[4] = {a.x, a.y, b.x, b.y};
              const int n = (int)((cols - gc) < 16 / kEl ? (cols - gc) : 16 / kEl);
#pragma unroll
              for (int e = 0; e < 16 / kEl; ++e) {
                if (e >= n) break;
                if (kBf16)
                  reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                else
                  reinterpret_cast<uint32_t*>(dst)[e] = w[e];
              }
            }
          }
        }
      }
    }
  };
  if (loader_wave)
    run(std::true_type{});
  else
    run(std::false_type{});
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
  const int64_t ntiles = ((cols + kDtCols - 1) / kDtCols) * ((rows + kDtRows - 1) / kDtRows);
  int64_t groups = (int64_t)device_cu_count() * 2;
  if (groups > ntiles) groups = ntiles;
  if (groups < 1) groups = 1;
  if (out_bf16)
    dequantize_cols_kernel<true><<<(unsigned)groups, kDtThreads, 0, s>>>(packed, scales, gscale,
                                                                         rows, cols, out);
  else
    dequantize_cols_kernel<false><<<(unsigned)groups, kDtThreads, 0, s>>>(packed, scales, gscale,
                                                                          rows, cols, out);
  return hipGetLastError();
}

}  // namespace nvfp4
