// quantize_cols.hip -- NVFP4 / Four-Over-Six quantization with blocks of 16
// consecutive rows of one column (e.g. gradients quantized along the token
// axis; "Technical summary: Four Over Six (4/6)", "Key contributions",
// applies the method to activations, weights and gradients).  The outputs
// are laid out as the row-blocked outputs of the transposed tensor.
//
// A workgroup owns a strip of 64 columns and a range of rows, and walks it
// in tiles of 64 rows x 64 columns:
//   1. load: each row segment of the tile is 128 contiguous bytes; a thread
//      reads 16 bytes (8 columns of one row) per load;
//   2. transpose through LDS: the tile is stored column-major (tileT[col][row])
//      with a row pitch of 72 elements; the pad keeps the 16-byte reads of
//      step 3 aligned and spreads the columns of a wave over the banks;
//   3. compute: a lane pair (l, l + 32) takes one block (16 rows of one
//      column), each lane reading its 8 rows as one 16-byte LDS read, and runs
//      the same block math as the row-wise kernel;
//   4. store: the 4 blocks of a column in this tile are 32 contiguous bytes
//      of codes.  Since a workgroup walks down the rows of its strip,
//      successive tiles extend the same output rows and the partial lines
//      merge in that XCD's L2.
// When a selection bitmap is requested, the kernel marks the kept candidate
// in bit 7 of the scale byte (always 0 in a non-negative E4M3 scale) and a
// second pass turns those bits into the bitmap and clears them, which avoids
// sub-byte write races between workgroups.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

constexpr int kTileRows = 64;
constexpr int kTileCols = 64;
constexpr int kPitch = kTileRows + 8;  // bf16 elements per LDS column

template <uint32_t V>
__global__ __launch_bounds__(kThreads) void quantize_cols_kernel(
    const uint16_t* __restrict__ in, int64_t rows, int64_t cols, int64_t rows_per_group,
    const float* __restrict__ gscale, uint32_t* __restrict__ packed, uint8_t* __restrict__ scales,
    double* __restrict__ err_sum) {
  constexpr bool k46 = (V & kVarFourOverSix) != 0;
  constexpr bool kMae = k46 && (V & kVarMae) != 0;
  constexpr bool kSel = (V & kVarSelmap) != 0;
  constexpr bool kErr = (V & kVarErr) != 0;
  constexpr bool kNeedErr = k46 || kErr;

  __shared__ float2 tab[128];
  __shared__ __attribute__((aligned(16))) uint16_t tileT[kTileCols * kPitch];
  __shared__ double wsum[kWavesPerGroup];

  const TensorScales ts = tensor_scales(*gscale);
  build_scale_table(tab, ts);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int64_t c0 = (int64_t)blockIdx.x * kTileCols;
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_group;
  int64_t r_end = r_begin + rows_per_group;
  if (r_end > rows) r_end = rows;
  const bool vec_ok = (cols % 8) == 0;
  const int64_t rb16 = rows / 16;  // blocks per output row (per column of x)
  double acc = 0.0;

  for (int64_t r0 = r_begin; r0 < r_end; r0 += kTileRows) {
    __syncthreads();  // previous tile fully consumed (and the table built)
    // 1 + 2: load 64 x 64 and store transposed.  512 segments of 8 columns.
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int seg = t + k * kThreads;
      const int row = seg >> 3, cseg = (seg & 7) * 8;
      const int64_t gr = r0 + row, gc = c0 + cseg;
      uint32_t wd[4] = {0u, 0u, 0u, 0u};
      if (gr < r_end) {
        const uint16_t* src = in + gr * cols + gc;
        if (vec_ok) {
          if (gc < cols) {
            const uint4 w = load_stream16(src);
            wd[0] = w.x; wd[1] = w.y; wd[2] = w.z; wd[3] = w.w;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (gc + j < cols) wd[j >> 1] |= (uint32_t)src[j] << ((j & 1) * 16);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        tileT[(cseg + j) * kPitch + row] = (uint16_t)(wd[j >> 1] >> ((j & 1) * 16));
    }
    __syncthreads();

    // 3 + 4: 256 blocks (64 columns x 4 row blocks).  In pass p, wave w
    // takes blocks (4p + w) * 32 + (lane & 31); lane l < 32 holds rows 0-7 of
    // its block and lane l + 32 rows 8-15.
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int blk = (p * kWavesPerGroup + (t >> 6)) * 32 + (lane & 31);
      const int col = blk >> 2, rb = blk & 3, h = lane >> 5;
      const uint4 w = *reinterpret_cast<const uint4*>(&tileT[col * kPitch + rb * 16 + h * 8]);
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
      const HalfBlock hb = quantize_half_block<k46, kMae, kNeedErr>(wd, ts.k6, ts.k4, tab);
      const int64_t gc = c0 + col;
      const int64_t grb = r0 / 16 + rb;  // block index along the column
      const bool valid = gc < cols && r0 + rb * 16 < r_end;
      if (valid) {
        packed[(gc * rows / 2 + grb * 8 + h * 4) / 4] = hb.word;
        if (h == 0) {
          uint32_t sb = hb.S;
          if (kSel && hb.pick4) sb |= 0x80u;
          scales[gc * rb16 + grb] = (uint8_t)sb;
        }
        if (kErr && h == 0) acc += (double)hb.err;
      }
    }
  }

  if (kErr) {
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) wsum[t >> 6] = acc;
    __syncthreads();
    if (t == 0) {
      double s = wsum[0];
      for (int k = 1; k < kWavesPerGroup; ++k) s += wsum[k];
      unsafeAtomicAdd(err_sum, s);
    }
  }
}

// Bitmap pass: byte j of the bitmap collects bit 7 of scale bytes 8j..8j+7,
// which are then cleared.
__global__ __launch_bounds__(kThreads) void selmap_from_scales_kernel(uint8_t* __restrict__ scales,
                                                                     int64_t nblocks,
                                                                     uint8_t* __restrict__ selmap) {
  const int64_t nbytes = (nblocks + 7) / 8;
  for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < nbytes;
       j += (int64_t)gridDim.x * kThreads) {
    uint32_t bits = 0u;
    for (int k = 0; k < 8; ++k) {
      const int64_t b = j * 8 + k;
      if (b < nblocks) {
        const uint32_t s = scales[b];
        bits |= (s >> 7) << k;
        if (s & 0x80u) scales[b] = (uint8_t)(s & 0x7Fu);
      }
    }
    selmap[j] = (uint8_t)bits;
  }
}

template <uint32_t V>
static hipError_t launch_cols_v(const uint16_t* in, int64_t rows, int64_t cols,
                                const float* gscale, uint8_t* packed, uint8_t* scales,
                                uint8_t* selmap, double* err_sum, hipStream_t s) {
  const int64_t strips = (cols + kTileCols - 1) / kTileCols;
  const int64_t row_tiles = (rows + kTileRows - 1) / kTileRows;
  // Enough groups to fill the chip several times over; each walks a
  // contiguous run of row tiles of its strip.
  const int64_t target = (int64_t)device_cu_count() * 8;
  int64_t splits = (target + strips - 1) / strips;
  if (splits > row_tiles) splits = row_tiles;
  if (splits < 1) splits = 1;
  const int64_t tiles_per_group = (row_tiles + splits - 1) / splits;
  splits = (row_tiles + tiles_per_group - 1) / tiles_per_group;
  dim3 grid((unsigned)strips, (unsigned)splits);
  quantize_cols_kernel<V><<<grid, kThreads, 0, s>>>(in, rows, cols, tiles_per_group * kTileRows,
                                                   gscale, reinterpret_cast<uint32_t*>(packed),
                                                   scales, err_sum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !(V & kVarSelmap)) return e;
  const int64_t nblocks = rows / 16 * cols;
  int64_t groups = ((nblocks + 7) / 8 + kThreads - 1) / kThreads;
  if (groups > 4096) groups = 4096;
  if (groups < 1) groups = 1;
  selmap_from_scales_kernel<<<(unsigned)groups, kThreads, 0, s>>>(scales, nblocks, selmap);
  return hipGetLastError();
}

hipError_t launch_quantize_cols(const uint16_t* in, int64_t rows, int64_t cols,
                                const float* gscale, uint32_t variant, uint8_t* packed,
                                uint8_t* scales, uint8_t* selmap, double* err_sum, hipStream_t s) {
#define NVFP4_COLS_CASE(v) \
  case v:                  \
    return launch_cols_v<v>(in, rows, cols, gscale, packed, scales, selmap, err_sum, s);
  switch (variant) {
    NVFP4_COLS_CASE(0)
    NVFP4_COLS_CASE(1)
    NVFP4_COLS_CASE(3)
    NVFP4_COLS_CASE(4)
    NVFP4_COLS_CASE(5)
    NVFP4_COLS_CASE(7)
    NVFP4_COLS_CASE(8)
    NVFP4_COLS_CASE(9)
    NVFP4_COLS_CASE(11)
    NVFP4_COLS_CASE(12)
    NVFP4_COLS_CASE(13)
    NVFP4_COLS_CASE(15)
    default:
      return hipErrorInvalidValue;
  }
#undef NVFP4_COLS_CASE
}

}  // namespace nvfp4
