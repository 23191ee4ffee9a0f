// quantize_cols.hip -- NVFP4 / Four-Over-Six quantization with blocks of 16
// consecutive rows of one column (e.g. gradients quantized along the token
// axis; "Technical summary: Four Over Six (4/6)", "Key contributions",
// applies the method to activations, weights and gradients).  The outputs
// are laid out as the row-blocked outputs of the transposed tensor: codes
// [cols][rows/2], scales [cols][rows/16], bitmap bit c*(rows/16) + rb.
//
// Tiles of 256 rows x 64 columns.  Per tile a workgroup of 8 waves
//   1. has the tile's 256 row segments of 128 contiguous bytes in the
//      registers of its four loading waves (8 x 16-byte loads per lane,
//      issued one tile ahead so they are in flight while the previous tile
//      is computed), which write them row-major into LDS (row pitch 136
//      bytes, see the pitches below);
//   2. lets every lane read a column pair over 16 rows (16 x 4-byte LDS
//      reads, consecutive banks across each half-wave), which are two whole
//      blocks; the lane repacks them and runs the same whole-block quantizer
//      as the row-wise kernel on each;
//   3. stages the codes (8 bytes per block), the scale bytes and the
//      selection flags per column in LDS, so that the four storing waves
//      send each column's 128 bytes of codes and 16 scale bytes out as
//      16-byte stores (whole 128-byte lines of codes per column and tile).
// The grid is persistent (a few workgroups per compute unit) and walks the
// tiles row-tile-major within each 64-column strip.  Workgroups are
// renumbered so that consecutive tiles run on one XCD: the 8 row tiles that
// share a 128-byte line of a column's scale bytes are then written through
// the same L2, which merges them.
//
// Dual emission (nvfp4_quantize_dual): the same tile also yields its 1024
// row-direction blocks, read from the LDS tile (32 contiguous bytes each),
// quantized by the same block quantizer and written in the row-blocked
// layout; such a call walks strips fastest instead.
#include <type_traits>

#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

#ifndef NVFP4_COLS_GROUPS_PER_CU
#define NVFP4_COLS_GROUPS_PER_CU 2
#endif
constexpr int kColsGroupsPerCu = NVFP4_COLS_GROUPS_PER_CU;
constexpr int kTileRows = 256;
constexpr int kTileCols = 64;
constexpr int kRowBlocks = kTileRows / 16;  // 16 row blocks per tile
// LDS pitches, chosen against bank conflicts (64 banks of 4 bytes):
//  - tile rows of 136 bytes (34 dwords): the two half-waves' column-pair
//    reads are 16 rows apart, 16 * 34 = 544 = 32 (mod 64) dwords, so they
//    fall in disjoint banks; rows are 8-byte aligned (two 8-byte writes);
//  - code columns of 132 bytes (33 dwords): the 32 columns 2cp written by a
//    half-wave start 66 cp = 2 cp (mod 64) dwords apart, all distinct;
//  - scale-byte columns of 20 bytes: 10 cp (mod 64) dwords, all distinct.
#ifndef NVFP4_COLS_IN_PITCH
#define NVFP4_COLS_IN_PITCH 136
#endif
#ifndef NVFP4_COLS_CODE_PITCH
#define NVFP4_COLS_CODE_PITCH 132
#endif
#ifndef NVFP4_COLS_S_PITCH
#define NVFP4_COLS_S_PITCH 20
#endif
constexpr int kInPitch = NVFP4_COLS_IN_PITCH;
constexpr int kCodePitch = NVFP4_COLS_CODE_PITCH;
constexpr int kSPitch = NVFP4_COLS_S_PITCH;
static_assert(kInPitch % 8 == 0 && kCodePitch % 4 == 0 && kSPitch % 4 == 0, "LDS alignment");
#ifndef NVFP4_COLS_THREADS
#define NVFP4_COLS_THREADS 512
#endif
constexpr int kColsThreads = NVFP4_COLS_THREADS;
constexpr int kColsWaves = kColsThreads / 64;
constexpr int kPasses = 512 / kColsThreads;        // column-pair tasks per lane
static_assert(kColsThreads == 256 || kColsThreads == 512, "tile mapping");


// kDual: also quantize the tile's row-direction blocks (16 contiguous
// elements of a row) into the row-blocked outputs packed_r / scales_r (scale
// bit 7 marks the kept max->4 candidate for the bitmap pass) and err_r.
// order: 0 walks row tiles fastest within a strip, 1 strips fastest.
template <uint32_t V, bool kDual>
__global__ __launch_bounds__(kColsThreads) void quantize_cols_kernel(
    const uint16_t* __restrict__ in, int64_t rows, int64_t cols, const float* __restrict__ gscale,
    uint8_t* __restrict__ packed, uint8_t* __restrict__ scales, uint8_t* __restrict__ selmap,
    double* __restrict__ err_sum, uint32_t* __restrict__ amax_out, uint8_t* __restrict__ packed_r,
    uint8_t* __restrict__ scales_r, double* __restrict__ err_r, int order) {
  constexpr bool k46 = (V & kVarFourOverSix) != 0;
  constexpr int kRule = !k46 ? kRuleMse
                        : (V & kVarMax) ? kRuleMax
                        : (V & kVarMae) ? kRuleMae
                                        : kRuleMse;
  constexpr bool kSel = (V & kVarSelmap) != 0;
  constexpr bool kErr = (V & kVarErr) != 0;
  constexpr bool kNeedErr = k46 || kErr;

  __shared__ float2 tab[128];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileRows * kInPitch];
  __shared__ __attribute__((aligned(16))) uint8_t codes[kTileCols * kCodePitch];
  __shared__ __attribute__((aligned(16))) uint8_t sbytes[kTileCols * kSPitch];
  __shared__ double wsum[kColsWaves];
  __shared__ double wsum_r[kColsWaves];
  __shared__ uint32_t wmax[kColsWaves];

  const TensorScales ts = tensor_scales(*gscale);
  build_scale_table(tab, ts);

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t nstrips = (cols + kTileCols - 1) / kTileCols;
  const int64_t nrt = (rows + kTileRows - 1) / kTileRows;
  const int64_t ntiles = nstrips * nrt;
  const int64_t rb_col = rows / 16;  // blocks per column = scale bytes per output row
  // Bitmap bytes are written directly when every column's bits start on a
  // byte boundary; otherwise bit 7 of the scale byte carries the flag to a
  // second pass.
  const bool sel_direct = (rb_col % 8) == 0;
  const bool vec_ok = (cols % 8) == 0;
  // 16-byte stores only where every column's run is 16-byte aligned; the
  // ABI guarantees 4-byte alignment of packed and none for scales.
  const bool codes16 = (reinterpret_cast<uintptr_t>(packed) % 16 == 0) && ((rows / 2) % 16 == 0);
  const bool scales16 = (reinterpret_cast<uintptr_t>(scales) % 16 == 0) && (rb_col % 16 == 0);

  // Consecutive logical ids on one XCD (workgroups are dispatched round-robin
  // over the 8 XCDs).
  const uint32_t nwg = gridDim.x;
  const uint32_t wg =
      (nwg % 8u == 0u) ? (blockIdx.x % 8u) * (nwg / 8u) + blockIdx.x / 8u : blockIdx.x;

  // Waves split by role (kSplit): the first half loads the tiles (one
  // tile ahead), the second half stores the codes, scale and bitmap bytes,
  // and all quantize.  A wave's memory counter then covers only its own
  // kind of access: the loading waves wait for their loads alone, never for
  // the previous tile's stores, which drain while the next tile is staged
  // and quantized.  The dual call (whose row-direction blocks are stored by
  // every lane) keeps one role.
  constexpr bool kSplit = !kDual;
  constexpr int kHalf = kColsThreads / 2;
  constexpr int kLoadLanes = kSplit ? kHalf : kColsThreads;
  constexpr int kLPL = kTileRows * kTileCols * 2 / (kLoadLanes * 16);  // loads per lane
  constexpr int kLR = kLoadLanes / 8;  // tile rows covered by one load
  const bool loader_wave = !kSplit || __builtin_amdgcn_readfirstlane(t) < kHalf;
  const int u = (kSplit && !loader_wave) ? t - kHalf : t;  // index within the role
  // Load k of a loading lane u covers tile row k * kLR + u/8, columns
  // (u%8)*8 .. +7.
  const int lrow = u >> 3, lseg = u & 7;
  auto tile_of = [&](int64_t tt, int64_t& strip, int64_t& rt) {
    if (order == 0) {
      strip = tt / nrt;
      rt = tt % nrt;
    } else {
      rt = tt / nstrips;
      strip = tt % nstrips;
    }
  };
  auto load_tile = [&](int64_t tt, u32x4* w) {
    int64_t strip, rt;
    tile_of(tt, strip, rt);
    const int64_t r0 = rt * kTileRows, c = strip * kTileCols + lseg * 8;
#pragma unroll
    for (int k = 0; k < kLPL; ++k) {
      const int64_t r = r0 + k * kLR + lrow;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (tt < ntiles && r < rows) {
        const uint16_t* src = in + r * cols + c;
        if (vec_ok) {
          if (c < cols) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c + j < cols) v[j >> 1] |= (uint32_t)src[j] << ((j & 1) * 16);
        }
      }
      w[k] = v;
    }
  };

  double acc = 0.0, acc_r = 0.0;
  float bmax = 0.0f;  // running block max for amax_out (padding blocks are 0)
  const bool codes_r16 =
      kDual && (reinterpret_cast<uintptr_t>(packed_r) % 16 == 0) && ((cols / 2) % 16 == 0);
  // Quantizes tile tt from the registers w, then refills w with tile
  // tt + nwg.  kLoad / kStore: this copy of the loop loads and stages the
  // tiles / stores the outputs (both without kSplit).
  auto process = [&](int64_t tt, u32x4* w, auto load_role) {
    constexpr bool kLoad = decltype(load_role)::value || !kSplit;
    constexpr bool kStore = !decltype(load_role)::value || !kSplit;
    int64_t strip, rt;
    tile_of(tt, strip, rt);
    const int64_t r0 = rt * kTileRows, c0 = strip * kTileCols;
    const int nrb = (int)((rows - r0) / 16 < kRowBlocks ? (rows - r0) / 16 : kRowBlocks);
    const int ncol = (int)(cols - c0 < kTileCols ? cols - c0 : kTileCols);

    __syncthreads();  // the previous tile's staging has been stored (and tab built)
    if constexpr (kLoad) {
#pragma unroll
      for (int k = 0; k < kLPL; ++k) {
        u32x2* dst = reinterpret_cast<u32x2*>(&tile[(k * kLR + lrow) * kInPitch + lseg * 16]);
        dst[0] = u32x2{w[k].x, w[k].y};
        dst[1] = u32x2{w[k].z, w[k].w};
      }
    }
    __syncthreads();
    if constexpr (kLoad) load_tile(tt + nwg, w);  // in flight during this tile's compute

    // 16 row blocks x 32 column pairs = 512 lane tasks, kPasses per lane:
    // in pass p, wave w takes row block (p * kColsWaves + w) * 2 + lane/32
    // and column pair lane%32.
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int rb = (p * kColsWaves + wave) * 2 + (lane >> 5);
      const int cp = lane & 31;
      uint32_t v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = *reinterpret_cast<const uint32_t*>(&tile[(rb * 16 + i) * kInPitch + cp * 4]);
      uint32_t wa[8], wb[8];  // columns 2cp and 2cp+1: rows 2j (low half), 2j+1
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        wa[j] = (v[2 * j] & 0xFFFFu) | (v[2 * j + 1] << 16);
        wb[j] = (v[2 * j] >> 16) | (v[2 * j + 1] & 0xFFFF0000u);
      }
      const Block16 qa = quantize_block16<k46, kRule, kNeedErr>(wa, ts.k6, ts.k4, tab);
      const Block16 qb = quantize_block16<k46, kRule, kNeedErr>(wb, ts.k6, ts.k4, tab);
      bmax = __builtin_elementwise_maximum(bmax, __builtin_elementwise_maximum(qa.b, qb.b));
      const int ca = 2 * cp, cb = 2 * cp + 1;
      u32x2 pa, pb;
      pa.x = qa.lo;
      pa.y = qa.hi;
      pb.x = qb.lo;
      pb.y = qb.hi;
      uint32_t* ka = reinterpret_cast<uint32_t*>(&codes[ca * kCodePitch + rb * 8]);
      uint32_t* kb = reinterpret_cast<uint32_t*>(&codes[cb * kCodePitch + rb * 8]);
      ka[0] = pa.x;
      ka[1] = pa.y;
      kb[0] = pb.x;
      kb[1] = pb.y;
      sbytes[ca * kSPitch + rb] = (uint8_t)(qa.S | (kSel && qa.pick4 ? 0x80u : 0u));
      sbytes[cb * kSPitch + rb] = (uint8_t)(qb.S | (kSel && qb.pick4 ? 0x80u : 0u));
      if (kErr && rb < nrb) {
        if (ca < ncol) acc += (double)qa.err;
        if (cb < ncol) acc += (double)qb.err;
      }
    }
    __syncthreads();

    // Codes: column c's nrb * 8 bytes go to packed[c][r0/2 ..]; each storing
    // lane stores 16-byte pieces (two row blocks each) of columns.
    constexpr int kStoreLanes = kSplit ? kHalf : kColsThreads;
    constexpr int kPieces = kTileCols * 8 / kStoreLanes;  // 16-byte pieces per lane
#pragma unroll
    for (int p = 0; p < (kStore ? kPieces : 0); ++p) {
      const int piece = p * kStoreLanes + u, c = piece >> 3, seg = piece & 7;
      if (c < ncol && 2 * seg < nrb) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(&codes[c * kCodePitch + seg * 16]);
        const u32x4 cw = {src[0], src[1], src[2], src[3]};
        uint8_t* dst = packed + (c0 + c) * (rows / 2) + r0 / 2 + seg * 16;
        const bool both = 2 * seg + 1 < nrb;
        if (codes16 && both) {
          __builtin_nontemporal_store(cw, reinterpret_cast<u32x4*>(dst));
        } else {
          uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);  // 4-byte aligned
          d32[0] = cw.x;
          d32[1] = cw.y;
          if (both) {
            d32[2] = cw.z;
            d32[3] = cw.w;
          }
        }
      }
    }
    // Scale bytes (and bitmap bytes): storing lane u < 64 handles column u.
    if (kStore && u < ncol) {
      const int t = u;  // the column
      const uint32_t* sw = reinterpret_cast<const uint32_t*>(&sbytes[t * kSPitch]);
      uint32_t s[4] = {sw[0], sw[1], sw[2], sw[3]};
      uint32_t bits = 0u;
      if (kSel && sel_direct) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // bit 7 of each byte -> bits 4k .. 4k+3 of the tile's 16 flags
          const uint32_t f = (s[k] >> 7) & 0x01010101u;
          bits |= ((f | (f >> 7) | (f >> 14) | (f >> 21)) & 15u) << (4 * k);
          s[k] &= 0x7F7F7F7Fu;
        }
      }
      uint8_t* dst = scales + (c0 + t) * rb_col + r0 / 16;
      if (scales16 && nrb == kRowBlocks) {
        u32x4 o;
        o.x = s[0];
        o.y = s[1];
        o.z = s[2];
        o.w = s[3];
        *reinterpret_cast<u32x4*>(dst) = o;
      } else {
        for (int k = 0; k < nrb; ++k) dst[k] = (uint8_t)(s[k >> 2] >> (8 * (k & 3)));
      }
      if (kSel && sel_direct) {
        // nrb is a multiple of 8 here: one or two whole bitmap bytes.
        uint8_t* bd = selmap + ((c0 + t) * rb_col + r0 / 16) / 8;
        bd[0] = (uint8_t)bits;
        if (nrb > 8) bd[1] = (uint8_t)(bits >> 8);
      }
    }

    if constexpr (kDual) {
      // Row-direction blocks of the same tile (still intact in LDS until the
      // next tile's first barrier): lane t takes tile row t/2 (per pass) and
      // its blocks 2*(t%2) and 2*(t%2) + 1, 32 contiguous bytes each.
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
        const int rr = p * (kColsThreads / 2) + (t >> 1), j0 = (t & 1) * 2;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(&tile[rr * kInPitch + j0 * 32]);
        uint32_t wa[8], wb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          wa[i] = src[i];
          wb[i] = src[8 + i];
        }
        const Block16 ra = quantize_block16<k46, kRule, kNeedErr>(wa, ts.k6, ts.k4, tab);
        const Block16 rb2 = quantize_block16<k46, kRule, kNeedErr>(wb, ts.k6, ts.k4, tab);
        const int64_t gr = r0 + rr, gc = c0 + 16 * j0;
        if (gr < rows && gc < cols) {
          const bool vb = gc + 16 < cols;
          uint8_t* dst = packed_r + gr * (cols / 2) + gc / 2;
          if (vb && codes_r16) {
            *reinterpret_cast<u32x4*>(dst) = u32x4{ra.lo, ra.hi, rb2.lo, rb2.hi};
          } else {
            uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);  // 4-byte aligned
            d32[0] = ra.lo;
            d32[1] = ra.hi;
            if (vb) {
              d32[2] = rb2.lo;
              d32[3] = rb2.hi;
            }
          }
          uint8_t* sd = scales_r + gr * (cols / 16) + gc / 16;
          sd[0] = (uint8_t)(ra.S | (kSel && ra.pick4 ? 0x80u : 0u));
          if (vb) sd[1] = (uint8_t)(rb2.S | (kSel && rb2.pick4 ? 0x80u : 0u));
          if (kErr) acc_r += (double)ra.err + (vb ? (double)rb2.err : 0.0);
        }
      }
    }
  };

  // Each role runs its own copy of the tile loop (the same barriers in the
  // same order), so that neither copy holds the other's memory operations.
  auto run = [&](auto load_role) {
    u32x4 w[kLPL];
    if (decltype(load_role)::value) load_tile(wg, w);
    for (int64_t tt = wg; tt < ntiles; tt += nwg) process(tt, w, load_role);
  };
  if (loader_wave)
    run(std::true_type{});
  else
    run(std::false_type{});

  if (amax_out) group_max_to<kColsWaves>(amax_out, bmax, wmax);  // uniform branch
  if (kErr) {
    for (int off = 32; off > 0; off >>= 1) {
      acc += __shfl_xor(acc, off);
      if (kDual) acc_r += __shfl_xor(acc_r, off);
    }
    if (lane == 0) {
      wsum[wave] = acc;
      wsum_r[wave] = acc_r;
    }
    __syncthreads();
    if (t == 0) {
      double s = wsum[0], sr = wsum_r[0];
      for (int k = 1; k < kColsWaves; ++k) {
        s += wsum[k];
        sr += wsum_r[k];
      }
      unsafeAtomicAdd(err_sum, s);
      if (kDual) unsafeAtomicAdd(err_r, sr);
    }
  }
}

// Bitmap pass for shapes whose columns' bits do not start on byte
// boundaries: byte j of the bitmap collects bit 7 of scale bytes 8j..8j+7,
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

template <uint32_t V, bool kDual>
static hipError_t launch_cols_v(const uint16_t* in, int64_t rows, int64_t cols,
                                const float* gscale, uint8_t* packed, uint8_t* scales,
                                uint8_t* selmap, double* err_sum, uint32_t* amax_out,
                                const DualOut* dual, hipStream_t s, Events ev) {
  constexpr bool kSel = (V & kVarSelmap) != 0;
  // Bitmap passes: the column-blocked bitmap when its columns' bits do not
  // start on byte boundaries, the row-blocked one of a dual call always.
  const bool pass_c = kSel && selmap && (rows / 16) % 8 != 0;
  const bool pass_r = kSel && kDual && dual->selmap_r;
  // The last kernel of the call ends the event bracket.
  const Events first{ev.start, (pass_c || pass_r) ? nullptr : ev.stop};
  const int64_t ntiles =
      ((cols + kTileCols - 1) / kTileCols) * ((rows + kTileRows - 1) / kTileRows);
  int64_t groups = (int64_t)device_cu_count() * kColsGroupsPerCu;
  if (groups > ntiles) groups = ntiles;
  if (groups < 1) groups = 1;
  // A dual call walks strips fastest, so that the four strips sharing each
  // 128-byte line of a row's codes are written through one L2 at once.
  hipError_t e = launch_with_events(
      quantize_cols_kernel<V, kDual>, dim3((unsigned)groups), dim3(kColsThreads), s, first, in,
      rows, cols, gscale, packed, scales, selmap, err_sum, amax_out,
      kDual ? dual->packed_r : nullptr, kDual ? dual->scales_r : nullptr,
      kDual ? dual->err_r : nullptr, kDual ? 1 : 0);
  if (e != hipSuccess) return e;
  auto bitmap_pass = [&](uint8_t* sc, int64_t nblocks, uint8_t* sel, bool last) {
    int64_t g2 = ((nblocks + 7) / 8 + kThreads - 1) / kThreads;
    if (g2 > 4096) g2 = 4096;
    if (g2 < 1) g2 = 1;
    return launch_with_events(selmap_from_scales_kernel, dim3((unsigned)g2), dim3(kThreads), s,
                              Events{nullptr, last ? ev.stop : nullptr}, sc, nblocks, sel);
  };
  if (pass_c) e = bitmap_pass(scales, rows / 16 * cols, selmap, !pass_r);
  if (e == hipSuccess && pass_r) e = bitmap_pass(dual->scales_r, rows * cols / 16, dual->selmap_r, true);
  return e;
}

hipError_t launch_quantize_cols(const uint16_t* in, int64_t rows, int64_t cols,
                                const float* gscale, uint32_t variant, uint8_t* packed,
                                uint8_t* scales, uint8_t* selmap, double* err_sum,
                                uint32_t* amax_out, const DualOut* dual, hipStream_t s,
                                Events ev) {
#define NVFP4_COLS_CASE(v)                                                                    \
  case v:                                                                                     \
    return dual ? launch_cols_v<v, true>(in, rows, cols, gscale, packed, scales, selmap,     \
                                         err_sum, amax_out, dual, s, ev)                     \
                : launch_cols_v<v, false>(in, rows, cols, gscale, packed, scales, selmap,    \
                                          err_sum, amax_out, dual, s, ev);
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
    NVFP4_COLS_CASE(17)
    NVFP4_COLS_CASE(21)
    NVFP4_COLS_CASE(25)
    NVFP4_COLS_CASE(29)
    default:
      return hipErrorInvalidValue;
  }
#undef NVFP4_COLS_CASE
}

}  // namespace nvfp4
