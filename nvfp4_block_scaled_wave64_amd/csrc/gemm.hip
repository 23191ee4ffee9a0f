// gemm.hip -- W4A4 product of two NVFP4 tensors on the gfx950 matrix cores.
//
// out[m][n] = ga * gb * sum_k a(m,k) * b(n,k), a = v * dec(S), for A [M][K]
// and B [N][K] both blocked along K (packed [rows][K/2], scales [rows][K/16]):
// a linear layer Y = X W^T with NVFP4 activations and weights ("Why Gated
// DeltaNet in hybrid 27B LLMs withstands 4-bit quantization", "Background"),
// and the augmented product of the "ARCQuant" summary ("Methodology"): the
// residual blocks sit along K, so that product is this one with K_in + S.
//
// Exactness of the operands.  v has at most 2 significant bits and dec(S) at
// most 4, so a = v * dec(S) has at most 6; its range [2^-10, 2688] lies in
// the normal range of binary16.  Each element is therefore decoded exactly to
// f16 (the FP4 code by v_cvt_scalef32_pk_f16_fp4 with scale 1, then one f16
// multiply by dec(S), itself exact in f16), and the f16 x f16 products of the
// MFMA are exact in fp32.  What differs from the binary64 definition is only
// the fp32 accumulation and the final scaling by RN(ga * gb).
//
// Layout on the matrix cores (v_mfma_f32_32x32x16_f16, wave64): lane l feeds
// row l % 32 of the A operand and column l % 32 of the B operand with 8
// consecutive k values, lanes 0-31 the first 8 and lanes 32-63 the next 8;
// accumulator element r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.  The sum over k does not depend on how k is split between
// the lanes, so within a 128-wide stage of K lane half h takes the stage's
// k values 64h .. 64h + 63 (four blocks) and feeds 8 of them to each of the
// eight MFMA steps; A and B use the same split, so the k values meet their
// partners.
//
// Data path.  A workgroup computes a 256 x 256 tile with four waves of
// 128 x 128 (the accumulators fill the 256 AGPRs), or, where that fills the
// compute units' rounds of tiles better (smaller products), a 256 x 128 or
// 128 x 128 tile with waves of 128 x 64 or 64 x 64.  K is walked in stages
// of 128 (eight blocks): the stage's codes (64 bytes per tile row of either
// operand, four lanes per row so that every request is one contiguous
// 64-byte piece) and scale bytes go from memory straight into a four-deep
// LDS ring, three stages ahead of the stage the matrix cores work on.  In LDS the 16-byte
// pieces of a row are XOR-swizzled by bits 2-3 of the row, which makes both
// the 16-byte writes and the fragment reads (16 lanes on 16 consecutive
// rows) free of bank conflicts.
#include <type_traits>

#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;                 // 4 waves as 2 x 2
constexpr int kTile = 256;                        // workgroup tile rows, at most
constexpr int kStageBlocks = 8;                   // blocks of K per stage (K = 128)
constexpr int kStages = 4;                        // LDS buffers
constexpr int kAhead = 3;                         // stages in flight ahead of the one computed
constexpr int kRowBytes = kStageBlocks * 8;       // code bytes per row and stage
constexpr int kScaleSlot = 16;                    // LDS bytes per row for its 8 scale bytes
// Per stage: A codes [kTileM][64], B codes [kTileN][64], A scale slots
// [kTileM][16], B scale slots [kTileN][16].
template <int kTileM, int kTileN>
constexpr int kStageBytes = (kTileM + kTileN) * (kRowBytes + kScaleSlot);
constexpr int kGroupM = 4;                        // tile rows per group of the walk

// Buffer resource from values the compiler may hold in vector registers but
// that are the same in every lane (keeps the resource in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const uint8_t* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane(bytes));
}

// LDS offset of 16-byte piece `piece` (0..3) of tile row `row` in a code area.
__device__ __forceinline__ uint32_t code_slot(uint32_t row, uint32_t piece) {
  return row * kRowBytes + 16u * (piece ^ ((row >> 2) & 3u));
}

// The loads of one stage go out in parts spread over the MFMA steps of the
// stage before (a burst of them would stall the in-order issue of the
// MFMAs): part q < 4 is the q-th code load of each operand (an operand with
// a 128-row tile has two), part 4 the scale load of A, part 5 that of B.
//
// Code loads go straight to LDS (buffer_load ... lds): lane l of load q
// writes bytes 16l .. 16l + 15 of the 1 KiB that holds tile rows
// R w + 16q .. R w + 16q + 15 (R = tile rows / 4 per wave), which is
// physical piece l % 4 of row R w + 16q + l / 4, so the lane loads the
// row's logical piece (l % 4) ^ ((row >> 2) & 3).  Scale loads do the same
// with one 16-byte window per row (lane l: row 64w + l, waves with no such
// rows loading into a spare buffer): the 16 bytes from the 4-byte
// boundary at or below the row's first scale byte of the stage, which
// contain its 8 bytes at offset (d0 + row * nblk) % 4 whatever K is (d0:
// the tile's first scale byte's offset above the 4-byte boundary below it,
// where the scale resource starts; the resource ends at the 4-byte boundary
// above the tile's last scale byte, because its range check drops whole
// dwords -- the extra bytes share a dword, hence a page, with valid ones and
// are never used).  Rows past the tile's valid rows read 0; blocks at or
// past the end of K are masked to scale 0 by the reader, so their codes
// (whatever they read) contribute 0.  With `live` false (no such stage)
// every load is out of range and writes zeros to a buffer that is not read
// again.
constexpr uint32_t kOut = 0xFFFFFFF0u;  // past any resource range: reads 0

// kRows: the operand's tile rows (256, or 128 for a narrow B tile), split
// evenly over the four waves.
template <int kRows>
__device__ __forceinline__ void issue_codes(__amdgpu_buffer_rsrc_t rc, uint8_t* codes_lds,
                                            uint32_t c, int q, bool live, uint32_t nblk,
                                            uint32_t wave, uint32_t lane) {
  const uint32_t first = (uint32_t)(kRows / 4) * wave + 16u * (uint32_t)q;
  const uint32_t row = first + (lane >> 2);
  const uint32_t piece = (lane & 3u) ^ ((row >> 2) & 3u);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rc, (__attribute__((address_space(3))) void*)(codes_lds + first * kRowBytes), 16,
      live ? row * (nblk * 8u) + c * kRowBytes + 16u * piece : kOut, 0, 0, 0);
}

// One load covers the 64 rows from `first` and writes their slots at dst.
__device__ __forceinline__ void issue_scales(__amdgpu_buffer_rsrc_t rs, uint8_t* dst,
                                             uint32_t first, uint32_t c, bool live, uint32_t nblk,
                                             uint32_t d0, uint32_t lane) {
  const uint32_t row = first + lane;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)dst, 16,
      live ? (d0 + row * nblk + c * kStageBlocks) & ~3u : kOut, 0, 0, 0);
}

// Scale-byte resource of a tile's rows (see issue_scales): starts at the
// 4-byte boundary at or below p, and ends at the one at or above p + bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scale_rsrc(const uint8_t* p, uint32_t bytes,
                                                             uint32_t& d0) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  d0 = __builtin_amdgcn_readfirstlane((uint32_t)(a & 3u));
  return uniform_rsrc(reinterpret_cast<const uint8_t*>(a - d0), (d0 + bytes + 3u) & ~3u);
}

// Vector-memory operations a wave issues per stage: its code loads of A
// (kTileM / 64) and B (kTileN / 64) and one scale load per operand.  With a
// 128-row tile of an operand only waves 0 and 1 have scale rows of it to
// load; waves 2 and 3 issue an out-of-range load into a spare 1 KiB of LDS
// that nobody reads, so every wave waits for the same count.
template <int kTileM, int kTileN>
constexpr int kLoadsPerStage = kTileM / 64 + kTileN / 64 + 2;
constexpr int kSpareBytes = 64 * kScaleSlot;

// Waits until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier after this wave's LDS writes have completed; the
// loads still in flight (the stages ahead) are not waited for.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Codes of tile row `row` for lane half h: piece 2h holds the stage's
// codes for MFMA steps 0-3, piece 2h + 1 those for steps 4-7.
__device__ __forceinline__ u32x4 read_codes(const uint8_t* codes, uint32_t row, uint32_t piece) {
  return *reinterpret_cast<const u32x4*>(codes + code_slot(row, piece));
}

// dec(S) of the four blocks of lane half h in stage c as f16 (E4M3 -> f16
// is exact): lo = blocks 4h, 4h + 1 (steps 0-3), hi = blocks 4h + 2, 4h + 3
// (steps 4-7).  The row's bytes sit at offset (d0 + row * nblk) % 4 of its slot
// (0 when d0 = 0 and nblk % 4 == 0); blocks at or past nblk read scale 0.
template <bool kAligned>
__device__ __forceinline__ void read_scales(const uint8_t* scales, uint32_t row, uint32_t h,
                                            uint32_t c, uint32_t nblk, uint32_t d0, f16x2& lo,
                                            f16x2& hi) {
  const uint32_t* slot = reinterpret_cast<const uint32_t*>(scales + row * kScaleSlot);
  uint32_t s;
  if constexpr (kAligned) {
    s = slot[h];
  } else {
    const uint32_t b = ((d0 + row * nblk) & 3u) + 4u * h;
    s = __builtin_amdgcn_alignbyte(slot[(b >> 2) + 1], slot[b >> 2], b & 3u);
  }
  const int32_t valid = (int32_t)nblk - (int32_t)(c * kStageBlocks + 4u * h);
  if (valid < 4) s = valid <= 0 ? 0u : s & (0xFFFFFFFFu >> (8 * (4 - valid)));
  lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true);
}

// The 8 f16 operand values of one MFMA step: the 8 codes of word w times
// dec(S) of their block.
__device__ __forceinline__ f16x8 decode8(uint32_t w, _Float16 d) {
  const f16x2 dd = {d, d};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * dd;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * dd;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * dd;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * dd;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  f32x2 p;
  p.x = x;
  p.y = 0.0f;
  return (uint16_t)__builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}

// One workgroup per 256 x kTileN output tile and split of K; tiles are
// walked in groups of kGroupM tile rows (the workgroups running together
// share A and B panels in L2), and consecutive units of the walk go to one
// XCD (workgroups are dealt round-robin over the 8 XCDs).  With kSplit the
// stages of K are divided into `splits` contiguous ranges; unit u covers
// range u / tiles of tile u % tiles and stores its raw fp32 sums in slice
// u / tiles of ws ([splits][M][N], passed as out); splitk_reduce_kernel then
// adds the slices.  Without kSplit, splits is 1 and the unit writes out.
template <bool kBf16, bool kAligned, int kTileM, int kTileN, bool kSplit>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(
    const uint8_t* __restrict__ pa, const uint8_t* __restrict__ sa, const float* __restrict__ ga,
    const uint8_t* __restrict__ pb, const uint8_t* __restrict__ sb, const float* __restrict__ gb,
    int64_t M, int64_t N, int64_t K, uint32_t tiles_m, uint32_t tiles_n, uint32_t per_xcd,
    uint32_t splits, void* __restrict__ out) {
  constexpr int kStage = kStageBytes<kTileM, kTileN>;
  constexpr int kCodesA = kTileM * kRowBytes, kCodesB = kTileN * kRowBytes;
  constexpr int kScalesA = kTileM * kScaleSlot;
  constexpr int kWaveTileM = kTileM / 2;       // wave tile rows (rows of A)
  constexpr int kFragsA = kWaveTileM / 32;     // 32 x 32 MFMA tiles per wave along A
  constexpr int kWaveTileN = kTileN / 2;       // wave tile columns (rows of B)
  constexpr int kFragsB = kWaveTileN / 32;     // 32 x 32 MFMA tiles per wave along B
  constexpr bool kSpare = kTileM < kTile || kTileN < kTile;
  __shared__ __align__(16) uint8_t lds[kStages * kStage + (kSpare ? kSpareBytes : 0)];
  const uint32_t tiles = tiles_m * tiles_n;
  const uint32_t U = (blockIdx.x % 8u) * per_xcd + blockIdx.x / 8u;
  if (U >= tiles * splits) return;
  const uint32_t split = U / tiles;
  const uint32_t L = U - split * tiles;
  const uint32_t group = L / (kGroupM * tiles_n);
  const uint32_t first_m = group * kGroupM;
  const uint32_t gm = min((uint32_t)kGroupM, tiles_m - first_m);
  const uint32_t in_group = L - group * kGroupM * tiles_n;
  const uint32_t tm = first_m + in_group % gm;
  const uint32_t tn = in_group / gm;

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wm = wave >> 1, wn = wave & 1u;
  const uint32_t h = lane >> 5, l32 = lane & 31u;
  const uint32_t nblk = (uint32_t)(K / 16);
  const uint32_t nstages = (nblk + kStageBlocks - 1) / kStageBlocks;
  // This unit's stages c_begin .. c_end - 1 (all of them without kSplit;
  // splits <= nstages, so no range is empty).
  const uint32_t c_begin = (uint32_t)((uint64_t)split * nstages / splits);
  const uint32_t c_end = (uint32_t)((uint64_t)(split + 1u) * nstages / splits);
  const uint32_t nst = c_end - c_begin;

  // Resources over this tile's rows of A and B (rows past M or N read 0).
  const int64_t m0 = (int64_t)tm * kTileM, n0 = (int64_t)tn * kTileN;
  const uint32_t rows_a = (uint32_t)min<int64_t>(kTileM, M - m0);
  const uint32_t rows_b = (uint32_t)min<int64_t>(kTileN, N - n0);
  // Whether this wave loads scale rows of A and of B (64 from row 64 * wave).
  const bool a_scales = kTileM >= kTile || wave < (uint32_t)(kTileM / 64);
  const bool b_scales = kTileN >= kTile || wave < (uint32_t)(kTileN / 64);
  const __amdgpu_buffer_rsrc_t rca = uniform_rsrc(pa + m0 * (K / 2), rows_a * nblk * 8u);
  uint32_t da = 0, db = 0;  // scale resources' offsets below their tiles' first bytes
  const __amdgpu_buffer_rsrc_t rsa = scale_rsrc(sa + m0 * (K / 16), rows_a * nblk, da);
  const __amdgpu_buffer_rsrc_t rcb = uniform_rsrc(pb + n0 * (K / 2), rows_b * nblk * 8u);
  const __amdgpu_buffer_rsrc_t rsb = scale_rsrc(sb + n0 * (K / 16), rows_b * nblk, db);

  f32x16 acc[kFragsA][kFragsB];
#pragma unroll
  for (int i = 0; i < kFragsA; ++i)
#pragma unroll
    for (int j = 0; j < kFragsB; ++j) acc[i][j] = f32x16{};

  auto stage_ptr = [&](uint32_t c) { return lds + (c % kStages) * kStage; };
  // Part q (0..5) of the loads of stage c (see issue_codes): the q-th code
  // load of A and of B (they have kTileM / 64 and kTileN / 64 of them), then
  // A's scale load, then B's.
  auto issue_part = [&](uint32_t c, int q, bool live) {
    uint8_t* st = stage_ptr(c);
    if (q < 4) {
      if (q < kTileM / 64) issue_codes<kTileM>(rca, st, c, q, live, nblk, wave, lane);
      if (q < kTileN / 64) issue_codes<kTileN>(rcb, st + kCodesA, c, q, live, nblk, wave, lane);
    } else if (q == 4) {
      uint8_t* dst = a_scales ? st + kCodesA + kCodesB + 64u * wave * kScaleSlot
                              : lds + kStages * kStage;
      issue_scales(rsa, dst, 64u * wave, c, live && a_scales, nblk, da, lane);
    } else {
      uint8_t* dst = b_scales ? st + kCodesA + kCodesB + kScalesA + 64u * wave * kScaleSlot
                              : lds + kStages * kStage;
      issue_scales(rsb, dst, 64u * wave, c, live && b_scales, nblk, db, lane);
    }
  };
  auto issue = [&](uint32_t c) {
#pragma unroll
    for (int q = 0; q < 6; ++q) issue_part(c, q, true);
  };

  // Pipeline: stage c is computed while the loads of stages c + 1 .. c + 3
  // are in flight; at the end of stage c this wave waits for its loads of
  // stage c + 2 (only stage c + 3's may stay outstanding) and the barrier
  // publishes them.  So during stage c, stages c and c + 1 are complete in
  // LDS, and buffer (c + 3) % 4, which receives stage c + 3, is read by
  // nobody.
  issue(c_begin);
  if (nst > 1) issue(c_begin + 1u);
  if (nst > 2) {
    issue(c_begin + 2u);
    wait_vm<kLoadsPerStage<kTileM, kTileN>>();
  } else {
    wait_vm<0>();
  }
  lds_barrier();

  // Operand r < kFragsA is A fragment r (tile row wm * kWaveTileM + 32r + l32), the
  // others B fragments (tile row wn * kWaveTileN + 32(r - kFragsA) + l32).
  // Software pipeline across stages: the codes of
  // steps 4-7 are read from LDS while steps 0-3 run, those of the next
  // stage's steps 0-3 (already in LDS: written before the previous barrier)
  // while steps 4-7 run, and each step's operands are decoded while the
  // matrix cores work on the step before.
  constexpr int kOps = kFragsA + kFragsB;
  auto op_row = [&](int r) {
    return r < kFragsA ? wm * kWaveTileM + 32u * (uint32_t)r + l32
                      : wn * kWaveTileN + 32u * (uint32_t)(r - kFragsA) + l32;
  };
  auto codes_of = [&](const uint8_t* st, int r) { return st + (r < kFragsA ? 0 : kCodesA); };
  auto scales_of = [&](const uint8_t* st, int r) {
    return st + kCodesA + kCodesB + (r < kFragsA ? 0 : kScalesA);
  };
  u32x4 lo[kOps], hi[kOps];
  f16x2 dlo[kOps], dhi[kOps], ndlo[kOps], ndhi[kOps];
  f16x8 op[2][kOps];
  {
    const uint8_t* st = stage_ptr(c_begin);
#pragma unroll
    for (int r = 0; r < kOps; ++r) {
      lo[r] = read_codes(codes_of(st, r), op_row(r), 2u * h);
      read_scales<kAligned>(scales_of(st, r), op_row(r), h, c_begin, nblk,
                            r < kFragsA ? da : db, dlo[r], dhi[r]);
    }
#pragma unroll
    for (int r = 0; r < kOps; ++r) op[0][r] = decode8(lo[r][0], dlo[r][0]);
  }
  // vm: vector-memory instructions to place among this step's MFMAs; the
  // next step's decode (8 VALU per operand) is spread evenly over them.  The
  // slots hold two VALU instructions more than the decode needs where that
  // measured faster (256 x 256 and 128 x 128 tiles): the stage's other VALU
  // work (scale bytes, addresses) then also lands between MFMAs instead of
  // in runs the matrix cores wait through.  Measured on MI355X: 32768 x 5120
  // x 5120 2% faster, 128 x 5120 x 5120 9.5% faster, 256 x 128 tiles
  // (1024 x 5120 x 5120) unchanged without the extra slots.
  constexpr int kValuPerMfma =
      8 * kOps / (kFragsA * kFragsB) + ((kTileM == kTileN) ? 2 : 0);
  auto mfma_step = [&](int cur, auto vm_c) {
    constexpr int vm = decltype(vm_c)::value;
#pragma unroll
    for (int i = 0; i < kFragsA; ++i)
#pragma unroll
      for (int j = 0; j < kFragsB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op[cur][i], op[cur][kFragsA + j],
                                                           acc[i][j], 0, 0, 0);
#pragma unroll
    for (int k = 0; k < kFragsA * kFragsB; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);  // decode
      if constexpr (vm > 0)
        if (k == 2) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);  // loads
    }
  };

  for (uint32_t c = c_begin; c < c_end; ++c) {
    const bool more = c + kAhead < c_end;
    const uint8_t* st = stage_ptr(c);
#pragma unroll
    for (int r = 0; r < kOps; ++r) hi[r] = read_codes(codes_of(st, r), op_row(r), 2u * h + 1u);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int cur = t & 1, nxt = cur ^ 1;
      issue_part(c + kAhead, t, more);
#pragma unroll
      for (int r = 0; r < kOps; ++r)
        op[nxt][r] = t < 3 ? decode8(lo[r][t + 1], dlo[r][(t + 1) >> 1])
                           : decode8(hi[r][0], dhi[r][0]);
      const int nvm = (t < kTileM / 64 ? 1 : 0) + (t < kTileN / 64 ? 1 : 0);
      if (nvm == 2)
        mfma_step(cur, std::integral_constant<int, 2>{});
      else if (nvm == 1)
        mfma_step(cur, std::integral_constant<int, 1>{});
      else
        mfma_step(cur, std::integral_constant<int, 0>{});
    }
    // The next stage's first codes and scales (stage c + 1 is in LDS; on the
    // last stage this reads a stale buffer whose values are never used).
    const uint8_t* sn = stage_ptr(c + 1);
#pragma unroll
    for (int r = 0; r < kOps; ++r) {
      lo[r] = read_codes(codes_of(sn, r), op_row(r), 2u * h);
      read_scales<kAligned>(scales_of(sn, r), op_row(r), h, c + 1u, nblk, r < kFragsA ? da : db,
                            ndlo[r], ndhi[r]);
    }
#pragma unroll
    for (int t = 4; t < 8; ++t) {
      const int cur = t & 1, nxt = cur ^ 1;
      if (t < 6) issue_part(c + kAhead, t, more);
#pragma unroll
      for (int r = 0; r < kOps; ++r)
        op[nxt][r] = t < 7 ? decode8(hi[r][t - 3], dhi[r][(t - 3) >> 1])
                           : decode8(lo[r][0], ndlo[r][0]);
      if (t < 6)
        mfma_step(cur, std::integral_constant<int, 1>{});
      else
        mfma_step(cur, std::integral_constant<int, 0>{});
    }
#pragma unroll
    for (int r = 0; r < kOps; ++r) {
      dlo[r] = ndlo[r];
      dhi[r] = ndhi[r];
    }
    // This stage's loads of stage c + 3 (issued even past the unit's last
    // stage, then out of range) may stay in flight; stage c + 2's are
    // complete.
    wait_vm<kLoadsPerStage<kTileM, kTileN>>();
    lds_barrier();
  }

  wait_vm<0>();
  // Epilogue: out = acc * RN(ga * gb), or with kSplit the raw sums into the
  // unit's slice (a multiply by 1 is exact).  One buffer resource per 32-row
  // slice (its range drops rows past M); a lane's column offset is per lane,
  // the row offset of accumulator element r a scalar (N <= 2^24 keeps a
  // slice's byte offsets in 32 bits).
  static_assert(!(kSplit && kBf16), "split units store fp32 sums");
  const float gab = kSplit ? 1.0f : (*ga) * (*gb);
  if constexpr (kSplit) out = static_cast<float*>(out) + (int64_t)split * M * N;
  const int64_t mw = m0 + wm * kWaveTileM, nw = n0 + wn * kWaveTileN;
  constexpr uint32_t kEsz = kBf16 ? 2u : 4u;
  const uint32_t row_bytes = (uint32_t)N * kEsz;
#pragma unroll
  for (int i = 0; i < kFragsA; ++i) {
    const int64_t r0 = mw + 32 * i;
    const uint32_t rows = (uint32_t)max<int64_t>(0, min<int64_t>(32, M - r0));
    const __amdgpu_buffer_rsrc_t ro =
        uniform_rsrc(static_cast<uint8_t*>(out) + r0 * (int64_t)row_bytes, rows * row_bytes);
#pragma unroll
    for (int j = 0; j < kFragsB; ++j) {
      const int64_t col = nw + 32 * j + l32;
      if (col >= N) continue;
      const uint32_t voff = 4u * h * row_bytes + (uint32_t)col * kEsz;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t soff = (uint32_t)(8 * (r / 4) + (r % 4)) * row_bytes;
        const float y = acc[i][j][r] * gab;
        if constexpr (kBf16)
          __builtin_amdgcn_raw_buffer_store_b16(to_bf16_bits(y), ro, voff, soff, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), ro, voff, soff, 0);
      }
    }
  }
}

template <bool kBf16, bool kAligned, int kTileM, int kTileN, bool kSplit>
hipError_t launch_gemm_v(const uint8_t* pa, const uint8_t* sa, const float* ga, const uint8_t* pb,
                         const uint8_t* sb, const float* gb, int64_t M, int64_t N, int64_t K,
                         uint32_t splits, void* out, hipStream_t s, Events ev) {
  const uint32_t tiles_m = (uint32_t)((M + kTileM - 1) / kTileM);
  const uint32_t tiles_n = (uint32_t)((N + kTileN - 1) / kTileN);
  const uint32_t per_xcd = (tiles_m * tiles_n * splits + 7u) / 8u;
  return launch_with_events(gemm_kernel<kBf16, kAligned, kTileM, kTileN, kSplit>,
                            dim3(per_xcd * 8u),
                            dim3(kGemmThreads), s, ev, pa, sa, ga, pb, sb, gb, M, N, K, tiles_m,
                            tiles_n, per_xcd, splits, out);
}

// Tile shape for an M x N product with `splits` units per tile.  Tiles run
// in rounds of one per compute unit; measured at full load, a 128 x 128
// tile takes about 0.43 and a 256 x 128 tile about 0.61 of the time of a
// 256 x 256 one (smaller tiles decode more per MFMA: 8 and 6 VALU
// instructions against 4), so each shape costs its rounds times that
// weight and the cheapest wins (ties to the larger tile).
enum class TileShape { k128x128, k256x128, k256x256 };
TileShape pick_tile(int64_t M, int64_t N, int64_t splits) {
  const int64_t cus = device_cu_count();
  auto cost = [&](int64_t tm, int64_t tn, int64_t weight) {
    const int64_t units = ((M + tm - 1) / tm) * ((N + tn - 1) / tn) * splits;
    return (units + cus - 1) / cus * weight;
  };
  const int64_t c_wide = cost(256, 256, 100), c_narrow = cost(256, 128, 61);
  const int64_t c_small = cost(128, 128, 43);
  if (c_small < c_narrow && c_small < c_wide) return TileShape::k128x128;
  return c_narrow < c_wide ? TileShape::k256x128 : TileShape::k256x256;
}

template <bool kBf16, bool kAligned>
hipError_t launch_gemm_t(const uint8_t* pa, const uint8_t* sa, const float* ga, const uint8_t* pb,
                         const uint8_t* sb, const float* gb, int64_t M, int64_t N, int64_t K,
                         void* out, hipStream_t s, Events ev) {
  const TileShape t = pick_tile(M, N, 1);
  if (t == TileShape::k128x128)
    return launch_gemm_v<kBf16, kAligned, 128, 128, false>(pa, sa, ga, pb, sb, gb, M, N, K, 1u,
                                                           out, s, ev);
  if (t == TileShape::k256x128)
    return launch_gemm_v<kBf16, kAligned, 256, 128, false>(pa, sa, ga, pb, sb, gb, M, N, K, 1u,
                                                           out, s, ev);
  return launch_gemm_v<kBf16, kAligned, 256, 256, false>(pa, sa, ga, pb, sb, gb, M, N, K, 1u,
                                                         out, s, ev);
}

// out[i] = (ws[0][i] + ws[1][i] + ... + ws[splits-1][i]) * RN(ga * gb), the
// slices added in order in fp32 (so one split reproduces the unsplit
// product bit for bit), over the mn elements of the product.  With kVec
// (mn a multiple of 4, ws 16-byte and out 4-element aligned) each thread
// takes 4 consecutive elements per step, with 16-byte loads.
template <bool kBf16, bool kVec>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws,
                                                            int64_t mn, uint32_t splits,
                                                            const float* __restrict__ ga,
                                                            const float* __restrict__ gb,
                                                            void* __restrict__ out) {
  const float gab = (*ga) * (*gb);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if constexpr (kVec) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int64_t n4 = mn / 4;
    const f32x4* w4 = reinterpret_cast<const f32x4*>(ws);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
      f32x4 t = w4[i];
      for (uint32_t q = 1; q < splits; ++q) {
        const f32x4 u = w4[(int64_t)q * n4 + i];
        t.x = t.x + u.x;
        t.y = t.y + u.y;
        t.z = t.z + u.z;
        t.w = t.w + u.w;
      }
      const float y0 = t.x * gab, y1 = t.y * gab, y2 = t.z * gab, y3 = t.w * gab;
      if constexpr (kBf16) {
        u32x2 o;
        o.x = (uint32_t)to_bf16_bits(y0) | ((uint32_t)to_bf16_bits(y1) << 16);
        o.y = (uint32_t)to_bf16_bits(y2) | ((uint32_t)to_bf16_bits(y3) << 16);
        static_cast<u32x2*>(out)[i] = o;
      } else {
        static_cast<f32x4*>(out)[i] = f32x4{y0, y1, y2, y3};
      }
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < mn; i += stride) {
      float t = ws[i];
      for (uint32_t q = 1; q < splits; ++q) t = t + ws[(int64_t)q * mn + i];
      const float y = t * gab;
      if constexpr (kBf16)
        static_cast<uint16_t*>(out)[i] = to_bf16_bits(y);
      else
        static_cast<float*>(out)[i] = y;
    }
  }
}

template <bool kAligned>
hipError_t launch_gemm_split_t(const uint8_t* pa, const uint8_t* sa, const float* ga,
                               const uint8_t* pb, const uint8_t* sb, const float* gb, int64_t M,
                               int64_t N, int64_t K, uint32_t splits, float* ws, hipStream_t s) {
  const TileShape t = pick_tile(M, N, splits);
  if (t == TileShape::k128x128)
    return launch_gemm_v<false, kAligned, 128, 128, true>(pa, sa, ga, pb, sb, gb, M, N, K, splits,
                                                          ws, s, Events{});
  if (t == TileShape::k256x128)
    return launch_gemm_v<false, kAligned, 256, 128, true>(pa, sa, ga, pb, sb, gb, M, N, K, splits,
                                                          ws, s, Events{});
  return launch_gemm_v<false, kAligned, 256, 256, true>(pa, sa, ga, pb, sb, gb, M, N, K, splits,
                                                        ws, s, Events{});
}

}  // namespace

hipError_t launch_gemm(const uint8_t* pa, const uint8_t* sa, const float* ga, const uint8_t* pb,
                       const uint8_t* sb, const float* gb, int64_t M, int64_t N, int64_t K,
                       int out_bf16, void* out, hipStream_t s, Events ev) {
  // Every scale row starts 4-byte aligned when K / 16 is a multiple of 4 and
  // the scale pointers are; otherwise the reader shifts each row's bytes
  // into place (scale windows start at the 4-byte boundary below them).
  const bool aligned = (K / 16) % 4 == 0 && (reinterpret_cast<uintptr_t>(sa) & 3u) == 0 &&
                       (reinterpret_cast<uintptr_t>(sb) & 3u) == 0;
  if (out_bf16)
    return aligned ? launch_gemm_t<true, true>(pa, sa, ga, pb, sb, gb, M, N, K, out, s, ev)
                   : launch_gemm_t<true, false>(pa, sa, ga, pb, sb, gb, M, N, K, out, s, ev);
  return aligned ? launch_gemm_t<false, true>(pa, sa, ga, pb, sb, gb, M, N, K, out, s, ev)
                 : launch_gemm_t<false, false>(pa, sa, ga, pb, sb, gb, M, N, K, out, s, ev);
}

hipError_t launch_gemm_splitk(const uint8_t* pa, const uint8_t* sa, const float* ga,
                              const uint8_t* pb, const uint8_t* sb, const float* gb, int64_t M,
                              int64_t N, int64_t K, uint32_t splits, int out_bf16, void* out,
                              float* ws, hipStream_t s) {
  const bool aligned = (K / 16) % 4 == 0 && (reinterpret_cast<uintptr_t>(sa) & 3u) == 0 &&
                       (reinterpret_cast<uintptr_t>(sb) & 3u) == 0;
  const hipError_t e =
      aligned ? launch_gemm_split_t<true>(pa, sa, ga, pb, sb, gb, M, N, K, splits, ws, s)
              : launch_gemm_split_t<false>(pa, sa, ga, pb, sb, gb, M, N, K, splits, ws, s);
  if (e != hipSuccess) return e;
  const int64_t mn = M * N;
  const uintptr_t out_align = out_bf16 ? 8u : 16u;
  const bool vec = mn % 4 == 0 && (reinterpret_cast<uintptr_t>(ws) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(out) & (out_align - 1u)) == 0;
  int64_t groups = ((vec ? mn / 4 : mn) + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (groups > cap) groups = cap;
  auto* k = out_bf16 ? (vec ? splitk_reduce_kernel<true, true> : splitk_reduce_kernel<true, false>)
                     : (vec ? splitk_reduce_kernel<false, true> : splitk_reduce_kernel<false, false>);
  k<<<(unsigned)groups, 256, 0, s>>>(ws, mn, splits, ga, gb, out);
  return hipGetLastError();
}

int gemm_splits_hint(int64_t M, int64_t N, int64_t K) {
  // The split count with the lowest modelled time, each split keeping at
  // least four stages of K.  Model (fitted to measurements on MI355X at
  // full load): a unit of S splits runs ceil(nstages / S) stages at 1.075,
  // 1.525 or 2.5 us per stage for the 128 x 128, 256 x 128 or 256 x 256 tile
  // the launch picks, plus 2 us of prologue and epilogue; units run in
  // rounds of one per compute unit; with S > 1 the reduce pass adds 3 us
  // plus 1.6 us per split and 2^20 outputs.
  const int64_t cus = device_cu_count();
  const int64_t nstages = (K / 16 + kStageBlocks - 1) / kStageBlocks;
  int64_t cap = nstages / 4;
  if (cap > kGemmMaxSplits) cap = kGemmMaxSplits;
  const double mn_mi = (double)M * (double)N / 1048576.0;
  int best_s = 1;
  double best = 0.0;
  for (int64_t S = 1; S <= (cap < 1 ? 1 : cap); ++S) {
    const TileShape t = pick_tile(M, N, S);
    const int64_t tm = t == TileShape::k128x128 ? 128 : 256;
    const int64_t tn = t == TileShape::k256x256 ? 256 : 128;
    const double per_stage = t == TileShape::k128x128   ? 1.075
                             : t == TileShape::k256x128 ? 1.525
                                                        : 2.5;
    const int64_t units = ((M + tm - 1) / tm) * ((N + tn - 1) / tn) * S;
    const int64_t rounds = (units + cus - 1) / cus;
    const int64_t stages = (nstages + S - 1) / S;
    double time = (double)rounds * ((double)stages * per_stage + 2.0);
    if (S > 1) time += 3.0 + 1.6 * (double)S * mn_mi;
    if (S == 1 || time < best) {
      best = time;
      best_s = (int)S;
    }
  }
  return best_s;
}

}  // namespace nvfp4
