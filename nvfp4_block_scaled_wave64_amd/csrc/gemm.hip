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
// the lanes, so a lane loads 32 consecutive codes (16 bytes, two blocks) of
// its row per 64-wide chunk of K and feeds them to four MFMA steps; A and B
// use the same split, so the k values meet their partners.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;           // 4 waves as 2 x 2
constexpr int kTileM = 256, kTileN = 256;   // workgroup tile
constexpr int kWaveM = 128, kWaveN = 128;   // wave tile
constexpr int kFm = kWaveM / 32, kFn = kWaveN / 32;  // 32 x 32 MFMA tiles per wave
constexpr int kGroupM = 4;                  // tile rows per group of the walk

// The operand fragment of one 32-row slice for one chunk: 32 codes of the
// lane's row (two blocks) and those blocks' scale bytes.
struct Frag {
  u32x4 codes;
  uint32_t scales;  // byte 0: first block, byte 1: second block
};

// Loads the fragment of tile row `r` (relative to the resource base) for
// chunk c; half h of the wave takes blocks 4c + 2h and 4c + 2h + 1.  A block
// at or past the end of K gets scale offset out of range (scale 0, so its
// values are 0 whatever its codes); rows past the end read 0.
__device__ __forceinline__ Frag load_frag(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                          uint32_t r, uint32_t c, uint32_t h, uint32_t nblk) {
  Frag f;
  const uint32_t blk = 4u * c + 2u * h;
  f.codes = __builtin_amdgcn_raw_buffer_load_b128(rc, r * (nblk * 8u) + blk * 8u, 0, 0);
  const uint32_t so = r * nblk + blk;
  const uint32_t s0 = __builtin_amdgcn_raw_buffer_load_b8(rs, blk < nblk ? so : 0xFFFFFFF0u, 0, 0);
  const uint32_t s1 =
      __builtin_amdgcn_raw_buffer_load_b8(rs, blk + 1u < nblk ? so + 1u : 0xFFFFFFF0u, 0, 0);
  f.scales = s0 | (s1 << 8);
  return f;
}

// The 8 f16 operand values of MFMA step t (0..3) of a fragment: codes
// 8t .. 8t+7 times dec(S) of their block (block 0 for t < 2).
__device__ __forceinline__ f16x8 decode_step(const Frag& f, f16x2 dec2, int t) {
  const uint32_t w = f.codes[t];
  const _Float16 d = (t < 2) ? dec2[0] : dec2[1];
  const f16x2 dd = {d, d};
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * dd;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * dd;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * dd;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * dd;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// dec(S) of the fragment's two blocks as f16 (E4M3 -> f16 is exact).
__device__ __forceinline__ f16x2 decode_scales(const Frag& f) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.scales, 1.0f, false);
}

// Buffer resource from values the compiler may hold in vector registers but
// that are the same in every lane (keeps the resource in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const uint8_t* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane(bytes));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  f32x2 p;
  p.x = x;
  p.y = 0.0f;
  return (uint16_t)__builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
}

// One workgroup per 256 x 256 output tile; tiles are walked in groups of
// kGroupM tile rows (the workgroups running together share A and B panels
// in L2), and consecutive tiles of the walk go to one XCD (workgroups are
// dealt round-robin over the 8 XCDs).
template <bool kBf16>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(
    const uint8_t* __restrict__ pa, const uint8_t* __restrict__ sa, const float* __restrict__ ga,
    const uint8_t* __restrict__ pb, const uint8_t* __restrict__ sb, const float* __restrict__ gb,
    int64_t M, int64_t N, int64_t K, uint32_t tiles_m, uint32_t tiles_n, uint32_t per_xcd,
    void* __restrict__ out) {
  const uint32_t total = tiles_m * tiles_n;
  const uint32_t L = (blockIdx.x % 8u) * per_xcd + blockIdx.x / 8u;
  if (L >= total) return;
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
  const uint32_t nchunks = (nblk + 3u) / 4u;

  // Resources over this tile's rows of A and B (rows past M or N read 0).
  const int64_t m0 = (int64_t)tm * kTileM + wm * kWaveM;
  const int64_t n0 = (int64_t)tn * kTileN + wn * kWaveN;
  const uint32_t rows_a = (uint32_t)max<int64_t>(0, min<int64_t>(kWaveM, M - m0));
  const uint32_t rows_b = (uint32_t)max<int64_t>(0, min<int64_t>(kWaveN, N - n0));
  const __amdgpu_buffer_rsrc_t rca = uniform_rsrc(pa + m0 * (K / 2), rows_a * nblk * 8u);
  const __amdgpu_buffer_rsrc_t rsa = uniform_rsrc(sa + m0 * (K / 16), rows_a * nblk);
  const __amdgpu_buffer_rsrc_t rcb = uniform_rsrc(pb + n0 * (K / 2), rows_b * nblk * 8u);
  const __amdgpu_buffer_rsrc_t rsb = uniform_rsrc(sb + n0 * (K / 16), rows_b * nblk);

  f32x16 acc[kFm][kFn];
#pragma unroll
  for (int i = 0; i < kFm; ++i)
#pragma unroll
    for (int j = 0; j < kFn; ++j) acc[i][j] = f32x16{};

  Frag fa[kFm], fb[kFn];
#pragma unroll
  for (int i = 0; i < kFm; ++i) fa[i] = load_frag(rca, rsa, 32u * i + l32, 0u, h, nblk);
#pragma unroll
  for (int j = 0; j < kFn; ++j) fb[j] = load_frag(rcb, rsb, 32u * j + l32, 0u, h, nblk);

  for (uint32_t c = 0; c < nchunks; ++c) {
    Frag na[kFm], nb[kFn];
    const uint32_t cn = c + 1u < nchunks ? c + 1u : c;
#pragma unroll
    for (int i = 0; i < kFm; ++i) na[i] = load_frag(rca, rsa, 32u * i + l32, cn, h, nblk);
#pragma unroll
    for (int j = 0; j < kFn; ++j) nb[j] = load_frag(rcb, rsb, 32u * j + l32, cn, h, nblk);

    f16x2 da[kFm], db[kFn];
#pragma unroll
    for (int i = 0; i < kFm; ++i) da[i] = decode_scales(fa[i]);
#pragma unroll
    for (int j = 0; j < kFn; ++j) db[j] = decode_scales(fb[j]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f16x8 a[kFm], b[kFn];
#pragma unroll
      for (int i = 0; i < kFm; ++i) a[i] = decode_step(fa[i], da[i], t);
#pragma unroll
      for (int j = 0; j < kFn; ++j) b[j] = decode_step(fb[j], db[j], t);
#pragma unroll
      for (int i = 0; i < kFm; ++i)
#pragma unroll
        for (int j = 0; j < kFn; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kFm; ++i) fa[i] = na[i];
#pragma unroll
    for (int j = 0; j < kFn; ++j) fb[j] = nb[j];
  }

  const float gab = (*ga) * (*gb);
#pragma unroll
  for (int i = 0; i < kFm; ++i)
#pragma unroll
    for (int j = 0; j < kFn; ++j) {
      const int64_t col = n0 + 32 * j + l32;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
        if (row >= M) continue;
        const float y = acc[i][j][r] * gab;
        if constexpr (kBf16)
          static_cast<uint16_t*>(out)[row * N + col] = to_bf16_bits(y);
        else
          static_cast<float*>(out)[row * N + col] = y;
      }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* pa, const uint8_t* sa, const float* ga, const uint8_t* pb,
                       const uint8_t* sb, const float* gb, int64_t M, int64_t N, int64_t K,
                       int out_bf16, void* out, hipStream_t s, Events ev) {
  const uint32_t tiles_m = (uint32_t)((M + kTileM - 1) / kTileM);
  const uint32_t tiles_n = (uint32_t)((N + kTileN - 1) / kTileN);
  const uint32_t total = tiles_m * tiles_n;
  const uint32_t per_xcd = (total + 7u) / 8u;
  const dim3 grid(per_xcd * 8u), block(kGemmThreads);
  if (out_bf16)
    return launch_with_events(gemm_kernel<true>, grid, block, s, ev, pa, sa, ga, pb, sb, gb, M,
                              N, K, tiles_m, tiles_n, per_xcd, out);
  return launch_with_events(gemm_kernel<false>, grid, block, s, ev, pa, sa, ga, pb, sb, gb, M, N,
                            K, tiles_m, tiles_n, per_xcd, out);
}

}  // namespace nvfp4
