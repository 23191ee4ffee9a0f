// nvfp4_device.h -- device-side building blocks of the gfx950 NVFP4 kernels.
//
// Number formats ("Technical summary: Four Over Six (4/6)", gist.science
// 2512.02010, "Problem statement" and "Implementation details"):
//   E2M1 element codes, magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3;
//   OCP E4M3FN block scales, bias 7, subnormals m * 2^-9, largest finite 448.
//
// All helpers here are exact: every rounding is one IEEE binary32 operation
// with round-to-nearest-even, fp32 denormals are preserved (the kernels are
// built without flush-to-zero), and the build disables fp contraction so
// that no a*b+c is fused unless written as __builtin_fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kFltMax = 3.40282346638528859812e+38f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: the input is read once).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Two bf16 values packed in one dword (element 2j in the low half) widened
// exactly to fp32: bf16 is the upper half of a binary32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- E4M3 ----

// Decode an E4M3 byte (0x00..0x7E).  Placing the 7 payload bits at bit 20 of a
// binary32 word gives dec(S) * 2^-120 for normal and subnormal codes alike
// (the E4M3 exponent bias 7 against binary32's 127); the multiply by 2^120 is
// exact.
__device__ __forceinline__ float e4m3_decode(uint32_t S) {
  return __uint_as_float(S << 20) * 0x1p120f;
}

// Encode s >= 0 to E4M3 with round-to-nearest-even, saturating at 448; NaN
// and non-positive inputs give 0.  Rounding to 3 fraction bits is a single
// add of C = 2^20 * P, where P is the power of two at or below max(s, 2^-6):
// the ulp of C is P/8, the spacing of E4M3 in the binade of s (and 2^-9 in
// the subnormal range).  The rounded value q times 2^-120 has the E4M3 code
// in bits 20..26 (see e4m3_decode).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  s = fminf(fmaxf(s, 0.0f), 448.0f);
  const float p = __uint_as_float(__float_as_uint(fmaxf(s, 0x1p-6f)) & 0x7F800000u);
  const float t = __builtin_fmaf(p, 0x1p20f, s);
  const float q = __builtin_fmaf(-p, 0x1p20f, t);
  return __float_as_uint(q * 0x1p-120f) >> 20;
}

// ---------------------------------------------------------------- E2M1 ----

// Round a >= 0 (finite or +inf) to the E2M1 magnitude grid with
// round-to-nearest-even, saturating at 6.  Same construction as e4m3_encode:
// the grid has 1 fraction bit, spacing 0.5 below 2 (C = 2^22), 1 in [2, 4)
// (C = 2^23) and 2 in [4, 8) (C = 2^24).  Clamping to 6 first keeps every
// result on the grid.  Returns the grid value (0, 0.5, ..., 6).
__device__ __forceinline__ float e2m1_round(float a) {
  a = fminf(a, 6.0f);
  const float p = __uint_as_float(__float_as_uint(fmaxf(a, 1.0f)) & 0x7F800000u);
  const float t = __builtin_fmaf(p, 0x1p22f, a);
  return __builtin_fmaf(-p, 0x1p22f, t);
}

// The 3-bit magnitude index of a grid value q in {0, 0.5, ..., 6}: q * 2^-126
// is a binary32 number whose exponent and top fraction bit are exactly the
// E2M1 exponent and mantissa (0.5 lands on the subnormal 2^-127).
__device__ __forceinline__ uint32_t e2m1_index(float q) {
  return __float_as_uint(q * 0x1p-126f) >> 22;
}

// ---------------------------------------------------------------- lanes ----

// Value of the neighbouring lane of a lane pair (lane ^ 1) via DPP
// quad_perm [1, 0, 3, 2].
__device__ __forceinline__ uint32_t pair_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ float pair_swap(float v) {
  return __uint_as_float(pair_swap(__float_as_uint(v)));
}

// Per-launch scale constants derived from g ("Implementation details": the
// tensor scale; the encode side uses its reciprocal).
struct TensorScales {
  float g;   // decode scale
  float G;   // encode scale 1/g, or 0 when not a positive finite number
  float k6;  // G / 6
  float k4;  // G / 4
};

__device__ __forceinline__ TensorScales tensor_scales(float g) {
  TensorScales t;
  t.g = g;
  float G = 1.0f / g;
  if (!(G > 0.0f && G <= kFltMax)) G = 0.0f;
  t.G = G;
  t.k6 = G / 6.0f;
  t.k4 = G / 4.0f;
  return t;
}

// Decode multiplier d = dec(S) * g and encode multiplier
// r = min(G * (1/dec(S)), FLT_MAX) (r = 0 for S = 0) of block scale S.
__device__ __forceinline__ float2 scale_pair(uint32_t S, const TensorScales& t) {
  const float dec = e4m3_decode(S);
  const float inv = (S == 0u) ? 0.0f : 1.0f / dec;
  float2 dr;
  dr.x = dec * t.g;
  dr.y = fminf(t.G * inv, kFltMax);
  return dr;
}

}  // namespace nvfp4

namespace nvfp4 {

// Result of one half block (8 elements) after the pair's joint decision.
struct HalfBlock {
  uint32_t word;  // 8 codes, element i in bits 4i..4i+3
  uint32_t S;     // kept E4M3 scale byte (same in both lanes of the pair)
  bool pick4;     // the max->4 candidate was kept
  float err;      // kept candidate's block error (same in both lanes)
};

// One lane's half of a block held by a lane pair: wd are the lane's 8 bf16
// values (element 2j in the low half of wd[j]); `odd` says whether this is
// the second half.  k_mine is k6 on even lanes and k4 on odd lanes (4/6);
// tab[S] = (d, r) for every scale byte.  Implements the block steps of the
// method: block max, candidate scales, E2M1 rounding, reconstruction error,
// selection ("Technical summary: Four Over Six (4/6)", "Adaptive block
// scaling algorithm"), with the error of each half summed sequentially and
// the two halves then added.
template <bool k46, bool kMae, bool kNeedErr>
__device__ __forceinline__ HalfBlock quantize_half_block(const uint32_t wd[4], bool odd,
                                                         float k_mine, const float2* tab) {
  float a[8];  // |x|
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[2 * j] = fabsf(bf16_lo(wd[j]));
    a[2 * j + 1] = fabsf(bf16_hi(wd[j]));
  }
  const float m = fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])),
                        fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7])));
  const float b = fmaxf(m, pair_swap(m));

  // Block scales: each lane encodes one candidate, the pair swaps them.
  const uint32_t s_mine = e4m3_encode(b * k_mine);
  uint32_t S6 = s_mine, S4 = s_mine;
  if (k46) {
    const uint32_t s_other = pair_swap(s_mine);
    S6 = odd ? s_other : s_mine;
    S4 = odd ? s_mine : s_other;
  }
  const float2 t6 = tab[S6];  // (d, r)
  const float2 t4 = k46 ? tab[S4] : t6;

  // Both candidates in magnitude: x and its reconstruction share a sign, so
  // |xhat - x| = |RN(q * d) - |x||.
  float q6[8], q4[8];
  float h6 = 0.0f, h4 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    q6[i] = e2m1_round(a[i] * t6.y);
    if (kNeedErr) {
      const float d6 = q6[i] * t6.x - a[i];
      h6 = kMae ? h6 + fabsf(d6) : __builtin_fmaf(d6, d6, h6);
    }
    if (k46) {
      q4[i] = e2m1_round(a[i] * t4.y);
      const float d4 = q4[i] * t4.x - a[i];
      h4 = kMae ? h4 + fabsf(d4) : __builtin_fmaf(d4, d4, h4);
    }
  }
  HalfBlock r;
  float e6 = 0.0f, e4 = 0.0f;
  if (kNeedErr) e6 = h6 + pair_swap(h6);  // lo + hi: the same sum on both lanes
  if (k46) e4 = h4 + pair_swap(h4);
  r.pick4 = k46 && (e4 < e6);             // ties and NaN keep max->6
  r.err = r.pick4 ? e4 : e6;
  r.S = r.pick4 ? S4 : S6;

  uint32_t word = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = (k46 && r.pick4) ? q4[i] : q6[i];
    const uint32_t sgn = (wd[i >> 1] >> ((i & 1) ? 28 : 12)) & 8u;  // sign of x -> bit 3
    word |= (e2m1_index(q) | sgn) << (4 * i);
  }
  r.word = word;
  return r;
}

// Build the per-workgroup table tab[S] = (d, r) for the 128 scale bytes.
__device__ __forceinline__ void build_scale_table(float2* tab, const TensorScales& ts) {
  for (uint32_t S = threadIdx.x; S < 128u; S += blockDim.x) tab[S] = scale_pair(S, ts);
}

}  // namespace nvfp4
