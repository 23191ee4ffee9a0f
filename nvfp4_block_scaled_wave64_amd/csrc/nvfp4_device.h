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

#include <type_traits>

namespace nvfp4 {

constexpr float kFltMax = 3.40282346638528859812e+38f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Cache policy of streaming loads: non-temporal (the input is read once).
constexpr int kStreamLoad = 2;
// Cache policy of the 8-byte code stores (512 contiguous bytes per wave
// step): sc1.  Measured on MI355X for the row quantizer's mixed stream (2 B
// read, 0.5625 B written per element), sc1 code stores beat non-temporal
// ones by about 2 us of 77 (and the no-arithmetic pattern by 4 us of 70).
// The scale bytes and bitmap bytes of neighbouring chunks fill their cache
// lines piecewise, so they are written with the default policy through the
// L2, which merges them.
#ifndef NVFP4_CODE_STORE_AUX
#define NVFP4_CODE_STORE_AUX 16
#endif
#ifndef NVFP4_MERGED_STORE_AUX
#define NVFP4_MERGED_STORE_AUX 0
#endif
constexpr int kStreamStore = NVFP4_CODE_STORE_AUX;
constexpr int kMergedStore = NVFP4_MERGED_STORE_AUX;

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

// Decode multiplier dec(S) * g of a stored scale byte S (0x00..0x7E as the
// quantizers write them).  0x7F, the E4M3FN NaN code, gives NaN: the
// outlier-channel path writes it for an invalid channel order, and the
// result must not read as numbers.
__device__ __forceinline__ float block_decode_scale(uint32_t S, float g) {
  return S == 0x7Fu ? __builtin_nanf("") : e4m3_decode(S) * g;
}

// E4M3 bytes of two block scales s0, s1 (s0 in bits 0-7, s1 in bits 8-15):
// round to nearest even, saturating at 448; NaN and non-positive inputs give
// 0.  Clamping to [0, 448] first makes the gfx950 conversion
// (v_cvt_pk_fp8_f32, OCP E4M3FN, round to nearest even) exact for every
// input; the test suite checks it against the CPU reference on every fp32
// bit pattern in [0, 464] and on the saturation range.
// Bits 16-31 of the result are unspecified.
__device__ __forceinline__ uint32_t e4m3_encode2(float s0, float s1) {
  s0 = fminf(fmaxf(s0, 0.0f), 448.0f);
  s1 = fminf(fmaxf(s1, 0.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s0, s1, (int)__builtin_bit_cast(uint32_t, s0),
                                                   false);
}

// ---------------------------------------------------------------- E2M1 ----

// E2M1 codes of 8 fp32 values, element i in bits 4i..4i+3: sign in bit 3,
// magnitude rounded to nearest even on {0, 0.5, 1, 1.5, 2, 3, 4, 6},
// saturating at 6 (infinities included).  gfx950's v_cvt_scalef32_pk_fp4_f32
// with scale 1.0 does exactly this for every non-NaN input (checked against
// the CPU reference on every fp32 in [0, 8] and on sampled wider and negative
// ranges by the test suite); scaled values are never NaN here.
__device__ __forceinline__ uint32_t e2m1_encode8(const float y[8]) {
  // Each conversion writes one byte of w; all four bytes are written, so the
  // starting value does not matter.
  uint32_t w = __float_as_uint(y[0]);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// Values of 8 E2M1 codes (exact; code 8 decodes to -0).
__device__ __forceinline__ void e2m1_decode8(uint32_t w, float v[8]) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
  v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
}

// Packed maximum of two pairs of 16-bit unsigned values (v_pk_max_u16):
// non-negative bf16 values order like their bit patterns.
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  const ushort2_t va = __builtin_bit_cast(ushort2_t, a), vb = __builtin_bit_cast(ushort2_t, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(va, vb));
}

// max(|a|, |b|, |c|) without canonicalising the operands (gfx950
// v_maximum3_f32); the inputs are never NaN.
__device__ __forceinline__ float absmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(fabsf(a), fabsf(b)),
                                       fabsf(c));
}

// Buffer resource over `bytes` bytes at p (raw, stride 0): loads past the end
// return 0 and stores past the end are dropped, so tails need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// p, which the caller knows to be the same in every lane of the wave, made
// visibly uniform to the compiler (two readfirstlane): a buffer resource
// built from it then stays in scalar registers, where the compiler could
// otherwise wrap every access in a loop over distinct lane values.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
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
// r = min(G * T[S], FLT_MAX) of block scale S, with T[S] = RN(1/dec(S)) by
// IEEE division (round to nearest even) for the finite scales S = 1..126
// and T = 0 otherwise (S = 0 gives r = 0).
__device__ __forceinline__ float2 scale_pair(uint32_t S, const TensorScales& t) {
  const float dec = e4m3_decode(S);
  float2 dr;
  dr.x = dec * t.g;
  dr.y = (S - 1u) < 126u ? fminf(t.G * (1.0f / dec), kFltMax) : 0.0f;
  return dr;
}

}  // namespace nvfp4

namespace nvfp4 {

// Result of one whole block of 16 elements held by one lane.
struct Block16 {
  uint32_t lo, hi;  // codes of elements 0-7 and 8-15 (element i in bits 4i..)
  float b;          // block max |x|
  uint32_t S;       // kept E4M3 scale byte
  bool pick4;       // the max->4 candidate was kept
  float err;        // kept candidate's block error
};

// Error measure of a candidate (the method's three selection rules:
// "Technical summary: Four Over Six (4/6)", "Adaptive block scaling
// algorithm").
enum : int { kRuleMse = 0, kRuleMae = 1, kRuleMax = 2 };

// Error of one candidate over 8 elements (x) given its codes (w) and decode
// multiplier d: sequential sum of squared (or absolute) differences, or
// their maximum, between the candidate's reconstruction v * d and x, each
// difference evaluated exactly and rounded once (fused multiply-add).
template <int kRule>
__device__ __forceinline__ float half_error(const float* x, uint32_t w, float d) {
  float v[8];
  e2m1_decode8(w, v);
  float h = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float dl = __builtin_fmaf(v[i], d, -x[i]);
    if (kRule == kRuleMax)
      h = __builtin_elementwise_maximum(h, fabsf(dl));
    else if (kRule == kRuleMae)
      h = h + fabsf(dl);
    else
      h = __builtin_fmaf(dl, dl, h);
  }
  return h;
}

// Block error from the two halves: their sum, or the larger for the
// maximum-error rule.
template <int kRule>
__device__ __forceinline__ float block_error(float lo, float hi) {
  return kRule == kRuleMax ? __builtin_elementwise_maximum(lo, hi) : lo + hi;
}

// One block of 16 fp32 values x[0..15] in one lane.  Implements the block
// steps of the method -- block max, the candidate scales, E2M1 codes,
// reconstruction error against the original values, selection ("Technical
// summary: Four Over Six (4/6)", "Adaptive block scaling algorithm") -- with
// each candidate's error summed over elements 0-7 and 8-15 sequentially and
// the two partial sums then added (or, for the maximum-error rule, the
// largest single difference).
//   `scales(S)` gives the (d, r) pair of scale byte S.
//   `mid()` (optional) runs right after both pairs are requested, before
//   they are used: a caller's slot for independent work, e.g. issuing the
//   next block's LDS reads behind the table reads.
struct NoMid {
  __device__ void operator()() const {}
};
template <bool k46, int kRule, bool kNeedErr, typename Scales, typename Mid = NoMid>
__device__ __forceinline__ Block16 quantize_block16_with(const float x[16], float k6, float k4,
                                                         const Scales& scales,
                                                         const Mid& mid = Mid{}) {
  constexpr bool kMid = !std::is_same<Mid, NoMid>::value;
  const float b = __builtin_elementwise_maximum(
      absmax3(absmax3(x[0], x[1], x[2]), absmax3(x[3], x[4], x[5]), absmax3(x[6], x[7], x[8])),
      absmax3(absmax3(x[9], x[10], x[11]), absmax3(x[12], x[13], x[14]), x[15]));

  const uint32_t S2 = e4m3_encode2(b * k6, k46 ? b * k4 : 0.0f);
  const uint32_t S6 = S2 & 0xFFu, S4 = (S2 >> 8) & 0xFFu;
  const float2 t6 = scales(S6);  // (d, r)
  float2 t4 = {0.0f, 0.0f};
  if constexpr (kMid) {
    if (k46) t4 = scales(S4);
    mid();
  }

  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[i] * t6.y;
  const uint32_t c6lo = e2m1_encode8(y);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[8 + i] * t6.y;
  const uint32_t c6hi = e2m1_encode8(y);
  float e6 = 0.0f;
  if (kNeedErr)
    e6 = block_error<kRule>(half_error<kRule>(x, c6lo, t6.x), half_error<kRule>(x + 8, c6hi, t6.x));

  Block16 r;
  r.b = b;
  r.lo = c6lo;
  r.hi = c6hi;
  r.S = S6;
  r.pick4 = false;
  r.err = e6;
  if (k46) {
    if constexpr (!kMid) t4 = scales(S4);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] * t4.y;
    const uint32_t c4lo = e2m1_encode8(y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[8 + i] * t4.y;
    const uint32_t c4hi = e2m1_encode8(y);
    const float e4 =
        block_error<kRule>(half_error<kRule>(x, c4lo, t4.x), half_error<kRule>(x + 8, c4hi, t4.x));
    r.pick4 = e4 < e6;  // ties and NaN keep max->6
    r.lo = r.pick4 ? c4lo : c6lo;
    r.hi = r.pick4 ? c4hi : c6hi;
    r.S = r.pick4 ? S4 : S6;
    r.err = r.pick4 ? e4 : e6;
  }
  return r;
}

// The same with the (d, r) pairs read from a table tab[S] (LDS).
template <bool k46, int kRule, bool kNeedErr, typename Mid = NoMid>
__device__ __forceinline__ Block16 quantize_block16f(const float x[16], float k6, float k4,
                                                     const float2* tab, const Mid& mid = Mid{}) {
  return quantize_block16_with<k46, kRule, kNeedErr>(
      x, k6, k4, [tab](uint32_t S) { return tab[S]; }, mid);
}

// The same for a block of 16 bf16 values: wd[0..7] hold them in pairs
// (element 2j in the low half of wd[j]).
template <bool k46, int kRule, bool kNeedErr>
__device__ __forceinline__ Block16 quantize_block16(const uint32_t wd[8], float k6, float k4,
                                                    const float2* tab) {
  float x[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[2 * j] = bf16_lo(wd[j]);
    x[2 * j + 1] = bf16_hi(wd[j]);
  }
  return quantize_block16f<k46, kRule, kNeedErr>(x, k6, k4, tab);
}

// Folds each lane's running maximum m (a non-negative float) into
// *amax_out: wave reduction on the bit patterns (non-negative floats order
// like their bits), one LDS slot per wave, one atomic per workgroup.  Every
// thread of the workgroup must call it (it contains a barrier).
template <int kWaves>
__device__ __forceinline__ void group_max_to(uint32_t* amax_out, float m, uint32_t* part) {
  uint32_t v = __float_as_uint(m);
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  if ((threadIdx.x & 63u) == 0u) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = part[0];
    for (int k = 1; k < kWaves; ++k) r = max(r, part[k]);
    atomicMax(amax_out, r);
  }
}

// Build the per-workgroup table tab[S] = (d, r) for the 128 scale bytes.
__device__ __forceinline__ void build_scale_table(float2* tab, const TensorScales& ts) {
  for (uint32_t S = threadIdx.x; S < 128u; S += blockDim.x) tab[S] = scale_pair(S, ts);
}

}  // namespace nvfp4
