// api.hip -- the C ABI (include/nvfp4.h): argument checks, then kernel
// launches on the caller's stream.  No allocation, no host synchronization.
#include <atomic>
#include <initializer_list>
#include <mutex>

#include "nvfp4.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace nvfp4

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

nvfp4_status hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

// Whether the byte ranges [a, a + an) and [b, b + bn) overlap.
bool overlap(const void* a, int64_t an, const void* b, int64_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)bn && y < x + (uintptr_t)an;
}

// A byte range of an argument (a null pointer or an empty range overlaps
// nothing).
struct Span {
  const void* p;
  int64_t bytes;
};

// Whether any output range overlaps an input range or another output range.
// Everything a call writes, or reads while other workgroups write (a tensor
// scale, an accumulator), counts as an output here.
bool outputs_overlap(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    if (!o->p || o->bytes <= 0) continue;
    for (const Span& i : ins)
      if (i.p && i.bytes > 0 && overlap(o->p, o->bytes, i.p, i.bytes)) return true;
    for (auto q = o + 1; q != outs.end(); ++q)
      if (q->p && q->bytes > 0 && overlap(o->p, o->bytes, q->p, q->bytes)) return true;
  }
  return false;
}

// Largest supported element count: keeps every byte offset and the bitmap
// bit index comfortably inside int64.
constexpr int64_t kMaxNumel = int64_t(1) << 46;

nvfp4_status check_shape(int64_t rows, int64_t cols, int block_axis) {
  if (rows <= 0 || cols <= 0) return NVFP4_ERR_SHAPE;
  if (rows > kMaxNumel / cols) return NVFP4_ERR_SHAPE;
  const int64_t along = block_axis == NVFP4_AXIS_COLS ? cols : rows;
  if (along % 16 != 0) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(nvfp4_status s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_ENUM: return "invalid block_axis, mode, rule, out_dtype, flags or eps";
    case NVFP4_ERR_SHAPE: return "invalid shape (extents must be positive, block axis a multiple of 16)";
    case NVFP4_ERR_ALIGN: return "misaligned pointer";
    case NVFP4_ERR_HIP: return "HIP kernel launch failed";
    case NVFP4_ERR_ALIAS: return "an output aliases an input it must not overwrite";
    case NVFP4_ERR_SCRATCH:
      return "the product needs more than the library's fixed scratch (splits * m * n > 2^23)";
  }
  return "unknown status";
}

nvfp4_status nvfp4_amax(const uint16_t* in_bf16, int64_t numel, float* amax_out, void* stream) {
  if (!in_bf16 || !amax_out) return NVFP4_ERR_NULL;
  if (numel <= 0 || numel > kMaxNumel) return NVFP4_ERR_SHAPE;
  if (!aligned(in_bf16, 16) || !aligned(amax_out, 4)) return NVFP4_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* acc = reinterpret_cast<uint32_t*>(amax_out);
  hipError_t e = nvfp4::launch_init(acc, nullptr, nullptr, 0, s);
  if (e == hipSuccess) e = nvfp4::launch_amax(in_bf16, numel, 0.0f, acc, s);
  return hip_status(e);
}

nvfp4_status nvfp4_global_scale(const float* amax, int mode, float* gscale_out, void* stream) {
  if (!amax || !gscale_out) return NVFP4_ERR_NULL;
  if (mode != NVFP4_MODE_STD && mode != NVFP4_MODE_4OVER6) return NVFP4_ERR_ENUM;
  if (!aligned(amax, 4) || !aligned(gscale_out, 4)) return NVFP4_ERR_ALIGN;
  const float six_m = mode == NVFP4_MODE_4OVER6 ? 6.0f * 256.0f : 6.0f * 448.0f;
  return hip_status(nvfp4::launch_global_scale(amax, six_m, gscale_out,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

nvfp4_status quantize_impl(const uint16_t* in_bf16, int64_t rows, int64_t cols, int block_axis,
                           int mode, int rule, uint32_t flags, uint8_t* packed_out,
                           uint8_t* scales_out, float* gscale_inout, uint8_t* selmap_out,
                           double* err_sum_out, float* amax_out, nvfp4::Events ev,
                           void* stream) {
  if (!in_bf16 || !packed_out || !scales_out || !gscale_inout) return NVFP4_ERR_NULL;
  if (block_axis != NVFP4_AXIS_ROWS && block_axis != NVFP4_AXIS_COLS) return NVFP4_ERR_ENUM;
  if (mode != NVFP4_MODE_STD && mode != NVFP4_MODE_4OVER6) return NVFP4_ERR_ENUM;
  if (rule != NVFP4_RULE_MSE && rule != NVFP4_RULE_MAE && rule != NVFP4_RULE_MAX)
    return NVFP4_ERR_ENUM;
  if (flags & ~uint32_t(NVFP4_FLAG_GSCALE_GIVEN | NVFP4_FLAG_ERR_ACCUMULATE))
    return NVFP4_ERR_ENUM;
  const nvfp4_status shape = check_shape(rows, cols, block_axis);
  if (shape != NVFP4_OK) return shape;
  if (!aligned(in_bf16, 16) || !aligned(packed_out, 4) || !aligned(gscale_inout, 4) ||
      !aligned(selmap_out, 4) || !aligned(err_sum_out, 8) || !aligned(amax_out, 4))
    return NVFP4_ERR_ALIGN;
  {
    const int64_t n = rows * cols, nb = n / 16;
    if (outputs_overlap({{packed_out, n / 2}, {scales_out, nb}, {gscale_inout, 4},
                         {selmap_out, (nb + 7) / 8}, {err_sum_out, 8}, {amax_out, 4}},
                        {{in_bf16, n * 2}}))
      return NVFP4_ERR_ALIAS;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool given = (flags & NVFP4_FLAG_GSCALE_GIVEN) != 0;
  double* err_zero = (flags & NVFP4_FLAG_ERR_ACCUMULATE) ? nullptr : err_sum_out;
  uint32_t variant = 0;
  if (mode == NVFP4_MODE_4OVER6) {
    variant |= nvfp4::kVarFourOverSix;
    if (rule == NVFP4_RULE_MAE) variant |= nvfp4::kVarMae;
    if (rule == NVFP4_RULE_MAX) variant |= nvfp4::kVarMax;
  }
  if (selmap_out) variant |= nvfp4::kVarSelmap;
  if (err_sum_out) variant |= nvfp4::kVarErr;

  hipError_t e = hipSuccess;
  uint32_t* acc = reinterpret_cast<uint32_t*>(gscale_inout);
  uint32_t* next = reinterpret_cast<uint32_t*>(amax_out);
  // One small kernel zeroes the scale accumulator (or the amax output) and
  // the error sum; the amax pass then leaves g itself in *gscale_inout.
  if (!given || err_zero || next)
    e = nvfp4::launch_init(given ? next : acc, err_zero, nullptr, 0, s);
  if (e == hipSuccess && !given) {
    const float six_m = mode == NVFP4_MODE_4OVER6 ? 6.0f * 256.0f : 6.0f * 448.0f;
    e = nvfp4::launch_amax(in_bf16, rows * cols, six_m, acc, s);
  }
  if (e == hipSuccess) {
    if (block_axis == NVFP4_AXIS_COLS)
      e = nvfp4::launch_quantize_rows(in_bf16, rows * cols / 16, gscale_inout, variant,
                                      packed_out, scales_out, selmap_out, err_sum_out, next, s,
                                      ev);
    else
      e = nvfp4::launch_quantize_cols(in_bf16, rows, cols, gscale_inout, variant, packed_out,
                                      scales_out, selmap_out, err_sum_out, next, nullptr, s, ev);
  }
  return hip_status(e);
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_quantize_ex(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                               int block_axis, int mode, int rule, uint32_t flags,
                               uint8_t* packed_out, uint8_t* scales_out, float* gscale_inout,
                               uint8_t* selmap_out, double* err_sum_out, void* stream) {
  return quantize_impl(in_bf16, rows, cols, block_axis, mode, rule, flags, packed_out,
                       scales_out, gscale_inout, selmap_out, err_sum_out, nullptr,
                       nvfp4::Events{}, stream);
}

nvfp4_status nvfp4_quantize_dual(const uint16_t* in_bf16, int64_t rows, int64_t cols, int mode,
                                 int rule, uint32_t flags, uint8_t* packed_r, uint8_t* scales_r,
                                 uint8_t* packed_c, uint8_t* scales_c, float* gscale_inout,
                                 uint8_t* selmap_r, uint8_t* selmap_c, double* err_sum_r,
                                 double* err_sum_c, void* stream) {
  if (!in_bf16 || !packed_r || !scales_r || !packed_c || !scales_c || !gscale_inout)
    return NVFP4_ERR_NULL;
  if ((selmap_r == nullptr) != (selmap_c == nullptr)) return NVFP4_ERR_NULL;
  if ((err_sum_r == nullptr) != (err_sum_c == nullptr)) return NVFP4_ERR_NULL;
  if (mode != NVFP4_MODE_STD && mode != NVFP4_MODE_4OVER6) return NVFP4_ERR_ENUM;
  if (rule != NVFP4_RULE_MSE && rule != NVFP4_RULE_MAE && rule != NVFP4_RULE_MAX)
    return NVFP4_ERR_ENUM;
  if (flags & ~uint32_t(NVFP4_FLAG_GSCALE_GIVEN | NVFP4_FLAG_ERR_ACCUMULATE))
    return NVFP4_ERR_ENUM;
  nvfp4_status shape = check_shape(rows, cols, NVFP4_AXIS_COLS);
  if (shape == NVFP4_OK) shape = check_shape(rows, cols, NVFP4_AXIS_ROWS);
  if (shape != NVFP4_OK) return shape;
  if (!aligned(in_bf16, 16) || !aligned(packed_r, 4) || !aligned(packed_c, 4) ||
      !aligned(gscale_inout, 4) || !aligned(selmap_r, 4) || !aligned(selmap_c, 4) ||
      !aligned(err_sum_r, 8) || !aligned(err_sum_c, 8))
    return NVFP4_ERR_ALIGN;
  {
    const int64_t n = rows * cols, nb = n / 16;
    if (outputs_overlap({{packed_r, n / 2}, {scales_r, nb}, {packed_c, n / 2}, {scales_c, nb},
                         {gscale_inout, 4}, {selmap_r, (nb + 7) / 8}, {selmap_c, (nb + 7) / 8},
                         {err_sum_r, 8}, {err_sum_c, 8}},
                        {{in_bf16, n * 2}}))
      return NVFP4_ERR_ALIAS;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool given = (flags & NVFP4_FLAG_GSCALE_GIVEN) != 0;
  const bool zero_err = err_sum_c && !(flags & NVFP4_FLAG_ERR_ACCUMULATE);
  uint32_t variant = 0;
  if (mode == NVFP4_MODE_4OVER6) {
    variant |= nvfp4::kVarFourOverSix;
    if (rule == NVFP4_RULE_MAE) variant |= nvfp4::kVarMae;
    if (rule == NVFP4_RULE_MAX) variant |= nvfp4::kVarMax;
  }
  if (selmap_c) variant |= nvfp4::kVarSelmap;
  if (err_sum_c) variant |= nvfp4::kVarErr;

  hipError_t e = hipSuccess;
  uint32_t* acc = reinterpret_cast<uint32_t*>(gscale_inout);
  // Zero the scale accumulator and both error sums (the row-blocked one as
  // two 32-bit words) in one small kernel.
  if (!given || zero_err)
    e = nvfp4::launch_init(given ? nullptr : acc, zero_err ? err_sum_c : nullptr,
                           zero_err ? reinterpret_cast<uint32_t*>(err_sum_r) : nullptr,
                           zero_err ? 2 : 0, s);
  if (e == hipSuccess && !given) {
    const float six_m = mode == NVFP4_MODE_4OVER6 ? 6.0f * 256.0f : 6.0f * 448.0f;
    e = nvfp4::launch_amax(in_bf16, rows * cols, six_m, acc, s);
  }
  if (e == hipSuccess) {
    const nvfp4::DualOut dual{packed_r, scales_r, selmap_r, err_sum_r};
    e = nvfp4::launch_quantize_cols(in_bf16, rows, cols, gscale_inout, variant, packed_c, scales_c,
                                    selmap_c, err_sum_c, nullptr, &dual, s, nvfp4::Events{});
  }
  return hip_status(e);
}

nvfp4_status nvfp4_quantize_delayed(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                                    int block_axis, int mode, int rule, uint32_t flags,
                                    uint8_t* packed_out, uint8_t* scales_out,
                                    const float* gscale_in, float* amax_out,
                                    uint8_t* selmap_out, double* err_sum_out, void* stream) {
  if (!gscale_in || !amax_out) return NVFP4_ERR_NULL;
  if (flags & ~uint32_t(NVFP4_FLAG_ERR_ACCUMULATE)) {
    if (!in_bf16 || !packed_out || !scales_out) return NVFP4_ERR_NULL;
    return NVFP4_ERR_ENUM;
  }
  // g is only read (NVFP4_FLAG_GSCALE_GIVEN); the kernels take it as const.
  return quantize_impl(in_bf16, rows, cols, block_axis, mode, rule,
                       flags | NVFP4_FLAG_GSCALE_GIVEN, packed_out, scales_out,
                       const_cast<float*>(gscale_in), selmap_out, err_sum_out, amax_out,
                       nvfp4::Events{}, stream);
}

nvfp4_status nvfp4_quantize_ex_timed(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                                     int block_axis, int mode, int rule, uint32_t flags,
                                     uint8_t* packed_out, uint8_t* scales_out,
                                     float* gscale_inout, uint8_t* selmap_out,
                                     double* err_sum_out, void* start_event, void* stop_event,
                                     void* stream) {
  return quantize_impl(in_bf16, rows, cols, block_axis, mode, rule, flags, packed_out,
                       scales_out, gscale_inout, selmap_out, err_sum_out, nullptr,
                       nvfp4::Events{static_cast<hipEvent_t>(start_event),
                                     static_cast<hipEvent_t>(stop_event)},
                       stream);
}

nvfp4_status nvfp4_quantize(const uint16_t* in_bf16, int64_t rows, int64_t cols, int block_axis,
                            int mode, int rule, uint8_t* packed_out, uint8_t* scales_out,
                            float* gscale_out, void* stream) {
  return nvfp4_quantize_ex(in_bf16, rows, cols, block_axis, mode, rule, 0u, packed_out,
                           scales_out, gscale_out, nullptr, nullptr, stream);
}

nvfp4_status nvfp4_dequantize(const uint8_t* packed, const uint8_t* scales, const float* gscale,
                              int64_t rows, int64_t cols, int block_axis, int out_dtype,
                              void* out, void* stream) {
  if (!packed || !scales || !gscale || !out) return NVFP4_ERR_NULL;
  if (block_axis != NVFP4_AXIS_ROWS && block_axis != NVFP4_AXIS_COLS) return NVFP4_ERR_ENUM;
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_ENUM;
  const nvfp4_status shape = check_shape(rows, cols, block_axis);
  if (shape != NVFP4_OK) return shape;
  if (!aligned(packed, 4) || !aligned(gscale, 4) || !aligned(out, 16)) return NVFP4_ERR_ALIGN;
  {
    const int64_t n = rows * cols;
    const int64_t esz = out_dtype == NVFP4_OUT_BF16 ? 2 : 4;
    if (outputs_overlap({{out, n * esz}}, {{packed, n / 2}, {scales, n / 16}, {gscale, 4}}))
      return NVFP4_ERR_ALIAS;
  }
  return hip_status(nvfp4::launch_dequantize(packed, scales, gscale, rows, cols, block_axis,
                                             out_dtype == NVFP4_OUT_BF16, out,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"

extern "C" {

nvfp4_status nvfp4_check_order(const int32_t* perm, int64_t cols, uint32_t* bad_out,
                               void* stream) {
  if (!perm || !bad_out) return NVFP4_ERR_NULL;
  if (cols <= 0 || cols > nvfp4::kResidualMaxCols) return NVFP4_ERR_SHAPE;
  if (!aligned(perm, 4) || !aligned(bad_out, 4)) return NVFP4_ERR_ALIGN;
  if (overlap(bad_out, 4, perm, cols * 4)) return NVFP4_ERR_ALIAS;
  return hip_status(nvfp4::launch_check_order(perm, cols, bad_out,
                                              static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_channel_order(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                                 uint32_t flags, float* absmax_inout, int32_t* perm_out,
                                 void* stream) {
  if (!in_bf16 || !absmax_inout || !perm_out) return NVFP4_ERR_NULL;
  if (flags & ~uint32_t(NVFP4_FLAG_STATS_ACCUMULATE)) return NVFP4_ERR_ENUM;
  const nvfp4_status shape = check_shape(rows, cols, NVFP4_AXIS_COLS);
  if (shape != NVFP4_OK) return shape;
  if (cols > nvfp4::kResidualMaxCols) return NVFP4_ERR_SHAPE;
  if (!aligned(in_bf16, 16) || !aligned(absmax_inout, 4) || !aligned(perm_out, 4))
    return NVFP4_ERR_ALIGN;
  const int64_t in_bytes = rows * cols * 2, vec_bytes = cols * 4;
  if (overlap(absmax_inout, vec_bytes, in_bf16, in_bytes) ||
      overlap(perm_out, vec_bytes, in_bf16, in_bytes) ||
      overlap(perm_out, vec_bytes, absmax_inout, vec_bytes))
    return NVFP4_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* bits = reinterpret_cast<uint32_t*>(absmax_inout);
  hipError_t e = hipSuccess;
  if (!(flags & NVFP4_FLAG_STATS_ACCUMULATE))
    e = nvfp4::launch_init(nullptr, nullptr, bits, cols, s);
  if (e == hipSuccess) e = nvfp4::launch_channel_absmax(in_bf16, rows, cols, bits, s);
  if (e == hipSuccess) e = nvfp4::launch_channel_rank(bits, cols, perm_out, s);
  return hip_status(e);
}

nvfp4_status nvfp4_quantize_residual(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                                     const int32_t* perm, int64_t nres, int mode, int rule,
                                     uint32_t flags, uint8_t* packed_out, uint8_t* scales_out,
                                     float* gscale_inout, void* stream) {
  if (!in_bf16 || !perm || !packed_out || !scales_out || !gscale_inout) return NVFP4_ERR_NULL;
  if (mode != NVFP4_MODE_STD && mode != NVFP4_MODE_4OVER6) return NVFP4_ERR_ENUM;
  if (rule != NVFP4_RULE_MSE && rule != NVFP4_RULE_MAE && rule != NVFP4_RULE_MAX)
    return NVFP4_ERR_ENUM;
  if (flags & ~uint32_t(NVFP4_FLAG_GSCALE_GIVEN | NVFP4_FLAG_RESIDUAL_DUPLICATE))
    return NVFP4_ERR_ENUM;
  const nvfp4_status shape = check_shape(rows, cols, NVFP4_AXIS_COLS);
  if (shape != NVFP4_OK) return shape;
  if (cols > nvfp4::kResidualMaxCols || nres < 0 || nres > cols || nres % 16 != 0)
    return NVFP4_ERR_SHAPE;
  if (!aligned(in_bf16, 16) || !aligned(perm, 4) || !aligned(packed_out, 4) ||
      !aligned(gscale_inout, 4))
    return NVFP4_ERR_ALIGN;
  const int64_t in_bytes = rows * cols * 2, width = cols + nres;
  const int64_t p_bytes = rows * width / 2, s_bytes = rows * width / 16;
  const void* outs[3] = {packed_out, scales_out, gscale_inout};
  const int64_t out_bytes[3] = {p_bytes, s_bytes, 4};
  for (int k = 0; k < 3; ++k) {
    if (overlap(outs[k], out_bytes[k], in_bf16, in_bytes) ||
        overlap(outs[k], out_bytes[k], perm, cols * 4))
      return NVFP4_ERR_ALIAS;
    for (int m = k + 1; m < 3; ++m)
      if (overlap(outs[k], out_bytes[k], outs[m], out_bytes[m])) return NVFP4_ERR_ALIAS;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t variant = 0;
  if (mode == NVFP4_MODE_4OVER6) {
    variant |= nvfp4::kVarFourOverSix;
    if (rule == NVFP4_RULE_MAE) variant |= nvfp4::kVarMae;
    if (rule == NVFP4_RULE_MAX) variant |= nvfp4::kVarMax;
  }
  hipError_t e = hipSuccess;
  if (!(flags & NVFP4_FLAG_GSCALE_GIVEN)) {
    uint32_t* acc = reinterpret_cast<uint32_t*>(gscale_inout);
    const float six_m = mode == NVFP4_MODE_4OVER6 ? 6.0f * 256.0f : 6.0f * 448.0f;
    e = nvfp4::launch_init(acc, nullptr, nullptr, 0, s);
    if (e == hipSuccess) e = nvfp4::launch_amax(in_bf16, rows * cols, six_m, acc, s);
  }
  if (e == hipSuccess)
    e = nvfp4::launch_quantize_residual(in_bf16, rows, cols, perm, nres, gscale_inout, variant,
                                        packed_out, scales_out,
                                        (flags & NVFP4_FLAG_RESIDUAL_DUPLICATE) != 0, s);
  return hip_status(e);
}

}  // extern "C"

extern "C" {

nvfp4_status nvfp4_rmsnorm_quantize_residual(const uint16_t* in_bf16, int64_t rows, int64_t cols,
                                             const uint16_t* weight_bf16, float eps,
                                             const int32_t* perm, int64_t nres, int mode,
                                             int rule, uint32_t flags, uint8_t* packed_out,
                                             uint8_t* scales_out, float* gscale_inout,
                                             float* amax_out, void* stream) {
  if (!in_bf16 || !perm || !packed_out || !scales_out || !gscale_inout) return NVFP4_ERR_NULL;
  if (mode != NVFP4_MODE_STD && mode != NVFP4_MODE_4OVER6) return NVFP4_ERR_ENUM;
  if (rule != NVFP4_RULE_MSE && rule != NVFP4_RULE_MAE && rule != NVFP4_RULE_MAX)
    return NVFP4_ERR_ENUM;
  if (flags & ~uint32_t(NVFP4_FLAG_GSCALE_GIVEN)) return NVFP4_ERR_ENUM;
  if (!(eps >= 0.0f && eps <= 3.0e38f)) return NVFP4_ERR_ENUM;  // finite, non-negative
  const nvfp4_status shape = check_shape(rows, cols, NVFP4_AXIS_COLS);
  if (shape != NVFP4_OK) return shape;
  if (cols > nvfp4::kRmsWideMaxCols || nres < 0 || nres > cols || nres % 16 != 0)
    return NVFP4_ERR_SHAPE;
  if (!aligned(in_bf16, 16) || !aligned(weight_bf16, 16) || !aligned(perm, 4) ||
      !aligned(packed_out, 4) || !aligned(gscale_inout, 4) || !aligned(amax_out, 4))
    return NVFP4_ERR_ALIGN;
  const int64_t in_bytes = rows * cols * 2, width = cols + nres;
  const void* outs[4] = {packed_out, scales_out, gscale_inout, amax_out};
  const int64_t out_bytes[4] = {rows * width / 2, rows * width / 16, 4, amax_out ? 4 : 0};
  for (int k = 0; k < 4; ++k) {
    if (overlap(outs[k], out_bytes[k], in_bf16, in_bytes) ||
        overlap(outs[k], out_bytes[k], perm, cols * 4) ||
        (weight_bf16 && overlap(outs[k], out_bytes[k], weight_bf16, cols * 2)))
      return NVFP4_ERR_ALIAS;
    for (int m = k + 1; m < 4; ++m)
      if (overlap(outs[k], out_bytes[k], outs[m], out_bytes[m])) return NVFP4_ERR_ALIAS;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t variant = 0;
  if (mode == NVFP4_MODE_4OVER6) {
    variant |= nvfp4::kVarFourOverSix;
    if (rule == NVFP4_RULE_MAE) variant |= nvfp4::kVarMae;
    if (rule == NVFP4_RULE_MAX) variant |= nvfp4::kVarMax;
  }
  const bool given = (flags & NVFP4_FLAG_GSCALE_GIVEN) != 0;
  uint32_t* acc = reinterpret_cast<uint32_t*>(gscale_inout);
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(amax_out);
  const nvfp4::RmsArgs ra{weight_bf16, eps, amax_bits};
  hipError_t e = hipSuccess;
  // One small kernel zeroes the scale accumulator (when g is computed) and
  // the amax output (when asked for).
  if (!given)
    e = nvfp4::launch_init(acc, nullptr, amax_bits, amax_bits ? 1 : 0, s);
  else if (amax_bits)
    e = nvfp4::launch_init(amax_bits, nullptr, nullptr, 0, s);
  if (e == hipSuccess && !given) {
    const float six_m = mode == NVFP4_MODE_4OVER6 ? 6.0f * 256.0f : 6.0f * 448.0f;
    e = nvfp4::launch_rms_amax(in_bf16, rows, cols, ra, six_m, acc, s);
  }
  if (e == hipSuccess)
    e = nvfp4::launch_rms_quantize_residual(in_bf16, rows, cols, perm, nres, gscale_inout,
                                            variant, packed_out, scales_out, ra, s);
  return hip_status(e);
}

}  // extern "C"

extern "C" {

static bool gemm_shape_ok(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 16 != 0 || k > (int64_t(1) << 24)) return false;
  if (n > (int64_t(1) << 24)) return false;
  return !(m > kMaxNumel / n || m > kMaxNumel / k || n > kMaxNumel / k);
}

nvfp4_status nvfp4_gemm(const uint8_t* a_packed, const uint8_t* a_scales, const float* a_gscale,
                        const uint8_t* b_packed, const uint8_t* b_scales, const float* b_gscale,
                        int64_t m, int64_t n, int64_t k, int out_dtype, void* out,
                        void* stream) {
  if (!a_packed || !a_scales || !a_gscale || !b_packed || !b_scales || !b_gscale || !out)
    return NVFP4_ERR_NULL;
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_ENUM;
  if (!gemm_shape_ok(m, n, k)) return NVFP4_ERR_SHAPE;
  const int64_t esz = out_dtype == NVFP4_OUT_BF16 ? 2 : 4;
  if (!aligned(a_packed, 4) || !aligned(b_packed, 4) || !aligned(a_gscale, 4) ||
      !aligned(b_gscale, 4) || !aligned(out, (uintptr_t)esz))
    return NVFP4_ERR_ALIGN;
  const int64_t out_bytes = m * n * esz;
  const void* ins[6] = {a_packed, a_scales, a_gscale, b_packed, b_scales, b_gscale};
  const int64_t in_bytes[6] = {m * k / 2, m * k / 16, 4, n * k / 2, n * k / 16, 4};
  for (int i = 0; i < 6; ++i)
    if (overlap(out, out_bytes, ins[i], in_bytes[i])) return NVFP4_ERR_ALIAS;
  return hip_status(nvfp4::launch_gemm(a_packed, a_scales, a_gscale, b_packed, b_scales,
                                       b_gscale, m, n, k, out_dtype == NVFP4_OUT_BF16, out,
                                       static_cast<hipStream_t>(stream), nvfp4::Events{}));
}

}  // extern "C"

namespace {

// Checks of nvfp4_gemm_splitk, in the header's order: null pointers, enums,
// shape, alignment, aliasing.  With workspace == nullptr and
// caller_workspace false (the allocation-free variant, whose scratch is the
// library's own) the workspace checks are skipped.
nvfp4_status check_gemm_splitk(const uint8_t* a_packed, const uint8_t* a_scales,
                               const float* a_gscale, const uint8_t* b_packed,
                               const uint8_t* b_scales, const float* b_gscale, int64_t m,
                               int64_t n, int64_t k, int splits, int out_dtype, void* out,
                               const float* workspace, int64_t workspace_floats,
                               bool caller_workspace) {
  if (!a_packed || !a_scales || !a_gscale || !b_packed || !b_scales || !b_gscale || !out ||
      (caller_workspace && !workspace))
    return NVFP4_ERR_NULL;
  if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16) return NVFP4_ERR_ENUM;
  if (!gemm_shape_ok(m, n, k)) return NVFP4_ERR_SHAPE;
  const int64_t nchunks = (k + 127) / 128;
  if (splits < 1 || splits > nvfp4::kGemmMaxSplits || splits > nchunks) return NVFP4_ERR_SHAPE;
  const int64_t ws_floats = (int64_t)splits * m * n;
  if (caller_workspace && workspace_floats < ws_floats) return NVFP4_ERR_SHAPE;
  const int64_t esz = out_dtype == NVFP4_OUT_BF16 ? 2 : 4;
  if (!aligned(a_packed, 4) || !aligned(b_packed, 4) || !aligned(a_gscale, 4) ||
      !aligned(b_gscale, 4) || !aligned(out, (uintptr_t)esz) ||
      (caller_workspace && !aligned(workspace, 4)))
    return NVFP4_ERR_ALIGN;
  const int64_t out_bytes = m * n * esz;
  const void* ins[7] = {a_packed, a_scales, a_gscale, b_packed, b_scales, b_gscale, out};
  const int64_t in_bytes[7] = {m * k / 2, m * k / 16, 4, n * k / 2, n * k / 16, 4, out_bytes};
  for (int i = 0; i < 7; ++i) {
    if (i < 6 && overlap(out, out_bytes, ins[i], in_bytes[i])) return NVFP4_ERR_ALIAS;
    if (caller_workspace && overlap(workspace, ws_floats * 4, ins[i], in_bytes[i]))
      return NVFP4_ERR_ALIAS;
  }
  return NVFP4_OK;
}

// Fixed scratch of nvfp4_gemm_splitk_noalloc: the per-range fp32 sums of
// one product, at most kScratchFloats of them (32 MiB), held by every device
// the library runs on until the process ends.  In host code `scratch` only
// names the variable; its device address (one per device) comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr int64_t kScratchFloats = int64_t(8) << 20;
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call for that device).
nvfp4_status scratch_on_current_device(float** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NVFP4_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return NVFP4_OK;
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_gemm_splitk(const uint8_t* a_packed, const uint8_t* a_scales,
                               const float* a_gscale, const uint8_t* b_packed,
                               const uint8_t* b_scales, const float* b_gscale, int64_t m,
                               int64_t n, int64_t k, int splits, int out_dtype, void* out,
                               float* workspace, int64_t workspace_floats, void* stream) {
  const nvfp4_status st =
      check_gemm_splitk(a_packed, a_scales, a_gscale, b_packed, b_scales, b_gscale, m, n, k,
                        splits, out_dtype, out, workspace, workspace_floats, true);
  if (st != NVFP4_OK) return st;
  return hip_status(nvfp4::launch_gemm_splitk(a_packed, a_scales, a_gscale, b_packed, b_scales,
                                              b_gscale, m, n, k, (uint32_t)splits,
                                              out_dtype == NVFP4_OUT_BF16, out, workspace,
                                              static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_gemm_splitk_noalloc(const uint8_t* a_packed, const uint8_t* a_scales,
                                       const float* a_gscale, const uint8_t* b_packed,
                                       const uint8_t* b_scales, const float* b_gscale, int64_t m,
                                       int64_t n, int64_t k, int splits, int out_dtype,
                                       void* out, void* stream) {
  // The checks of nvfp4_gemm_splitk without the workspace ones (the
  // library's scratch cannot overlap caller memory), then the size limit,
  // all before any HIP call.
  nvfp4_status st =
      check_gemm_splitk(a_packed, a_scales, a_gscale, b_packed, b_scales, b_gscale, m, n, k,
                        splits, out_dtype, out, nullptr, 0, false);
  if (st != NVFP4_OK) return st;
  if ((int64_t)splits * m * n > kScratchFloats) return NVFP4_ERR_SCRATCH;
  float* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != NVFP4_OK) return st;
  return hip_status(nvfp4::launch_gemm_splitk(a_packed, a_scales, a_gscale, b_packed, b_scales,
                                              b_gscale, m, n, k, (uint32_t)splits,
                                              out_dtype == NVFP4_OUT_BF16, out, ws,
                                              static_cast<hipStream_t>(stream)));
}

int nvfp4_gemm_splits_hint(int64_t m, int64_t n, int64_t k) {
  if (!gemm_shape_ok(m, n, k)) return 0;
  return nvfp4::gemm_splits_hint(m, n, k);
}

}  // extern "C"
