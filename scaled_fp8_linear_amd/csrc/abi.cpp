// C ABI of the scaled FP8 linear layer: argument checking and dispatch.
// The declarations, with the meaning of every argument, are in include/fp8lin.h.
#include "../../include/fp8lin.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return FP8_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int64_t kMaxOperandBytes = (int64_t)1 << 31;
constexpr int64_t kMaxContraction = (int64_t)1 << 17;

// Checks shared by the three GEMM entry points. A is [rows_a, kc], B is [rows_b, kc].
int check_gemm(const char* fn, const void* a, const void* b, const float* s1, const float* s2,
               const void* d, int64_t rows_a, int64_t rows_b, int64_t kc, int64_t m_valid,
               int gran, bool a_e5m2) {
  if (rows_a < 0 || rows_b < 0 || kc < 0)
    return fail(FP8_ERR_SHAPE, "%s: negative size", fn);
  if (rows_a % 16 || rows_b % 16 || kc % 16)
    return fail(FP8_ERR_SHAPE,
                "%s: sizes must be multiples of 16 (got %lld x %lld x %lld); FP8 GEMMs need the "
                "token count and every dimension divisible by 16",
                fn, (long long)rows_a, (long long)rows_b, (long long)kc);
  if (m_valid < 0 || m_valid > rows_a)
    return fail(FP8_ERR_SHAPE, "%s: M_valid=%lld outside [0, %lld]", fn, (long long)m_valid,
                (long long)rows_a);
  if (gran != FP8_TENSORWISE && gran != FP8_BLOCK_1x128)
    return fail(FP8_ERR_UNSUPPORTED, "%s: granularity %d (use FP8_TENSORWISE or FP8_BLOCK_1x128)",
                fn, gran);
  if (a_e5m2 && gran != FP8_TENSORWISE)
    return fail(FP8_ERR_UNSUPPORTED, "%s: e5m2 operands (FP8_A_E5M2) are for FP8_TENSORWISE", fn);
  if (gran == FP8_BLOCK_1x128 && kc % 128)
    return fail(FP8_ERR_SHAPE, "%s: block recipe needs the contraction size %% 128 == 0 (got %lld)",
                fn, (long long)kc);
  if (rows_a * kc >= kMaxOperandBytes || rows_b * kc >= kMaxOperandBytes ||
      rows_a * rows_b * 2 >= kMaxOperandBytes)
    return fail(FP8_ERR_UNSUPPORTED, "%s: an operand or the output holds 2^31 bytes or more", fn);
  if (kc >= kMaxContraction)
    return fail(FP8_ERR_UNSUPPORTED, "%s: contraction size %lld >= 2^17", fn, (long long)kc);
  if (rows_a * rows_b > 0) {
    if (!d) return fail(FP8_ERR_NULL, "%s: NULL output", fn);
    // an empty contraction reads neither operands nor scales (the output is all zeros)
    if (kc > 0 && (!a || !b || !s1 || !s2))
      return fail(FP8_ERR_NULL, "%s: NULL operand or scale pointer", fn);
    if (!aligned16(a) || !aligned16(b) || !aligned16(d))
      return fail(FP8_ERR_ALIGN, "%s: operands and output must be 16-byte aligned", fn);
  }
  return FP8_OK;
}

}  // namespace

extern "C" {

const char* fp8_last_error(void) { return g_err; }

const char* fp8_version(void) { return "fp8lin 0.1 gfx950"; }

int fp8_quantize_amax(const void* x, int64_t rows, int64_t cols, int64_t rows_valid, int gran,
                      const float* scale_inv, void* q, void* q_t, float* amax, float* scale,
                      float* scale_t, void* stream) {
  const char* fn = "fp8_quantize_amax";
  const bool accumulate = (gran & FP8_AMAX_ACCUMULATE) != 0;
  const bool e5m2 = (gran & FP8_E5M2) != 0;
  gran &= ~(FP8_AMAX_ACCUMULATE | FP8_E5M2);
  if (accumulate && gran != FP8_TENSORWISE)
    return fail(FP8_ERR_UNSUPPORTED, "%s: FP8_AMAX_ACCUMULATE is for FP8_TENSORWISE", fn);
  if (e5m2 && gran != FP8_TENSORWISE)
    return fail(FP8_ERR_UNSUPPORTED, "%s: FP8_E5M2 codes are for FP8_TENSORWISE", fn);
  if (rows < 0 || cols < 0) return fail(FP8_ERR_SHAPE, "%s: negative size", fn);
  if (rows_valid < 0 || rows_valid > rows)
    return fail(FP8_ERR_SHAPE, "%s: rows_valid=%lld outside [0, %lld]", fn, (long long)rows_valid,
                (long long)rows);
  const int64_t mult = (gran == FP8_TENSORWISE) ? 16 : 128;
  if (rows % mult || cols % mult)
    return fail(FP8_ERR_SHAPE, "%s: rows and cols must be multiples of %lld (got %lld x %lld)", fn,
                (long long)mult, (long long)rows, (long long)cols);
  if (rows * cols > 0 && !x) return fail(FP8_ERR_NULL, "%s: x is NULL", fn);
  if (!aligned16(x) || !aligned16(q) || !aligned16(q_t))
    return fail(FP8_ERR_ALIGN, "%s: x, q and q_t must be 16-byte aligned", fn);
  const hipStream_t s = as_stream(stream);
  auto* xb = static_cast<const uint16_t*>(x);
  auto* qb = static_cast<uint8_t*>(q);
  auto* qtb = static_cast<uint8_t*>(q_t);
  switch (gran) {
    case FP8_TENSORWISE:
      if ((q || q_t) && !scale_inv) return fail(FP8_ERR_NULL, "%s: scale_inv is NULL", fn);
      if (scale || scale_t)
        return fail(FP8_ERR_UNSUPPORTED, "%s: scale/scale_t are outputs of the block modes only", fn);
      return hip_status(
          fp8lin::launch_quantize_tensorwise(xb, rows, cols, rows_valid, scale_inv, qb, qtb, amax,
                                             accumulate, e5m2, s),
          fn);
    case FP8_BLOCK_1x128:
    case FP8_BLOCK_128x128:
      if (scale_inv)
        return fail(FP8_ERR_UNSUPPORTED, "%s: block modes compute their own multipliers; pass NULL", fn);
      if ((q == nullptr) != (scale == nullptr))
        return fail(FP8_ERR_NULL, "%s: q and scale must both be given or both be NULL", fn);
      if ((q_t == nullptr) != (scale_t == nullptr))
        return fail(FP8_ERR_NULL, "%s: q_t and scale_t must both be given or both be NULL", fn);
      if (gran == FP8_BLOCK_128x128) {
        if (rows_valid != rows)
          return fail(FP8_ERR_SHAPE, "%s: 128x128 tiles (weights) take no padding rows", fn);
        return hip_status(fp8lin::launch_quantize_block_128x128(xb, rows, cols, qb, qtb, amax,
                                                                scale, scale_t, s),
                          fn);
      }
      return hip_status(fp8lin::launch_quantize_block_1x128(xb, rows, cols, rows_valid, qb, qtb,
                                                            amax, scale, scale_t, s),
                        fn);
    default:
      return fail(FP8_ERR_UNSUPPORTED, "%s: unknown granularity %d", fn, gran);
  }
}

int fp8_scale_update(int mode, float* amax, float* hist, int32_t len, int32_t pos,
                     float* scale, float* scale_inv, void* stream) {
  const char* fn = "fp8_scale_update";
  const bool clear = (mode & FP8_SCALE_CLEAR_AMAX) != 0;
  const bool e5m2 = (mode & FP8_E5M2) != 0;
  mode &= ~(FP8_SCALE_CLEAR_AMAX | FP8_E5M2);
  if (clear && mode != FP8_SCALE_FROM_AMAX && mode != FP8_SCALE_RECORD)
    return fail(FP8_ERR_UNSUPPORTED, "%s: FP8_SCALE_CLEAR_AMAX needs a mode that reads amax", fn);
  if (e5m2 && mode != FP8_SCALE_FROM_AMAX && mode != FP8_SCALE_REFRESH)
    return fail(FP8_ERR_UNSUPPORTED, "%s: FP8_E5M2 goes with a mode that writes scales", fn);
  switch (mode) {
    case FP8_SCALE_FROM_AMAX:
      if (!amax || !scale || !scale_inv) return fail(FP8_ERR_NULL, "%s: NULL pointer", fn);
      break;
    case FP8_SCALE_RECORD:
      if (!amax || !hist) return fail(FP8_ERR_NULL, "%s: NULL pointer", fn);
      if (len < 1 || pos < 0 || pos >= len)
        return fail(FP8_ERR_SHAPE, "%s: pos=%d outside a ring of %d", fn, pos, len);
      break;
    case FP8_SCALE_REFRESH:
      if (!hist || !scale || !scale_inv) return fail(FP8_ERR_NULL, "%s: NULL pointer", fn);
      if (len < 1) return fail(FP8_ERR_SHAPE, "%s: empty history", fn);
      break;
    default:
      return fail(FP8_ERR_UNSUPPORTED, "%s: unknown mode %d", fn, mode);
  }
  return hip_status(fp8lin::launch_scale_update(mode, amax, clear, hist, len, pos, scale,
                                                scale_inv, e5m2, as_stream(stream)),
                    fn);
}

int fp8_linear_fwd(const void* qx, const void* qw, const float* sx, const float* sw, void* y,
                   int64_t M, int64_t N, int64_t K, int64_t M_valid, int gran, void* stream) {
  const bool a5 = (gran & FP8_A_E5M2) != 0;
  gran &= ~FP8_A_E5M2;
  int e = check_gemm("fp8_linear_fwd", qx, qw, sx, sw, y, M, N, K, M_valid, gran, a5);
  if (e) return e;
  if (gran == FP8_BLOCK_1x128 && N % 128)
    return fail(FP8_ERR_SHAPE, "fp8_linear_fwd: block recipe needs N %% 128 == 0");
  return hip_status(fp8lin::launch_gemm_fp8(static_cast<const uint8_t*>(qx),
                                            static_cast<const uint8_t*>(qw), sx, sw, nullptr,
                                            static_cast<uint16_t*>(y), M, N, K, M_valid,
                                            gran == FP8_BLOCK_1x128, 128, a5, as_stream(stream)),
                    "fp8_linear_fwd");
}

int fp8_linear_fwd_current(const void* x, const void* w, int64_t M, int64_t N, int64_t K,
                           void* y, float* scales, void* qx, void* qw, void* stream) {
  const char* fn = "fp8_linear_fwd_current";
  if (M < 16 || N < 16 || K < 128 || M % 16 || N % 16 || K % 128)
    return fail(FP8_ERR_SHAPE,
                "%s: M and N must be positive multiples of 16 and K a positive multiple of 128 "
                "(got %lld x %lld x %lld)",
                fn, (long long)M, (long long)N, (long long)K);
  if ((M + N) * K > fp8lin::kSmallLinearCodes)
    return fail(FP8_ERR_UNSUPPORTED,
                "%s: (M + N) K = %lld bytes of codes exceed the small-linear limit of %d; use "
                "fp8_quantize_amax, fp8_scale_update and fp8_linear_fwd",
                fn, (long long)((M + N) * K), fp8lin::kSmallLinearCodes);
  if (!x || !w || !y || !scales) return fail(FP8_ERR_NULL, "%s: NULL x, w, y or scales", fn);
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || !aligned16(qx) || !aligned16(qw))
    return fail(FP8_ERR_ALIGN, "%s: x, w, y, qx and qw must be 16-byte aligned", fn);
  return hip_status(fp8lin::launch_linear_current_small(
                        static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), (int)M,
                        (int)N, (int)K, static_cast<uint16_t*>(y), scales,
                        static_cast<uint8_t*>(qx), static_cast<uint8_t*>(qw), as_stream(stream)),
                    fn);
}

int fp8_linear_fwd_bias(const void* qx, const void* qw, const float* sx, const float* sw,
                        const void* bias, void* y, int64_t M, int64_t N, int64_t K,
                        int64_t M_valid, int gran, void* stream) {
  const char* fn = "fp8_linear_fwd_bias";
  if (bias == nullptr)
    return fp8_linear_fwd(qx, qw, sx, sw, y, M, N, K, M_valid, gran, stream);
  if (gran & FP8_A_E5M2)
    return fail(FP8_ERR_UNSUPPORTED, "%s: the bias epilogue takes e4m3 operands", fn);
  int e = check_gemm(fn, qx, qw, sx, sw, y, M, N, K, M_valid, gran, false);
  if (e) return e;
  if (gran != FP8_TENSORWISE)
    return fail(FP8_ERR_UNSUPPORTED, "%s: the bias epilogue is for FP8_TENSORWISE", fn);
  if (!aligned16(bias)) return fail(FP8_ERR_ALIGN, "%s: bias must be 16-byte aligned", fn);
  return hip_status(fp8lin::launch_gemm_fp8(static_cast<const uint8_t*>(qx),
                                            static_cast<const uint8_t*>(qw), sx, sw,
                                            static_cast<const uint16_t*>(bias),
                                            static_cast<uint16_t*>(y), M, N, K, M_valid, false,
                                            128, false, as_stream(stream)),
                    fn);
}

int fp8_bias_grad(const void* g, int64_t rows, int64_t cols, int64_t rows_valid, void* db,
                  void* stream) {
  const char* fn = "fp8_bias_grad";
  if (rows < 0 || cols < 0) return fail(FP8_ERR_SHAPE, "%s: negative size", fn);
  if (cols % 16) return fail(FP8_ERR_SHAPE, "%s: cols=%lld not a multiple of 16", fn,
                             (long long)cols);
  if (rows_valid < 0 || rows_valid > rows)
    return fail(FP8_ERR_SHAPE, "%s: rows_valid=%lld outside [0, %lld]", fn,
                (long long)rows_valid, (long long)rows);
  if (cols > 0 && !db) return fail(FP8_ERR_NULL, "%s: db is NULL", fn);
  if (rows_valid > 0 && cols > 0 && !g) return fail(FP8_ERR_NULL, "%s: g is NULL", fn);
  if (!aligned16(g)) return fail(FP8_ERR_ALIGN, "%s: g must be 16-byte aligned", fn);
  if (rows * cols * 2 >= kMaxOperandBytes)
    return fail(FP8_ERR_UNSUPPORTED, "%s: g holds 2^31 bytes or more", fn);
  return hip_status(fp8lin::launch_bias_grad(static_cast<const uint16_t*>(g), rows, cols,
                                             rows_valid, static_cast<uint16_t*>(db),
                                             as_stream(stream)),
                    fn);
}

int fp8_linear_dgrad(const void* qg, const void* qw_t, const float* sg, const float* sw, void* dx,
                     int64_t M, int64_t N, int64_t K, int64_t M_valid, int gran, void* stream) {
  const bool a5 = (gran & FP8_A_E5M2) != 0;
  gran &= ~FP8_A_E5M2;
  int e = check_gemm("fp8_linear_dgrad", qg, qw_t, sg, sw, dx, M, K, N, M_valid, gran, a5);
  if (e) return e;
  if (gran == FP8_BLOCK_1x128 && K % 128)
    return fail(FP8_ERR_SHAPE, "fp8_linear_dgrad: block recipe needs K %% 128 == 0");
  return hip_status(fp8lin::launch_gemm_fp8(static_cast<const uint8_t*>(qg),
                                            static_cast<const uint8_t*>(qw_t), sg, sw, nullptr,
                                            static_cast<uint16_t*>(dx), M, K, N, M_valid,
                                            gran == FP8_BLOCK_1x128, 128, a5, as_stream(stream)),
                    "fp8_linear_dgrad");
}

int fp8_linear_wgrad(const void* qg_t, const void* qx_t, const float* sg, const float* sx, void* dw,
                     int64_t M, int64_t N, int64_t K, int gran, void* stream) {
  const bool a5 = (gran & FP8_A_E5M2) != 0;
  gran &= ~FP8_A_E5M2;
  int e = check_gemm("fp8_linear_wgrad", qg_t, qx_t, sg, sx, dw, N, K, M, N, gran, a5);
  if (e) return e;
  return hip_status(fp8lin::launch_gemm_fp8(static_cast<const uint8_t*>(qg_t),
                                            static_cast<const uint8_t*>(qx_t), sg, sx, nullptr,
                                            static_cast<uint16_t*>(dw), N, K, M, N,
                                            gran == FP8_BLOCK_1x128, 1, a5, as_stream(stream)),
                    "fp8_linear_wgrad");
}

int fp8_pad_tokens(const void* x, int64_t T, int64_t cols, int32_t multiple, void* x_pad,
                   int64_t* T_pad, void* stream) {
  const char* fn = "fp8_pad_tokens";
  if (!T_pad) return fail(FP8_ERR_NULL, "%s: T_pad is NULL", fn);
  if (T < 0 || cols < 0) return fail(FP8_ERR_SHAPE, "%s: negative size", fn);
  if (multiple < 1) return fail(FP8_ERR_SHAPE, "%s: multiple=%d must be >= 1", fn, multiple);
  const int64_t pad = ((-T) % multiple + multiple) % multiple;
  *T_pad = T + pad;
  if (!x_pad) return ok();
  if (T * cols > 0 && !x) return fail(FP8_ERR_NULL, "%s: x is NULL", fn);
  return hip_status(fp8lin::launch_pad_tokens(static_cast<const uint16_t*>(x), T, cols, *T_pad,
                                              static_cast<uint16_t*>(x_pad), as_stream(stream)),
                    fn);
}

int fp8_align_multiple(int layout, int64_t batch, int32_t tp, int32_t cp, int32_t base,
                       int32_t* seq_multiple, int32_t* total_multiple) {
  const char* fn = "fp8_align_multiple";
  if (!seq_multiple || !total_multiple) return fail(FP8_ERR_NULL, "%s: NULL output", fn);
  if (batch < 1 || tp < 1 || cp < 1 || base < 1)
    return fail(FP8_ERR_SHAPE, "%s: batch, tp, cp and base must be positive", fn);
  auto gcd = [](int64_t a, int64_t b) {
    while (b) { const int64_t t = a % b; a = b; b = t; }
    return a;
  };
  int64_t seq = 1, total = 1;
  if (layout == FP8_LAYOUT_THD) {
    seq = cp > 1 ? 2 * (int64_t)cp : 1;
    total = (int64_t)base * cp * tp;
  } else if (layout == FP8_LAYOUT_BSHD) {
    if (cp != 1)
      return fail(FP8_ERR_UNSUPPORTED, "%s: BSHD alignment covers tensor/sequence parallelism only",
                  fn);
    const int64_t bt = (int64_t)base * tp;
    const int64_t need = bt / gcd(batch, bt);
    seq = tp / gcd(tp, need) * need;                  // lcm(tp, need)
  } else {
    return fail(FP8_ERR_UNSUPPORTED, "%s: unknown layout %d", fn, layout);
  }
  if (seq > 0x7FFFFFFF || total > 0x7FFFFFFF)
    return fail(FP8_ERR_SHAPE, "%s: multiple does not fit 32 bits", fn);
  *seq_multiple = (int32_t)seq;
  *total_multiple = (int32_t)total;
  return ok();
}

namespace {

// cu: nseq + 1 non-decreasing host offsets starting at 0.
int check_offsets(const char* fn, const int64_t* cu, int32_t nseq, const char* what) {
  if (!cu) return fail(FP8_ERR_NULL, "%s: %s is NULL", fn, what);
  if (cu[0] != 0) return fail(FP8_ERR_SHAPE, "%s: %s[0] must be 0", fn, what);
  for (int32_t i = 0; i < nseq; ++i)
    if (cu[i + 1] < cu[i])
      return fail(FP8_ERR_SHAPE, "%s: %s decreases at %d", fn, what, i);
  return FP8_OK;
}

}  // namespace

int fp8_pad_varlen(const void* x, const int64_t* cu_seqlens, int32_t nseq, int64_t cols,
                   int32_t seq_multiple, int32_t total_multiple, void* x_pad,
                   int64_t* cu_seqlens_pad, int64_t* T_pad, void* stream) {
  const char* fn = "fp8_pad_varlen";
  if (!T_pad) return fail(FP8_ERR_NULL, "%s: T_pad is NULL", fn);
  if (nseq < 0 || cols < 0) return fail(FP8_ERR_SHAPE, "%s: negative size", fn);
  if (seq_multiple < 1 || total_multiple < 1)
    return fail(FP8_ERR_SHAPE, "%s: multiples must be >= 1", fn);
  if (cols % 16) return fail(FP8_ERR_SHAPE, "%s: cols=%lld not a multiple of 16", fn, (long long)cols);
  int e = check_offsets(fn, cu_seqlens, nseq, "cu_seqlens");
  if (e) return e;
  // padded offsets on the host
  int64_t end = 0;
  int64_t* pad_off = cu_seqlens_pad;
  for (int32_t i = 0; i <= nseq; ++i) {
    if (i > 0) {
      const int64_t len = cu_seqlens[i] - cu_seqlens[i - 1];
      end += len + ((-len) % seq_multiple + seq_multiple) % seq_multiple;
    }
    if (pad_off) pad_off[i] = end;
  }
  *T_pad = end + ((-end) % total_multiple + total_multiple) % total_multiple;
  if (!x_pad) return ok();
  if (!pad_off) return fail(FP8_ERR_NULL, "%s: cu_seqlens_pad is needed with x_pad", fn);
  if (*T_pad == 0 || cols == 0) return ok();                 // nothing to write
  if (x == x_pad) return fail(FP8_ERR_UNSUPPORTED, "%s: x_pad must not be x", fn);
  if (cu_seqlens[nseq] * cols > 0 && !x) return fail(FP8_ERR_NULL, "%s: x is NULL", fn);
  if (!aligned16(x) || !aligned16(x_pad))
    return fail(FP8_ERR_ALIGN, "%s: x and x_pad must be 16-byte aligned", fn);
  return hip_status(fp8lin::launch_pad_varlen(true, static_cast<const uint16_t*>(x),
                                              static_cast<uint16_t*>(x_pad), cols, cu_seqlens,
                                              pad_off, nseq, *T_pad, as_stream(stream)),
                    fn);
}

int fp8_unpad_varlen(const void* x_pad, const int64_t* cu_seqlens, const int64_t* cu_seqlens_pad,
                     int32_t nseq, int64_t cols, void* x, void* stream) {
  const char* fn = "fp8_unpad_varlen";
  if (nseq < 0 || cols < 0) return fail(FP8_ERR_SHAPE, "%s: negative size", fn);
  if (cols % 16) return fail(FP8_ERR_SHAPE, "%s: cols=%lld not a multiple of 16", fn, (long long)cols);
  int e = check_offsets(fn, cu_seqlens, nseq, "cu_seqlens");
  if (e) return e;
  e = check_offsets(fn, cu_seqlens_pad, nseq, "cu_seqlens_pad");
  if (e) return e;
  for (int32_t i = 0; i < nseq; ++i)
    if (cu_seqlens_pad[i + 1] - cu_seqlens_pad[i] < cu_seqlens[i + 1] - cu_seqlens[i])
      return fail(FP8_ERR_SHAPE, "%s: padded sequence %d is shorter than the sequence", fn, i);
  if (cu_seqlens[nseq] * cols == 0) return ok();
  if (!x || !x_pad) return fail(FP8_ERR_NULL, "%s: NULL tensor", fn);
  if (x == x_pad) return fail(FP8_ERR_UNSUPPORTED, "%s: x must not be x_pad", fn);
  if (!aligned16(x) || !aligned16(x_pad))
    return fail(FP8_ERR_ALIGN, "%s: x and x_pad must be 16-byte aligned", fn);
  return hip_status(fp8lin::launch_pad_varlen(false, static_cast<const uint16_t*>(x_pad),
                                              static_cast<uint16_t*>(x), cols, cu_seqlens,
                                              cu_seqlens_pad, nseq, cu_seqlens_pad[nseq],
                                              as_stream(stream)),
                    fn);
}

}  // extern "C"
