/*
 * fp8lin.h -- C ABI of the MI355X (gfx950) scaled FP8 linear layer.
 *
 * The layer is y = x W^T computed as a "TE-style" scaled FP8 linear:
 * operands are quantized to OCP e4m3 with per-tensor (or per-tile) float32
 * scales, multiplied on the FP8 matrix cores with float32 accumulation, and
 * the scales are folded in after accumulation. Sources, cited per function:
 *
 *   [AstrAI]    AstrAI, astrai/extension/fp8_state.py (module comment on the
 *               GEMM layout, FP8TensorMeta, FP8State.step,
 *               _update_delayed_scale, fp8_linear_forward/backward).
 *   [SpecForge] SpecForge PR 2, "Add training.fp8_linear: torchao
 *               Float8Linear with float8 all-gather", Conclusion
 *               (Constraints bullet) and Modifications.
 *   [NeMo]      NeMo PR 15754, "Add FP8 support for SALMAutomodel", review
 *               thread on BSHD/THD padding; TE's "recipe=block".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is DEVICE memory on the current HIP device, owned
 *   and allocated by the caller; the library allocates nothing and keeps no
 *   state between calls (it is safe to call from several host threads).
 * - Layouts are dense row-major. bf16 tensors are 2 bytes per element, e4m3
 *   tensors 1 byte per element (OCP E4M3: bias 7, max 448, NaN 0x7F/0xFF,
 *   no infinities), scales and amaxes are float32.
 * - `stream` is a hipStream_t passed as void*; NULL is the null stream. All
 *   work is enqueued asynchronously on it; nothing synchronizes the host.
 * - Return value: FP8_OK, or an fp8_status error code for arguments rejected
 *   on the host before anything is enqueued (then fp8_last_error() says
 *   why), or FP8_ERR_HIP if a launch failed. Faults inside kernels surface
 *   at the caller's next synchronization, as usual for HIP.
 * - Pointers must be 16-byte aligned; row counts / column counts must be
 *   multiples of 16 where stated ([SpecForge]: FP8 GEMMs need the token count
 *   and every converted dimension divisible by 16).
 * - Sizes are int64_t; every operand of a GEMM must hold fewer than 2^31
 *   bytes, and the contraction length must be below 2^17.
 */
#ifndef FP8LIN_H
#define FP8LIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8_status {
  FP8_OK = 0,
  FP8_ERR_NULL = 1,        /* a required pointer is NULL                     */
  FP8_ERR_SHAPE = 2,       /* a size is negative, not a multiple of 16, ... */
  FP8_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned              */
  FP8_ERR_UNSUPPORTED = 4, /* valid request the library does not implement  */
  FP8_ERR_HIP = 5          /* a HIP launch or runtime call failed           */
} fp8_status;

/* Scaling granularity of a quantized operand. */
typedef enum fp8_granularity {
  FP8_TENSORWISE = 0,   /* one float32 scale per tensor                        */
  FP8_BLOCK_1x128 = 1,  /* one scale per 1x128 tile along the contraction dim  */
  FP8_BLOCK_128x128 = 2 /* one scale per 128x128 tile (weights)                */
} fp8_granularity;

/* Modes of fp8_scale_update. */
typedef enum fp8_scale_mode {
  FP8_SCALE_FROM_AMAX = 0, /* scale, scale_inv from one amax (delayed or current) */
  FP8_SCALE_RECORD = 1,    /* push an amax into the weight history ring           */
  FP8_SCALE_REFRESH = 2    /* scale, scale_inv from the maximum of the ring       */
} fp8_scale_mode;

/*
 * Flags OR-ed into fp8_quantize_amax's gran / fp8_scale_update's mode. A
 * delayed-scaling step consumes each amax exactly once, so the update that
 * reads it can also clear it, and the next quantize pass can fold its max
 * into the cleared value instead of zeroing it first (one launch less per
 * quantized tensor).
 */
enum {
  FP8_AMAX_ACCUMULATE = 0x100, /* fp8_quantize_amax, TENSORWISE only: amax[0]
                                  = max(amax[0], max|x|) instead of being
                                  overwritten; amax[0] must hold a
                                  non-negative float32 (or NaN) on entry  */
  FP8_SCALE_CLEAR_AMAX = 0x100 /* fp8_scale_update, FROM_AMAX and RECORD:
                                  after amax[0] is read it is set to +0   */
};

/*
 * The hybrid format: gradients coded in OCP E5M2 (sign, 5 exponent bits with
 * bias 15, 2 mantissa bits; largest finite value 57344 = 0x7B; 0x7C is
 * infinity and 0x7D..0x7F NaN), activations and weights in E4M3. E5M2 trades
 * one mantissa bit for a range of 2^-16 .. 57344. The pages name E4M3 only;
 * this is the e5m2 gradient variant the same TE-style design allows, run on
 * gfx950's mixed-format FP8 matrix instructions.
 */
enum {
  FP8_E5M2 = 0x200,   /* fp8_quantize_amax (TENSORWISE): emit E5M2 codes, scale_inv
                         being 57344/amax; fp8_scale_update (FROM_AMAX, REFRESH):
                         the format maximum is 57344 instead of 448            */
  FP8_A_E5M2 = 0x200  /* fp8_linear_fwd/dgrad/wgrad (TENSORWISE, no bias): the
                         FIRST operand (x, g or g^T) holds E5M2 codes; the second
                         stays E4M3                                            */
};

/*
 * fp8_quantize_amax -- fused bf16 -> e4m3 quantize with its amax, emitting
 * the row-major codes and their transpose in one pass over x.
 *
 * Source: [AstrAI] module comment ("D = A_SCALE * B_SCALE * A * B", scales
 * amax/448, quantization multiplies by 1/scale) and fp8_linear_forward's
 * docstring (the quantize kernel emits the current amax; no separate
 * abs/max reduce).
 *
 *   x          bf16 [rows, cols], read-only.
 *   rows, cols >= 0, both multiples of 16 (multiples of 128 in BLOCK modes).
 *   rows_valid 0 <= rows_valid <= rows. Rows r >= rows_valid are token
 *              padding: they are NOT read (they may hold anything), they do
 *              not enter amax, and their codes are written as 0x00.
 *   gran       FP8_TENSORWISE, FP8_BLOCK_1x128 or FP8_BLOCK_128x128.
 *
 * FP8_TENSORWISE:
 *   scale_inv  float32 [1]: the multiplier 448/amax of the scale in force.
 *              Required when q or q_t is non-NULL.
 *   q          e4m3 [rows, cols] or NULL:  q[r,c] = e4m3(float32(x[r,c]) * *scale_inv),
 *              one float32 multiply rounded to nearest even, then round to
 *              nearest even on the e4m3 grid, saturating to +-448; NaN stays
 *              NaN (0x7F with its sign); -0 and negative underflow give 0x80.
 *   q_t        e4m3 [cols, rows] or NULL: q_t[c,r] = q[r,c].
 *   amax       float32 [1] or NULL: OVERWRITTEN with max |x[r,c]| over the
 *              valid rows (exact; 0 for empty input; NaN if a valid element is
 *              NaN). Computed on the same pass. With FP8_AMAX_ACCUMULATE in
 *              gran it becomes max(amax[0], that maximum) instead.
 *   scale, scale_t  must be NULL.
 *   With FP8_E5M2 in gran the codes are OCP E5M2 instead: the same float32
 *   product, round to nearest even on the E5M2 grid (subnormals down to
 *   2^-16 kept), saturating to +-57344 (also for +-inf); a NaN product gives
 *   0x7F with its input's sign.
 *
 * FP8_BLOCK_1x128 (activations, gradients; current per-tile scaling):
 *   scale_inv  must be NULL (each tile's multiplier is computed in the pass
 *              as 448/max(tile_amax, 1e-12) with IEEE division).
 *   q, scale   q e4m3 [rows, cols] with tiles of 1x128 along cols;
 *              scale float32 [rows, cols/128] = max(tile_amax,1e-12)/448.
 *              Both NULL or both non-NULL.
 *   q_t, scale_t  the transposed copy QUANTIZED AGAIN with 1x128 tiles along
 *              rows (the contraction index of wgrad): q_t e4m3 [cols, rows],
 *              scale_t float32 [cols, rows/128]. Both NULL or both non-NULL.
 *   amax       float32 [rows, cols/128] or NULL: the tile amaxes of q's tiles.
 *
 * FP8_BLOCK_128x128 (weights): rows_valid must equal rows.
 *   q, scale   scale float32 [rows/128, cols/128].
 *   q_t, scale_t  q_t[c,r] = q[r,c]; scale_t [cols/128, rows/128] is the
 *              transposed grid (the same tiles).
 *   amax       float32 [rows/128, cols/128] or NULL.
 *
 * Errors: FP8_ERR_NULL (x NULL with rows*cols > 0, required output missing),
 * FP8_ERR_SHAPE, FP8_ERR_ALIGN, FP8_ERR_HIP.
 */
int fp8_quantize_amax(const void* x, int64_t rows, int64_t cols, int64_t rows_valid,
                      int gran, const float* scale_inv, void* q, void* q_t, float* amax,
                      float* scale, float* scale_t, void* stream);

/*
 * fp8_scale_update -- the delayed-scaling bookkeeping, on the device.
 *
 * Source: [AstrAI] _update_delayed_scale, FP8TensorMeta.record/refresh,
 * FP8State.step.
 *
 * FP8_SCALE_FROM_AMAX: a = max(amax[0], 1e-12f) (NaN is kept);
 *   scale[0] = a / 448, scale_inv[0] = 448 / a, each ONE correctly rounded
 *   float32 division. Called after the pass that produced amax, this is the
 *   one-step-delayed activation/gradient update; called before the
 *   quantize pass on the same tensor it is current scaling. hist, len, pos
 *   are ignored.
 * FP8_SCALE_RECORD: hist[pos] = amax[0]; 0 <= pos < len. The ring index
 *   lives on the host ([AstrAI] record keeps idx as a Python int), so the
 *   caller advances pos = (pos + 1) % len. scale, scale_inv are ignored.
 * FP8_SCALE_REFRESH: m = max(hist[0..len)) (NaN propagates); if m > 0:
 *   scale[0] = m / 448, scale_inv[0] = 448 / m; otherwise both are left as
 *   they were. amax and pos are ignored. The ring starts as all ones and the
 *   caller refreshes when its step counter reaches a multiple of 16.
 * FP8_SCALE_CLEAR_AMAX (flag, FROM_AMAX and RECORD): amax[0] is set to +0
 *   after it is read, ready for a FP8_AMAX_ACCUMULATE quantize pass.
 * FP8_E5M2 (flag, FROM_AMAX and REFRESH): 57344 replaces 448 in both
 *   divisions, for a tensor coded in E5M2.
 *
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE (len < 1, pos out of range, bad mode
 * -> FP8_ERR_UNSUPPORTED), FP8_ERR_HIP.
 */
int fp8_scale_update(int mode, float* amax, float* hist, int32_t len, int32_t pos,
                     float* scale, float* scale_inv, void* stream);

/*
 * fp8_linear_fwd -- y = x W^T as the scaled FP8 GEMM.
 *
 * Source: [AstrAI] module comment "D = A_SCALE * B_SCALE * A * B" and
 * fp8_linear_forward (the scaled forward kernel call).
 *
 *   qx  e4m3 [M, K], qw e4m3 [N, K] (both contraction-index-last).
 *   y   bf16 [M, N]: y[m,n] = bf16_rne(sx * sw * sum_k qx[m,k] * qw[n,k])
 *       for m < M_valid (float32 accumulation on the matrix cores, scales
 *       applied in float32 after accumulation), y[m,n] = 0 for m >= M_valid.
 *   FP8_TENSORWISE: sx, sw float32 [1] (dequant scales amax/448).
 *   FP8_BLOCK_1x128 (the block recipe): sx [M, K/128], sw [N/128, K/128];
 *       the scales multiply each 128-wide partial sum.
 *   M, N, K multiples of 16 (K, N multiples of 128 in the block recipe);
 *   0 <= M_valid <= M. FP8_A_E5M2 OR-ed into gran (FP8_TENSORWISE only): the
 *   first operand holds E5M2 codes (the same for dgrad's qg and wgrad's qg_t,
 *   the hybrid format's gradients). K = 0 (an empty sum) writes +0 everywhere and reads
 *   neither operands nor scales, which may then be NULL (the same holds for
 *   the contraction size of dgrad and wgrad).
 */
int fp8_linear_fwd(const void* qx, const void* qw, const float* sx, const float* sw, void* y,
                   int64_t M, int64_t N, int64_t K, int64_t M_valid, int gran, void* stream);

/*
 * fp8_linear_dgrad -- dx = g W from the e4m3 gradient and W's transposed copy.
 *
 * Source: [AstrAI] fp8_linear_backward (input gradient of the scaled backward).
 *
 *   qg  e4m3 [M, N], qw_t e4m3 [K, N] (the q_t output of quantizing W [N, K]).
 *   dx  bf16 [M, K]: dx[m,k] = bf16_rne(sg * sw * sum_n qg[m,n] * qw_t[k,n])
 *       for m < M_valid, 0 otherwise.
 *   FP8_TENSORWISE: sg, sw float32 [1].
 *   FP8_BLOCK_1x128: sg [M, N/128], sw = W's scale_t grid [K/128, N/128].
 */
int fp8_linear_dgrad(const void* qg, const void* qw_t, const float* sg, const float* sw, void* dx,
                     int64_t M, int64_t N, int64_t K, int64_t M_valid, int gran, void* stream);

/*
 * fp8_linear_wgrad -- dW = g^T x from the two transposed copies.
 *
 * Source: [AstrAI] fp8_linear_backward (weight gradient); [SpecForge]
 * Constraints bullet: this GEMM contracts over the token count M, which is
 * why M must be a multiple of 16.
 *
 *   qg_t e4m3 [N, M], qx_t e4m3 [K, M] (q_t outputs of quantizing g and x).
 *   dw   bf16 [N, K]: dw[n,k] = bf16_rne(sg * sx * sum_m qg_t[n,m] * qx_t[k,m]).
 *        Padded tokens contribute nothing because their codes are 0x00; with
 *        M = 0 (no tokens) dw is all +0.
 *   FP8_TENSORWISE: sg, sx float32 [1] -- sx must be the scale that
 *        quantized x in the forward (not the updated one).
 *   FP8_BLOCK_1x128: sg = g's scale_t [N, M/128], sx = x's scale_t [K, M/128].
 */
int fp8_linear_wgrad(const void* qg_t, const void* qx_t, const float* sg, const float* sx, void* dw,
                     int64_t M, int64_t N, int64_t K, int gran, void* stream);

/*
 * fp8_linear_fwd_current -- one current-scaling forward of a small linear in one
 * launch: the amax of x and of W, their scales, the casts and the GEMM.
 *
 * Source: [SpecForge] Modifications (torchao Float8Linear with dynamic
 * tensorwise scaling: amax first, then the scale, then the cast); [AstrAI]
 * _update_delayed_scale (scale = amax/448, multiplier 448/amax, amax clamped
 * at 1e-12) applied with no delay; [NeMo] reply on FP8 speedups (on very small
 * matmuls the scaling overhead can exceed the gain, which is why this is one
 * launch).
 *
 *   x       bf16 [M, K]; w bf16 [N, K]. M, N positive multiples of 16, K a
 *           positive multiple of 128, and (M + N) * K <= 65536: one workgroup per
 *           16x16 tile of y reads the whole of both operands for the amaxes, so
 *           this call is for small linears only; larger ones use fp8_quantize_amax,
 *           fp8_scale_update and fp8_linear_fwd (FP8_ERR_UNSUPPORTED says so).
 *   y       bf16 [M, N] out: y[m,n] = bf16_rne(float32(sx * sw) *
 *           sum_k qx[m,k] * qw[n,k]), float32 accumulation.
 *   scales  float32 [4] out: {sx, sw, sx_inv, sw_inv}, each scale
 *           max(amax, 1e-12)/448 and multiplier 448/max(amax, 1e-12), amax the
 *           largest |value| of the whole tensor (NaN if any element is NaN).
 *   qx, qw  e4m3 [M, K] and [N, K] out, or NULL: the codes (for a backward).
 * All device pointers 16-byte aligned (scales: 4-byte). Same results, bit for
 * bit in codes and scales, as fp8_quantize_amax (with a cleared amax),
 * fp8_scale_update(FP8_SCALE_FROM_AMAX) and fp8_linear_fwd in sequence.
 * Errors: FP8_ERR_SHAPE, FP8_ERR_UNSUPPORTED, FP8_ERR_NULL, FP8_ERR_ALIGN.
 */
int fp8_linear_fwd_current(const void* x, const void* w, int64_t M, int64_t N, int64_t K,
                           void* y, float* scales, void* qx, void* qw, void* stream);

/*
 * fp8_linear_fwd_bias -- fp8_linear_fwd with a bias added in the GEMM's epilogue.
 *
 * Source: [AstrAI] fp8_linear_forward(x, w, bias): the bias goes to the scaled
 * forward kernel with the operands.
 *
 *   bias  bf16 [N] or NULL (NULL: exactly fp8_linear_fwd). FP8_TENSORWISE only.
 *   y     y[m,n] = bf16_rne(float32(sx * sw * sum_k qx[m,k] * qw[n,k]) + float32(bias[n]))
 *         for m < M_valid (one rounding, after the bias), 0 otherwise; with K = 0
 *         the valid rows are the bias.
 *   Other arguments and errors as fp8_linear_fwd; bias must be 16-byte aligned.
 */
int fp8_linear_fwd_bias(const void* qx, const void* qw, const float* sx, const float* sw,
                        const void* bias, void* y, int64_t M, int64_t N, int64_t K,
                        int64_t M_valid, int gran, void* stream);

/*
 * fp8_bias_grad -- the bias gradient: column sums of the output gradient.
 *
 * Source: [AstrAI] fp8_linear_backward(g, x, w, masks): masks select the input,
 * weight and bias gradients of the linear.
 *
 *   g     bf16 [rows, cols], cols a multiple of 16; rows r >= rows_valid are token
 *         padding and are not read.
 *   db    bf16 [cols]: db[c] = bf16_rne(sum over r < rows_valid of float32(g[r,c])),
 *         float32 sums in a fixed order (the same result on every call); 0 if
 *         rows_valid = 0.
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_ALIGN (g 16-byte aligned),
 * FP8_ERR_UNSUPPORTED (g of 2^31 bytes or more), FP8_ERR_HIP.
 */
int fp8_bias_grad(const void* g, int64_t rows, int64_t cols, int64_t rows_valid, void* db,
                  void* stream);

/*
 * fp8_pad_tokens -- pad a packed token batch to a multiple of `multiple` rows.
 *
 * Source: [NeMo] review thread, "pad = (-T) % seq_multiple"; [SpecForge]
 * Constraints bullet (multiple of 16 for float8 GEMMs).
 *
 *   x        bf16 [T, cols] (read-only unless x_pad == x).
 *   T, cols  >= 0; multiple >= 1.
 *   T_pad    host int64 out: T + ((-T) mod multiple). Required.
 *   x_pad    NULL: only T_pad is computed (nothing is enqueued).
 *            == x: in place; the buffer holds T_pad rows and rows [T, T_pad)
 *            are zeroed.
 *            otherwise bf16 [T_pad, cols]: rows [0, T) copied, [T, T_pad) zeroed.
 *   Padding goes at the end of the concatenated batch.
 */
int fp8_pad_tokens(const void* x, int64_t T, int64_t cols, int32_t multiple, void* x_pad,
                   int64_t* T_pad, void* stream);

/* Layouts of fp8_align_multiple. */
enum { FP8_LAYOUT_THD = 0, FP8_LAYOUT_BSHD = 1 };

/*
 * fp8_align_multiple -- the token multiples a layout needs under tensor (tp),
 * sequence and context (cp) parallelism. Host-only integer arithmetic.
 *
 * Source: [NeMo] review thread on BSHD padding: with sequence parallelism the
 * local GEMM sees M = B*T/tp tokens, so FP8 needs B*T % (base*tp) == 0 and
 * T % tp == 0, which padding T to base*tp/gcd(B, base*tp) alone does not
 * give (the thread's case B=16, tp=4 asks only for a multiple of 2); the
 * THD helper pads the packed total to base * cp_size * tp_size.
 *
 *   layout  FP8_LAYOUT_THD (packed): *seq_multiple = 2*cp if cp > 1 else 1 (a
 *           reading: load-balanced context parallelism cuts each sequence into
 *           2*cp chunks), *total_multiple = base*cp*tp.
 *           FP8_LAYOUT_BSHD (B sequences padded to one length T; cp must be 1):
 *           *seq_multiple = lcm(tp, base*tp/gcd(B, base*tp)) for T,
 *           *total_multiple = 1.
 *   batch   B (BSHD; ignored for THD), tp, cp, base >= 1 (base: the FP8 multiple,
 *           16 for this library's GEMMs).
 * Errors: FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_UNSUPPORTED (unknown layout,
 * BSHD with cp > 1).
 */
int fp8_align_multiple(int layout, int64_t batch, int32_t tp, int32_t cp, int32_t base,
                       int32_t* seq_multiple, int32_t* total_multiple);

/*
 * fp8_pad_varlen -- pad every sequence of a packed batch, then the batch.
 *
 * Source: [NeMo] review thread (per-layout token multiples, above); [NeMo-packed]
 * NeMo Speech PR 16194 summary: padding-free packed batches with CP/FSDP/FP8
 * alignment.
 *
 *   x             bf16 [cu_seqlens[nseq], cols], the sequences packed in order.
 *   cu_seqlens    HOST int64 [nseq + 1]: 0 = cu[0] <= cu[1] <= ... (sequence i is
 *                 rows cu[i] .. cu[i+1]).
 *   seq_multiple  each sequence of length L takes L + ((-L) mod seq_multiple) rows;
 *   total_multiple  the padded sequences' end E is padded to E + ((-E) mod total_multiple).
 *   cu_seqlens_pad  HOST int64 [nseq + 1] out (required with x_pad): where sequence i
 *                 starts in x_pad; cu_seqlens_pad[nseq] = E.
 *   T_pad         HOST int64 out, required: the padded row count.
 *   x_pad         NULL: only the offsets are computed (nothing is enqueued).
 *                 Otherwise bf16 [T_pad, cols], not aliasing x: sequence rows copied,
 *                 every padding row zero.
 *   cols          a multiple of 16; x and x_pad 16-byte aligned.
 * Zero padding rows quantize to 0x00 and add nothing to any GEMM sum; the
 * forward output and dx at those rows are 0 (without a bias).
 */
int fp8_pad_varlen(const void* x, const int64_t* cu_seqlens, int32_t nseq, int64_t cols,
                   int32_t seq_multiple, int32_t total_multiple, void* x_pad,
                   int64_t* cu_seqlens_pad, int64_t* T_pad, void* stream);

/*
 * fp8_unpad_varlen -- the inverse gather: x[cu[i] + j] = x_pad[cu_pad[i] + j] for
 * j < cu[i+1] - cu[i] (e.g. dx of a padded batch back to the packed tokens).
 *   x_pad bf16 [>= cu_pad[nseq], cols]; x bf16 [cu[nseq], cols], not aliasing x_pad.
 *   cu_seqlens, cu_seqlens_pad  HOST int64 [nseq + 1], both from 0 and non-decreasing,
 *   every padded sequence at least as long as its sequence.
 */
int fp8_unpad_varlen(const void* x_pad, const int64_t* cu_seqlens, const int64_t* cu_seqlens_pad,
                     int32_t nseq, int64_t cols, void* x, void* stream);

/* Message for the last error returned on the calling thread ("" if none). */
const char* fp8_last_error(void);

/* Library version, e.g. "fp8lin 0.1 gfx950". */
const char* fp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8LIN_H */
