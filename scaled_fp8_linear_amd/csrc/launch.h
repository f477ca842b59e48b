// Internal launchers: one per kernel family. Host-side argument checking lives
// in abi.cpp; these only enqueue work on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s);

// accumulate: fold max|x| into amax[0] instead of zeroing it first; e5m2: OCP e5m2
// codes instead of e4m3.
hipError_t launch_quantize_tensorwise(const uint16_t* x, int64_t rows, int64_t cols,
                                      int64_t rows_valid, const float* scale_inv, uint8_t* q,
                                      uint8_t* q_t, float* amax, bool accumulate, bool e5m2,
                                      hipStream_t s);

// Block recipe: 1x128 tiles (activations/gradients), 128x128 tiles (weights).
hipError_t launch_quantize_block_1x128(const uint16_t* x, int64_t rows, int64_t cols,
                                       int64_t rows_valid, uint8_t* q, uint8_t* q_t,
                                       float* amax, float* scale, float* scale_t, hipStream_t s);
hipError_t launch_quantize_block_128x128(const uint16_t* x, int64_t rows, int64_t cols,
                                         uint8_t* q, uint8_t* q_t, float* amax, float* scale,
                                         float* scale_t, hipStream_t s);

// clear_amax: set amax[0] to +0 after reading it (modes 0 and 1); e5m2: the format
// maximum is 57344 instead of 448 (modes 0 and 2).
hipError_t launch_scale_update(int mode, float* amax, bool clear_amax, float* hist, int32_t len,
                               int32_t pos, float* scale, float* scale_inv, bool e5m2,
                               hipStream_t s);

// Current-scaling forward of a small linear in one launch, one workgroup per 16x16 tile of
// y. Each workgroup reads the whole of x and W for the amaxes, so (M + N) K, the bytes of
// codes of both operands, is capped; a tile's own 32 K bytes of codes live in LDS between
// the cast and the GEMM.
constexpr int kSmallLinearCodes = 64 * 1024;
hipError_t launch_linear_current_small(const uint16_t* x, const uint16_t* w, int M, int N, int K,
                                       uint16_t* y, float* scales, uint8_t* qx, uint8_t* qw,
                                       hipStream_t s);

hipError_t launch_pad_tokens(const uint16_t* x, int64_t T, int64_t cols, int64_t T_pad,
                             uint16_t* x_pad, hipStream_t s);

// Sequences per launch of the per-sequence padding kernel (its row offsets travel in the
// kernel arguments).
constexpr int kSeqPerLaunch = 128;

// pad: x [cu[nseq], cols] -> x_pad [T_pad, cols] (sequence i at row cu_pad[i], zero rows
// after it up to cu_pad[i + 1], zero rows from cu_pad[nseq] to T_pad); !pad: the inverse
// gather x_pad -> x. cu, cu_pad: host offsets [nseq + 1]; cols % 8 == 0, 16-byte aligned rows.
hipError_t launch_pad_varlen(bool pad, const uint16_t* in, uint16_t* out, int64_t cols,
                             const int64_t* cu, const int64_t* cu_pad, int32_t nseq,
                             int64_t T_pad, hipStream_t s);

// D[m,n] = bf16(scale * sum_k A[m,k] * B[n,k] (+ bias[n])); A [M,K], B [N,K], D [M,N].
// Tensorwise: scale = sa[0] * sb[0]; bias bf16 [N] or nullptr. Block: sa [M, K/128];
// sb [N/b_rows, K/128] with b_rows = 128 (weight tiles) or 1 (1x128 tiles); no bias.
// Rows m >= M_valid of D are 0. a_e5m2: A holds OCP e5m2 codes (tensorwise, no bias).
hipError_t launch_gemm_fp8(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                           const uint16_t* bias, uint16_t* D, int64_t M, int64_t N, int64_t K,
                           int64_t M_valid, bool block_scaled, int b_rows_per_scale, bool a_e5m2,
                           hipStream_t s);

// D[m, :] = bias for m < M_valid, 0 below (the output of an empty contraction with bias).
hipError_t launch_bias_rows(const uint16_t* bias, uint16_t* D, int64_t M, int64_t N,
                            int64_t M_valid, hipStream_t s);

// db[c] = bf16(sum over r < rows_valid of g[r, c]), float32 sums in a fixed order.
hipError_t launch_bias_grad(const uint16_t* g, int64_t rows, int64_t cols, int64_t rows_valid,
                            uint16_t* db, hipStream_t s);

}  // namespace fp8lin
