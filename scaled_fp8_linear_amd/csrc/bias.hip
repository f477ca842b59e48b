// Bias of the linear layer: its gradient, and the output of an empty contraction.
//
// AstrAI, astrai/extension/fp8_state.py: fp8_linear_forward(x, w, bias) hands the bias to
// the scaled forward kernel, and fp8_linear_backward's masks ask for the input, weight and
// bias gradients. The bias joins the forward GEMM's epilogue (gemm_fp8.hip); this file
// holds
//  * bias_grad_kernel: db[c] = sum over the valid rows r of g[r, c], float32 sums in a
//    fixed order (so the result is the same on every run), rounded once to bf16;
//  * bias_rows_kernel: y[m, :] = bias for the valid rows, 0 below (a forward with K = 0).
#include "common.h"
#include "launch.h"

namespace fp8lin {

namespace {

constexpr int kGradCols = 64;            // columns per workgroup
constexpr int kGradThreads = 256;        // 8 lanes x 8 columns per row, 32 row groups
constexpr int kRowGroups = kGradThreads / (kGradCols / 8);

// Workgroup b owns columns [64 b, 64 b + 64). Lane t sums the 8 columns 8 (t % 8) .. + 8
// of the rows t / 8, t / 8 + 32, ... (one 16-byte load per row: 8 lanes read a row's
// 128 contiguous bytes); the 32 row-group sums of each column are then added in row-group
// order through LDS.
__global__ void __launch_bounds__(kGradThreads)
bias_grad_kernel(const uint16_t* __restrict__ g, int64_t rows_valid, int64_t cols,
                 uint16_t* __restrict__ db) {
  __shared__ float part[kRowGroups][kGradCols + 1];
  const int t = threadIdx.x;
  const int cc = t % 8, rg = t / 8;
  const int64_t c0 = (int64_t)blockIdx.x * kGradCols + 8 * cc;
  const bool live = c0 < cols;           // cols is a multiple of 16, so 8 columns fit
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (live) {
    const uint16_t* p = g + c0;
    int64_t r = rg;
    // four rows per round, loaded before they are added (in row order)
    for (; r + 3 * kRowGroups < rows_valid; r += 4 * kRowGroups) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = *reinterpret_cast<const uint4*>(p + (r + u * kRowGroups) * cols);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s[0] += bf16_lo(v[u].x); s[1] += bf16_hi(v[u].x);
        s[2] += bf16_lo(v[u].y); s[3] += bf16_hi(v[u].y);
        s[4] += bf16_lo(v[u].z); s[5] += bf16_hi(v[u].z);
        s[6] += bf16_lo(v[u].w); s[7] += bf16_hi(v[u].w);
      }
    }
    for (; r < rows_valid; r += kRowGroups) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + r * cols);
      s[0] += bf16_lo(v.x); s[1] += bf16_hi(v.x);
      s[2] += bf16_lo(v.y); s[3] += bf16_hi(v.y);
      s[4] += bf16_lo(v.z); s[5] += bf16_hi(v.z);
      s[6] += bf16_lo(v.w); s[7] += bf16_hi(v.w);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][8 * cc + e] = s[e];
  __syncthreads();
  if (t < kGradCols) {
    const int64_t c = (int64_t)blockIdx.x * kGradCols + t;
    if (c < cols) {
      float acc = 0.f;
      for (int k = 0; k < kRowGroups; ++k) acc += part[k][t];
      db[c] = (uint16_t)f32_to_bf16_bits(acc);
    }
  }
}

// 8 bf16 (16 bytes) per item: row m, column chunk c8 of the [M, N] output.
__global__ void bias_rows_kernel(const uint16_t* __restrict__ bias, uint16_t* __restrict__ D,
                                 int64_t M, int64_t N, int64_t M_valid) {
  const int64_t chunks = N / 8, items = M * chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items; i += stride) {
    const int64_t m = i / chunks, c = (i % chunks) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < M_valid) v = *reinterpret_cast<const uint4*>(bias + c);
    *reinterpret_cast<uint4*>(D + m * N + c) = v;
  }
}

}  // namespace

hipError_t launch_bias_grad(const uint16_t* g, int64_t rows, int64_t cols, int64_t rows_valid,
                            uint16_t* db, hipStream_t s) {
  (void)rows;
  if (cols == 0) return hipSuccess;
  const int64_t blocks = (cols + kGradCols - 1) / kGradCols;
  hipLaunchKernelGGL(bias_grad_kernel, dim3((unsigned)blocks), dim3(kGradThreads), 0, s, g,
                     rows_valid, cols, db);
  return hipGetLastError();
}

hipError_t launch_bias_rows(const uint16_t* bias, uint16_t* D, int64_t M, int64_t N,
                            int64_t M_valid, hipStream_t s) {
  const int64_t items = M * (N / 8);
  if (items == 0) return hipSuccess;
  int64_t blocks = (items + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(bias_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, bias, D, M, N,
                     M_valid);
  return hipGetLastError();
}

}  // namespace fp8lin
