// Token-count padding of a packed batch (NeMo PR 15754 review thread:
// pad = (-T) % seq_multiple; SpecForge PR 2, Constraints: FP8 GEMMs need the
// token count to be a multiple of 16). Rows [0, T) are copied (unless the
// copy is in place) and rows [T, T_pad) are zeroed. Pure HBM copy: 512 workgroups
// of 256 lanes stride over the rows, each lane moving four 16-byte units per step
// (the four streaming loads issued before the first store). A fixed grid keeps
// every CU busy to the end, where one workgroup per 128 KB left a part-filled
// last round (117 MB: 4.8 against 5.7 TB/s).
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace fp8lin {

namespace {

constexpr int kPadLanes = 256, kPadUnits = 4;    // 16-byte units per lane and step
constexpr int64_t kPadBlocks = 512;

__global__ void __launch_bounds__(kPadLanes)
pad_rows_kernel(const uint4* __restrict__ src, int64_t n_copy, uint4* __restrict__ dst,
                int64_t n_total) {
  const int64_t step = (int64_t)gridDim.x * (kPadLanes * kPadUnits);
  for (int64_t base = (int64_t)blockIdx.x * (kPadLanes * kPadUnits) + threadIdx.x; base < n_total;
       base += step) {
    uint4 v[kPadUnits];
#pragma unroll
    for (int j = 0; j < kPadUnits; ++j) {
      const int64_t i = base + (int64_t)kPadLanes * j;
      v[j] = i < n_copy ? ld_stream16(src + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kPadUnits; ++j) {
      const int64_t i = base + (int64_t)kPadLanes * j;
      if (i < n_total) dst[i] = v[j];
    }
  }
}

__global__ void __launch_bounds__(256)
pad_rows_bytes_kernel(const uint16_t* __restrict__ src, int64_t n_copy, uint16_t* __restrict__ dst,
                      int64_t n_total) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_total; i += stride) {
    dst[i] = (i < n_copy) ? src[i] : (uint16_t)0;
  }
}

}  // namespace

hipError_t launch_pad_tokens(const uint16_t* x, int64_t T, int64_t cols, int64_t T_pad,
                             uint16_t* x_pad, hipStream_t s) {
  const bool in_place = (x == x_pad);
  const int64_t first = in_place ? T * cols : 0;           // elements already in place
  const int64_t n_copy = T * cols - first;
  const int64_t n_total = T_pad * cols - first;
  if (n_total <= 0) return hipSuccess;
  const uint16_t* src = x + first;
  uint16_t* dst = x_pad + first;
  const bool vec = ((first % 8) == 0) && ((n_copy % 8) == 0) && ((n_total % 8) == 0) &&
                   ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 == 0);
  if (vec) {
    const int64_t units = n_total / 8;
    const int64_t blocks =
        std::min(kPadBlocks, (units + kPadLanes * kPadUnits - 1) / (kPadLanes * kPadUnits));
    hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)blocks), dim3(kPadLanes), 0, s,
                       reinterpret_cast<const uint4*>(src), n_copy / 8,
                       reinterpret_cast<uint4*>(dst), units);
  } else {
    int64_t blocks = (n_total + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(pad_rows_bytes_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, n_copy,
                       dst, n_total);
  }
  return hipGetLastError();
}

}  // namespace fp8lin
