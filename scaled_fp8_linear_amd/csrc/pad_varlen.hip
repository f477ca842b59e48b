// Per-sequence padding of a packed (THD) token batch, and its inverse.
//
// NeMo PR 15754, review thread on BSHD padding: under tensor / sequence /
// context parallelism every rank's share of the tokens must be a multiple of
// the FP8 multiple and a sequence split over ranks must split evenly, so a
// packed batch pads each sequence to a multiple of its own and the whole batch
// to another (the thread's THD helper: 8 * cp_size * tp_size).
//
// pad:   sequence i (rows src[i] .. src[i+1] of x) goes to rows dst[i] .. of
//        x_pad, followed by zero rows up to dst[i+1]; rows past the last
//        sequence's padded end are zero (the total padding).
// unpad: the inverse gather, rows dst[i] + j of x_pad -> rows src[i] + j of x.
// Pure HBM copy (2 bytes read and 2 written per element): a workgroup moves
// kRows rows per step with 16-byte loads and stores, every lane issuing all its
// loads of the step (kRows x kUnits) before its first store. The row offsets travel in
// the kernel arguments (up to kSeqPerLaunch sequences per launch), so the call
// needs no device memory of its own; the sequence that holds a row is found by
// a binary search that is uniform across the workgroup.
#include "common.h"
#include "launch.h"

namespace fp8lin {

namespace {

struct SeqTable {
  int32_t n;                          // sequences in this launch
  int64_t src[kSeqPerLaunch + 1];     // packed row offsets of the sequences (absolute)
  int64_t dst[kSeqPerLaunch + 1];     // padded row offsets
};

// Largest i in [0, n] with off[i] <= r (off non-decreasing, off[0] <= r).
__device__ __forceinline__ int find_seq(const int64_t* off, int n, int64_t r) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// rows per step; 16-byte units per lane and row; workgroups (measured at 54 784 x 4096:
// 256 of them 4.1 TB/s, 512 5.5, 1024 5.2)
constexpr int kRows = 4, kUnits = 2;
constexpr int64_t kVarlenBlocks = 512;

// PAD: output rows [row_begin, row_end) of x_pad. UNPAD: output rows [row_begin, row_end)
// of x. chunks = cols / 8 (16-byte units per row).
template <bool PAD>
__global__ void __launch_bounds__(256)
pad_varlen_kernel(const uint4* __restrict__ in, uint4* __restrict__ out, int64_t chunks,
                  SeqTable tab, int64_t row_begin, int64_t row_end) {
  // the offsets in LDS, where the searches read them
  __shared__ int64_t s_src[kSeqPerLaunch + 1], s_dst[kSeqPerLaunch + 1];
  for (int i = threadIdx.x; i <= tab.n; i += blockDim.x) {
    s_src[i] = tab.src[i];
    s_dst[i] = tab.dst[i];
  }
  __syncthreads();
  for (int64_t r0 = row_begin + (int64_t)kRows * blockIdx.x; r0 < row_end;
       r0 += (int64_t)kRows * gridDim.x) {
    // the source row of each output row of the step (uniform): -1 a zero row, -2 none
    int64_t from[kRows];
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int64_t r = r0 + k;
      from[k] = -2;
      if (r < row_end) {
        from[k] = -1;
        if (PAD) {
          const int i = find_seq(s_dst, tab.n, r);
          if (i < tab.n && r - s_dst[i] < s_src[i + 1] - s_src[i])
            from[k] = s_src[i] + (r - s_dst[i]);
        } else {
          const int i = find_seq(s_src, tab.n, r);
          from[k] = s_dst[i] + (r - s_src[i]);
        }
      }
    }
    for (int64_t c0 = threadIdx.x; c0 < chunks; c0 += 256 * kUnits) {
      uint4 v[kRows][kUnits];
#pragma unroll
      for (int k = 0; k < kRows; ++k)
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
          const int64_t c = c0 + 256 * j;
          v[k][j] = from[k] >= 0 && c < chunks ? ld_stream16(in + from[k] * chunks + c)
                                              : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
      for (int k = 0; k < kRows; ++k)
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
          const int64_t c = c0 + 256 * j;
          if (from[k] >= -1 && c < chunks) out[(r0 + k) * chunks + c] = v[k][j];
        }
    }
  }
}

hipError_t launch_rows(bool pad, const uint16_t* in, uint16_t* out, int64_t cols,
                       const SeqTable& tab, int64_t row_begin, int64_t row_end, hipStream_t s) {
  if (row_end <= row_begin) return hipSuccess;
  int64_t blocks = (row_end - row_begin + kRows - 1) / kRows;
  if (blocks > kVarlenBlocks) blocks = kVarlenBlocks;
  const int64_t chunks = cols / 8;
  if (pad)
    hipLaunchKernelGGL(pad_varlen_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(in), reinterpret_cast<uint4*>(out), chunks,
                       tab, row_begin, row_end);
  else
    hipLaunchKernelGGL(pad_varlen_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(in), reinterpret_cast<uint4*>(out), chunks,
                       tab, row_begin, row_end);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pad_varlen(bool pad, const uint16_t* in, uint16_t* out, int64_t cols,
                             const int64_t* cu, const int64_t* cu_pad, int32_t nseq,
                             int64_t T_pad, hipStream_t s) {
  if (cols == 0) return hipSuccess;
  for (int32_t s0 = 0; s0 < nseq || (s0 == 0 && nseq == 0); s0 += kSeqPerLaunch) {
    const int32_t n = nseq - s0 < kSeqPerLaunch ? nseq - s0 : kSeqPerLaunch;
    SeqTable tab;
    tab.n = n;
    for (int32_t i = 0; i <= n; ++i) {
      tab.src[i] = cu[s0 + i];
      tab.dst[i] = cu_pad[s0 + i];
    }
    const bool last = s0 + n >= nseq;
    hipError_t e;
    if (pad)        // this launch's padded rows, and the total padding after the last one
      e = launch_rows(true, in, out, cols, tab, tab.dst[0], last ? T_pad : tab.dst[n], s);
    else
      e = launch_rows(false, in, out, cols, tab, tab.src[0], tab.src[n], s);
    if (e != hipSuccess) return e;
    if (nseq == 0) break;
  }
  return hipSuccess;
}

}  // namespace fp8lin
