// Fused bf16 -> e4m3 (or e5m2) quantize + amax + transposed copy (tensorwise scaling).
//
// What it computes (AstrAI, astrai/extension/fp8_state.py: module comment on
// the GEMM layout and fp8_linear_forward's docstring): for a bf16 [rows, cols]
// tensor x and the float32 multiplier scale_inv (= 448/amax of the scale in
// force), q[r,c] = e4m3(float32(x[r,c]) * scale_inv), its transpose q_t, and
// amax = max|x| over the valid rows, taken in the same pass ("free" amax).
// Gradients may instead be coded in OCP e5m2 (the hybrid format: wider range,
// one mantissa bit less), with the multiplier 57344/amax.
//
// Design (HBM-bound: 2 bytes read, 2 bytes written per element):
//  * a workgroup of 1024 lanes owns a TR x TC tile (128 x 256);
//  * every lane reads 4 consecutive rows x 8 columns with 16-byte loads, all
//    issued before any is used; the 64 lanes of a wavefront cover two 512-byte
//    row segments per load;
//  * q is written straight from registers (8 bytes per lane per row);
//  * the 4x8 code block is transposed in registers into eight 4-byte column
//    pieces that go to LDS; after one barrier each lane gathers 16 rows of
//    one column and writes q_t with 16-byte stores, 128 contiguous bytes per
//    q_t row per 8 lanes;
//  * amax is a max over the 15-bit magnitudes of the bf16 patterns (exact,
//    and NaN patterns sort above infinity), reduced across the wavefront with
//    shuffles, across the workgroup in LDS, and published with ONE atomicMax
//    per workgroup on the float bits (non-negative floats order as integers).
#include "common.h"
#include "launch.h"

namespace fp8lin {

namespace {

// Tile of TR rows x TC columns per workgroup of THREADS lanes. NT selects
// streaming (non-temporal) accesses per stream: bit 0 the bf16 loads, bit 1 the
// q stores, bit 2 the q_t stores.
template <int TR, int TC, int THREADS, int NT>
struct QCfg {
  static constexpr int kQTR = TR, kQTC = TC, kQThreads = THREADS;
  static constexpr int kNT = NT;
  static constexpr int kColDwords = TR / 4;          // dwords per transposed column piece
  static constexpr int kChunks = TC / 8;             // 8-column chunks per tile row
  static constexpr int kGroups = THREADS / kChunks;  // 4-row groups per pass
  static constexpr int kRowsPerPass = 4 * kGroups;
  static constexpr int kPasses = TR / kRowsPerPass;
  static_assert(THREADS % kChunks == 0 && TR % kRowsPerPass == 0, "tile shape");
};

// Physical dword slot of logical dword `i` of column `c` in the LDS tile.
// XOR with the column's chunk index spreads the lanes that store the same
// logical dword over the banks.
template <int COLDW>
__device__ __forceinline__ int lds_slot(int c, int i) {
  return c * COLDW + (i ^ ((c >> 3) & (COLDW - 1)));
}

template <int NT>
__device__ __forceinline__ uint4 ld16(const void* p) {
  if constexpr ((NT & 1) != 0) return ld_stream16(p);
  else return *reinterpret_cast<const uint4*>(p);
}
template <int NT>
__device__ __forceinline__ void st16(void* p, uint4 v) {
  if constexpr ((NT & 4) != 0) st_stream16(p, v);
  else *reinterpret_cast<uint4*>(p) = v;
}
template <int NT>
__device__ __forceinline__ void st8(void* p, uint32_t a, uint32_t b) {
  if constexpr ((NT & 2) != 0) st_stream8(p, a, b);
  else *reinterpret_cast<uint2*>(p) = make_uint2(a, b);
}

// FMT: 0 OCP e4m3 codes, 1 OCP e5m2 codes (gradients in the hybrid format).
template <class QC, int FMT>
__global__ void __launch_bounds__(QC::kQThreads)
quantize_tensorwise_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                           int64_t rows_valid, const float* __restrict__ scale_inv_p,
                           uint8_t* __restrict__ q, uint8_t* __restrict__ q_t,
                           uint32_t* __restrict__ amax_bits, int64_t tiles_c) {
  constexpr int kQTR = QC::kQTR, kQTC = QC::kQTC, kQThreads = QC::kQThreads;
  constexpr int kColDwords = QC::kColDwords;
  constexpr int NT = QC::kNT;
  __shared__ uint32_t tile_t[kQTC * kColDwords];
  __shared__ uint32_t wave_max[kQThreads / 64];

  const int t = threadIdx.x;
  const int64_t tile = blockIdx.x;
  const int64_t row0 = (tile / tiles_c) * kQTR;
  const int64_t col0 = (tile % tiles_c) * kQTC;
  const bool want_q = q != nullptr, want_t = q_t != nullptr;
  const bool want_codes = want_q | want_t;
  const float s = want_codes ? *scale_inv_p : 1.0f;

  const int cc = t % QC::kChunks;   // 8-column chunk inside the tile
  const int rg = t / QC::kChunks;   // 4-row group
  const int64_t col = col0 + 8 * cc;
  const bool col_ok = col < cols;
  constexpr int kPasses = QC::kPasses;
  constexpr int kRPP = QC::kRowsPerPass;

  // All loads of the lane (4 per pass) go out before any is used. Rows past rows_valid
  // (token padding) and columns past cols are not read: those lanes skip the load and
  // hold zeros.
  uint4 v[kPasses][4];
  bool ok[kPasses][4];
#pragma unroll
  for (int p = 0; p < kPasses; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = row0 + kRPP * p + 4 * rg + i;
      ok[p][i] = col_ok && (r < rows_valid);
      v[p][i] = ok[p][i] ? ld16<NT>(x + r * cols + col) : make_uint4(0, 0, 0, 0);
    }
  uint32_t mx = 0;
#pragma unroll
  for (int p = 0; p < kPasses; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m0 = v[p][i].x & 0x7FFF7FFFu, m1 = v[p][i].y & 0x7FFF7FFFu;
      const uint32_t m2 = v[p][i].z & 0x7FFF7FFFu, m3 = v[p][i].w & 0x7FFF7FFFu;
      const uint32_t a = max(max(m0 & 0xFFFFu, m0 >> 16), max(m1 & 0xFFFFu, m1 >> 16));
      const uint32_t b = max(max(m2 & 0xFFFFu, m2 >> 16), max(m3 & 0xFFFFu, m3 >> 16));
      mx = max(mx, max(a, b));
    }

  if (want_codes) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int lr = kRPP * p + 4 * rg;      // first of 4 consecutive tile rows
      uint32_t lo[4], hi[4];   // codes of columns 0..3 / 4..7 of each row
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = quant4_fmt<FMT>(v[p][i].x, v[p][i].y, s, s, s, s);
        hi[i] = quant4_fmt<FMT>(v[p][i].z, v[p][i].w, s, s, s, s);
        if (!ok[p][i]) { lo[i] = 0u; hi[i] = 0u; }      // padding rows are written as 0x00
      }
      if (want_q) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t r = row0 + lr + i;
          if (col_ok && r < rows)
            st8<NT>(q + r * cols + col, lo[i], hi[i]);
        }
      }
      if (want_t) {
        // 4x4 byte transposes: column j of the chunk gets bytes j of rows 0..3.
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t* w = half ? hi : lo;
          // interleave bytes of rows (0,1) and (2,3), then the 16-bit halves
          uint32_t a01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // r0b0 r1b0 r0b1 r1b1
          uint32_t b01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // r0b2 r1b2 r0b3 r1b3
          uint32_t a23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
          uint32_t b23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
          uint32_t c0 = __builtin_amdgcn_perm(a23, a01, 0x05040100u);     // col 0: r0 r1 r2 r3
          uint32_t c1 = __builtin_amdgcn_perm(a23, a01, 0x07060302u);     // col 1
          uint32_t c2 = __builtin_amdgcn_perm(b23, b01, 0x05040100u);     // col 2
          uint32_t c3 = __builtin_amdgcn_perm(b23, b01, 0x07060302u);     // col 3
          const int cb = 8 * cc + 4 * half;
          const int di = lr >> 2;
          tile_t[lds_slot<kColDwords>(cb + 0, di)] = c0;
          tile_t[lds_slot<kColDwords>(cb + 1, di)] = c1;
          tile_t[lds_slot<kColDwords>(cb + 2, di)] = c2;
          tile_t[lds_slot<kColDwords>(cb + 3, di)] = c3;
        }
      }
    }
  }

  if (amax_bits != nullptr) {
    mx = wave_max_u32(mx);
    if ((t & 63) == 0) wave_max[t >> 6] = mx;
  }
  if (want_t || amax_bits != nullptr) __syncthreads();
  if (amax_bits != nullptr && t == 0) {
    uint32_t m = wave_max[0];
#pragma unroll
    for (int w = 1; w < kQThreads / 64; ++w) m = max(m, wave_max[w]);
    atomicMax(amax_bits, m << 16);
  }
  if (!want_t) return;

  // q_t: each item is 16 consecutive rows of one column (one 16-byte store).
  constexpr int kChunksPerCol = kQTR / 16;
  constexpr int kItems = kQTC * kChunksPerCol;
#pragma unroll
  for (int it = 0; it < kItems / kQThreads; ++it) {
    const int idx = it * kQThreads + t;
    const int c = idx / kChunksPerCol;
    const int ch = idx % kChunksPerCol;
    const int64_t gc = col0 + c;
    const int64_t gr = row0 + 16 * ch;
    if (gc < cols && gr < rows) {
      uint4 o;
      o.x = tile_t[lds_slot<kColDwords>(c, 4 * ch + 0)];
      o.y = tile_t[lds_slot<kColDwords>(c, 4 * ch + 1)];
      o.z = tile_t[lds_slot<kColDwords>(c, 4 * ch + 2)];
      o.w = tile_t[lds_slot<kColDwords>(c, 4 * ch + 3)];
      st16<NT>(q_t + gc * rows + gr, o);
    }
  }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

template <class QC>
hipError_t run_q(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_valid,
                 const float* scale_inv, uint8_t* q, uint8_t* q_t, float* amax, bool e5m2,
                 hipStream_t s) {
  const int64_t tiles_r = (rows + QC::kQTR - 1) / QC::kQTR;
  const int64_t tiles_c = (cols + QC::kQTC - 1) / QC::kQTC;
  const int64_t tiles = tiles_r * tiles_c;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (e5m2)
    hipLaunchKernelGGL((quantize_tensorwise_kernel<QC, 1>), dim3((unsigned)tiles),
                       dim3(QC::kQThreads), 0, s, x, rows, cols, rows_valid, scale_inv, q, q_t,
                       reinterpret_cast<uint32_t*>(amax), tiles_c);
  else
    hipLaunchKernelGGL((quantize_tensorwise_kernel<QC, 0>), dim3((unsigned)tiles),
                       dim3(QC::kQThreads), 0, s, x, rows, cols, rows_valid, scale_inv, q, q_t,
                       reinterpret_cast<uint32_t*>(amax), tiles_c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

hipError_t launch_quantize_tensorwise(const uint16_t* x, int64_t rows, int64_t cols,
                                      int64_t rows_valid, const float* scale_inv, uint8_t* q,
                                      uint8_t* q_t, float* amax, bool accumulate, bool e5m2,
                                      hipStream_t s) {
  hipError_t e = hipSuccess;
  if (amax != nullptr && !accumulate) {
    e = launch_fill_u32(reinterpret_cast<uint32_t*>(amax), 0u, 1, s);
    if (e != hipSuccess) return e;
  }
  if (rows == 0 || cols == 0) return hipSuccess;
  if (q == nullptr && q_t == nullptr && amax == nullptr) return hipSuccess;
  if (rows_valid == 0) {
    // nothing to read: every code is 0x00 (amax was set to 0 above, or keeps its value)
    // (a fill kernel, not a memset: the call may be captured in a graph)
    if (q != nullptr &&
        (e = launch_fill_u32(reinterpret_cast<uint32_t*>(q), 0u, rows * cols / 4, s)) != hipSuccess)
      return e;
    if (q_t != nullptr &&
        (e = launch_fill_u32(reinterpret_cast<uint32_t*>(q_t), 0u, rows * cols / 4, s)) != hipSuccess)
      return e;
    return hipSuccess;
  }
  // 128 x 256 tiles for 1024 lanes (one pass: four 16-byte loads per lane, 16 waves per
  // workgroup); streaming loads and q stores, ordinary q_t stores. q_t leaves as 128-byte
  // pieces of rows that lie `rows` bytes apart; streaming stores send each piece to HBM
  // alone, which costs a third of the rate on tall tensors (54672 x 4096: 3.4 against
  // 4.7 TB/s), while the cached path merges neighbouring pieces first. Measured per shape
  // against 256 lanes (four passes): 5-15% faster (x [8192, 4096] 28.3 -> 26.9 us,
  // W [14336, 4096] 47.9 -> 42.2, g [8192, 14336] 96.3 -> 90.1, [54672, 4096] 194 -> 165);
  // 512 lanes fall in between.
  return run_q<QCfg<128, 256, 1024, 3>>(x, rows, cols, rows_valid, scale_inv, q, q_t, amax,
                                        e5m2, s);
}

}  // namespace fp8lin
