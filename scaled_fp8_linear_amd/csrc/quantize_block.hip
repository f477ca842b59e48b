// Block-recipe quantize: per-tile current scaling in one pass over x.
//
// The block recipe (TransformerEngine "recipe=block", named in NeMo PR 15754)
// scales activations and gradients per 1x128 tile along the GEMM contraction
// index and weights per 128x128 tile. Each tile's scale follows AstrAI's
// _update_delayed_scale applied to the tile's own amax, with no delay:
// scale = max(tile_amax, 1e-12)/448, multiplier 448/max(tile_amax, 1e-12).
//
// A workgroup owns a 128x128 tile of x (256 lanes, each an 8x8 block:
// 8 consecutive rows x 8 columns with 16-byte loads):
//  * 1x128 mode: q uses one scale per tile ROW (reduced over the 16 lanes
//    that share a row); the transposed copy q_t is quantized AGAIN with one
//    scale per tile COLUMN (1x128 along the rows of x, i.e. along the token
//    index that wgrad contracts over), reduced over the 16 row groups;
//  * 128x128 mode: one scale for the whole tile; q_t is q transposed.
// The transposed codes go through LDS (4-row dword pieces, XOR-swizzled) and
// leave with 16-byte stores, as in the tensorwise pass; as there, the loads and
// the q stores stream (non-temporal) and the q_t stores take the cached path.
#include "common.h"
#include "launch.h"

namespace fp8lin {

namespace {

constexpr int kBT = 128;                 // tile edge
constexpr int kBThreads = 256;
static_assert(kBThreads == 2 * kBT, "one lane per tile row and one per tile column");
constexpr int kBColDwords = kBT / 4;     // 32 dwords per transposed column

__device__ __forceinline__ int bslot(int c, int i) {
  return c * kBColDwords + (i ^ ((c >> 3) & (kBColDwords - 1)));
}

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// 4 rows x 4 codes (one dword per row) -> 4 column dwords (rows 0..3 in bytes 0..3).
__device__ __forceinline__ void transpose4x4(const uint32_t w0, const uint32_t w1,
                                             const uint32_t w2, const uint32_t w3, uint32_t* c) {
  uint32_t a01 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);
  uint32_t b01 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);
  uint32_t a23 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
  uint32_t b23 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
  c[0] = __builtin_amdgcn_perm(a23, a01, 0x05040100u);
  c[1] = __builtin_amdgcn_perm(a23, a01, 0x07060302u);
  c[2] = __builtin_amdgcn_perm(b23, b01, 0x05040100u);
  c[3] = __builtin_amdgcn_perm(b23, b01, 0x07060302u);
}

__device__ __forceinline__ uint32_t codes4(uint32_t d0, uint32_t d1, float s0, float s1, float s2,
                                           float s3) {
  return quant4(d0, d1, s0, s1, s2, s3);
}

template <bool W128>
__global__ void __launch_bounds__(kBThreads)
quantize_block_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                      int64_t rows_valid, uint8_t* __restrict__ q, uint8_t* __restrict__ q_t,
                      float* __restrict__ amax_out, float* __restrict__ scale,
                      float* __restrict__ scale_t, int64_t tiles_c) {
  __shared__ uint32_t tile_t[kBT * kBColDwords];      // 16 KiB
  __shared__ uint32_t col_red[4][kBT];                 // per-wave column maxima
  __shared__ uint32_t row_red[kBT];                    // row maxima
  __shared__ float sinv_r[kBT], sinv_c[kBT];           // row and column multipliers
  __shared__ uint32_t tile_red[4];

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
  const int64_t row0 = tr * kBT, col0 = tc * kBT;
  const int cc = t & 15;       // 8-column chunk
  const int rg = t >> 4;       // 8-row group (0..15)
  const int64_t col = col0 + 8 * cc;
  const int64_t kblocks = cols / kBT, rblocks = rows / kBT;

  uint4 v[8];
  bool ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = row0 + 8 * rg + i;
    ok[i] = r < rows_valid;
    v[i] = ok[i] ? ld_stream16(x + r * cols + col) : make_uint4(0, 0, 0, 0);
  }

  // ---- per-row maxima (row tiles), per-column maxima (column tiles): maxima of the 15-bit
  // magnitudes, two columns at a time (packed 16-bit max over the 4 dwords of a row)
  uint32_t rmax[8];
  us2 cm[4] = {us2{0, 0}, us2{0, 0}, us2{0, 0}, us2{0, 0}};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const us2 a = __builtin_bit_cast(us2, v[i].x & 0x7FFF7FFFu);
    const us2 b = __builtin_bit_cast(us2, v[i].y & 0x7FFF7FFFu);
    const us2 c = __builtin_bit_cast(us2, v[i].z & 0x7FFF7FFFu);
    const us2 d = __builtin_bit_cast(us2, v[i].w & 0x7FFF7FFFu);
    cm[0] = __builtin_elementwise_max(cm[0], a);
    cm[1] = __builtin_elementwise_max(cm[1], b);
    cm[2] = __builtin_elementwise_max(cm[2], c);
    cm[3] = __builtin_elementwise_max(cm[3], d);
    const us2 r = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                            __builtin_elementwise_max(c, d));
    rmax[i] = max((uint32_t)r[0], (uint32_t)r[1]);
  }
  uint32_t cmax[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cmax[2 * j] = cm[j][0];
    cmax[2 * j + 1] = cm[j][1];
  }

  float rs_inv[8], cs_inv[8];
  if (!W128) {
    // rows: reduce over the 16 lanes with the same rg (lane bits 0..3)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)rmax[i], off, 64);
        rmax[i] = max(rmax[i], o);
      }
    }
    // columns: reduce over rg within the wave (lane bits 4, 5), then across waves
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t o = (uint32_t)__shfl_xor((int)cmax[j], 16, 64);
      cmax[j] = max(cmax[j], o);
      o = (uint32_t)__shfl_xor((int)cmax[j], 32, 64);
      cmax[j] = max(cmax[j], o);
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) col_red[wave][8 * cc + j] = cmax[j];
    }
    if (cc == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) row_red[8 * rg + i] = rmax[i];
    }
    __syncthreads();
    // each scale once: lane t < 128 takes tile row t, lane 128 + c tile column c (rows and
    // columns of a block tile are whole: both are multiples of 128)
    if (t < kBT) {
      const uint32_t m = row_red[t];
      float s, si;
      scale_pair(__uint_as_float(m << 16), &s, &si);
      sinv_r[t] = si;
      const int64_t r = row0 + t;
      if (scale) scale[r * kblocks + tc] = s;
      if (amax_out) amax_out[r * kblocks + tc] = __uint_as_float(m << 16);
    } else {
      const int c = t - kBT;
      const uint32_t m = max(max(col_red[0][c], col_red[1][c]), max(col_red[2][c], col_red[3][c]));
      float s, si;
      scale_pair(__uint_as_float(m << 16), &s, &si);
      sinv_c[c] = si;
      if (scale_t) scale_t[(col0 + c) * rblocks + tr] = s;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) rs_inv[i] = sinv_r[8 * rg + i];
#pragma unroll
    for (int j = 0; j < 8; ++j) cs_inv[j] = sinv_c[8 * cc + j];
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, rmax[i]);
    m = wave_max_u32(m);
    if (lane == 0) tile_red[wave] = m;
    __syncthreads();
    m = max(max(tile_red[0], tile_red[1]), max(tile_red[2], tile_red[3]));
    float s, si;
    scale_pair(__uint_as_float(m << 16), &s, &si);
#pragma unroll
    for (int i = 0; i < 8; ++i) { rs_inv[i] = si; cs_inv[i] = si; }
    if (t == 0) {
      if (scale) scale[tr * kblocks + tc] = s;
      if (scale_t) scale_t[tc * rblocks + tr] = s;
      if (amax_out) amax_out[tr * kblocks + tc] = __uint_as_float(m << 16);
    }
  }

  // ---- q: row scales
  if (q != nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = row0 + 8 * rg + i;
      const float s = rs_inv[i];
      uint32_t lo = codes4(v[i].x, v[i].y, s, s, s, s);
      uint32_t hi = codes4(v[i].z, v[i].w, s, s, s, s);
      if (!ok[i]) { lo = 0u; hi = 0u; }
      if (r < rows) st_stream8(q + r * cols + col, lo, hi);
    }
  }
  if (q_t == nullptr) return;

  // ---- q_t: column scales (equal to the tile scale in 128x128 mode)
  uint32_t lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    lo[i] = codes4(v[i].x, v[i].y, cs_inv[0], cs_inv[1], cs_inv[2], cs_inv[3]);
    hi[i] = codes4(v[i].z, v[i].w, cs_inv[4], cs_inv[5], cs_inv[6], cs_inv[7]);
    if (!ok[i]) { lo[i] = 0u; hi[i] = 0u; }
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t* w = half ? hi : lo;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {        // rows 0..3 and 4..7 of the 8x8 block
      uint32_t c4[4];
      transpose4x4(w[4 * rb + 0], w[4 * rb + 1], w[4 * rb + 2], w[4 * rb + 3], c4);
      const int di = 2 * rg + rb;           // dword index of these 4 rows
#pragma unroll
      for (int j = 0; j < 4; ++j) tile_t[bslot(8 * cc + 4 * half + j, di)] = c4[j];
    }
  }
  __syncthreads();
  constexpr int kChunks = kBT / 16;                 // 16-row chunks per column
  constexpr int kItems = kBT * kChunks;             // 1024
#pragma unroll
  for (int it = 0; it < kItems / kBThreads; ++it) {
    const int idx = it * kBThreads + t;
    const int c = idx / kChunks, ch = idx % kChunks;
    const int64_t gc = col0 + c, gr = row0 + 16 * ch;
    uint4 o;
    o.x = tile_t[bslot(c, 4 * ch + 0)];
    o.y = tile_t[bslot(c, 4 * ch + 1)];
    o.z = tile_t[bslot(c, 4 * ch + 2)];
    o.w = tile_t[bslot(c, 4 * ch + 3)];
    *reinterpret_cast<uint4*>(q_t + gc * rows + gr) = o;
  }
}

template <bool W128>
hipError_t launch_block(const uint16_t* x, int64_t rows, int64_t cols, int64_t rows_valid,
                        uint8_t* q, uint8_t* q_t, float* amax, float* scale, float* scale_t,
                        hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t tiles_c = cols / kBT;
  const int64_t tiles = (rows / kBT) * tiles_c;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_block_kernel<W128>, dim3((unsigned)tiles), dim3(kBThreads), 0, s, x,
                     rows, cols, rows_valid, q, q_t, amax, scale, scale_t, tiles_c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_block_1x128(const uint16_t* x, int64_t rows, int64_t cols,
                                       int64_t rows_valid, uint8_t* q, uint8_t* q_t,
                                       float* amax, float* scale, float* scale_t, hipStream_t s) {
  return launch_block<false>(x, rows, cols, rows_valid, q, q_t, amax, scale, scale_t, s);
}

hipError_t launch_quantize_block_128x128(const uint16_t* x, int64_t rows, int64_t cols,
                                         uint8_t* q, uint8_t* q_t, float* amax, float* scale,
                                         float* scale_t, hipStream_t s) {
  return launch_block<true>(x, rows, cols, rows, q, q_t, amax, scale, scale_t, s);
}

}  // namespace fp8lin
