// Current-scaling forward of a small linear in one launch.
//
// Dynamic (current) tensorwise scaling, as torchao's Float8Linear does it (SpecForge PR 2,
// Modifications): amax of x and of W, scale = max(amax, 1e-12)/448 and multiplier
// 448/max(amax, 1e-12) for each (AstrAI _update_delayed_scale with no delay), the casts,
// then y = bf16(sx sw Qx Qw^T). Done as separate passes, a small linear is a chain of
// launches whose overheads dwarf its arithmetic (the NeMo PR 15754 thread: on very small
// matmuls the scaling costs more than FP8 gains). Here one launch does all of it: the
// operands' codes stay in LDS between the cast and the matrix instruction.
//
// One workgroup of 256 lanes (4 waves) per 16x16 tile of y. Each workgroup:
//  1. loads its own 32 code rows (16 of x, 16 of W), up to kLocal 16-byte pieces per lane,
//     then the amax of the whole of x and of W over 16-byte pieces (exact: a max of the
//     15-bit magnitudes of the bf16 patterns, NaN above infinity), reduced by wave shuffles
//     and LDS. Every workgroup computes the same amaxes; after the first, the pieces come
//     from the cache. With no exchange between workgroups there is nothing to wait for;
//  2. lanes 0 and 1 turn the two amaxes into scales and multipliers (workgroup 0 also
//     writes them out);
//  3. casts its 32 rows into LDS in the fragment layout of the 16x16x128 FP8 matrix
//     instruction (and to qx, qw when asked for: x rows by the tiles of the first tile
//     column, W rows by those of the first tile row, so each code is written once). Pieces
//     past kLocal per lane are read again, kBatch per lane and step;
//  4. wave 0 runs one matrix instruction per 128 K bytes and stores the tile scaled by
//     sx sw (one float32 product), rounded to bf16.
// Against one workgroup for the whole linear, this spreads the casts and the matrix work
// over (M/16)(N/16) compute units at the price of reading the inputs once per tile.
#include "common.h"
#include "launch.h"

namespace fp8lin {

namespace {

constexpr int kLThreads = 256;
constexpr int kLStep = 128;              // K bytes per matrix instruction
constexpr int kBatch = 8;                // 16-byte pieces per lane and step of a pass
constexpr int kAll = 16;                 // amax pieces per lane loaded at once (ALL)
constexpr int kLocal = 4;                // own pieces per lane loaded before the amax pass
constexpr int kTileRows = 32;            // code rows of a tile: 16 of x, then 16 of W

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// LDS layout of a tile's codes: K step ks (128 K bytes), row r (0..15 x, 16..31 W) at
// (ks 32 + r) 128; 16-byte chunk c of the row at chunk c ^ swz(r), which spreads the 16
// rows a fragment read touches over the banks.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 5; }

__device__ __forceinline__ uint32_t mag_max8(uint4 v) {
  const us2 a = __builtin_bit_cast(us2, v.x & 0x7FFF7FFFu);
  const us2 b = __builtin_bit_cast(us2, v.y & 0x7FFF7FFFu);
  const us2 c = __builtin_bit_cast(us2, v.z & 0x7FFF7FFFu);
  const us2 d = __builtin_bit_cast(us2, v.w & 0x7FFF7FFFu);
  const us2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                          __builtin_elementwise_max(c, d));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}

// ALL: the amax pass issues all of a lane's loads (at most kAll) before using any;
// otherwise kBatch per step.
template <bool ALL>
__global__ void __launch_bounds__(kLThreads)
linear_current_small_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                            int M, int N, int K, uint16_t* __restrict__ y,
                            float* __restrict__ scales, uint8_t* __restrict__ qx,
                            uint8_t* __restrict__ qw) {
  // a tile's 32 K bytes of codes; M + N >= 32, so 32 K <= (M + N) K <= kSmallLinearCodes
  __shared__ __attribute__((aligned(16))) uint8_t codes[kSmallLinearCodes];
  __shared__ uint32_t red[2][kLThreads / 64];
  __shared__ float sc[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int kc = K / 8;                  // 16-byte pieces (8 values) per row
  const int pieces = (M + N) * kc;       // of the whole input: rows of x, then rows of W
  const int tn = N / 16;
  const int m0 = (blockIdx.x / tn) * 16, n0 = (blockIdx.x % tn) * 16;
  const int own = kTileRows * kc;        // pieces of the tile's own rows
  auto piece = [&](int id) -> uint4 {
    const int r = id / kc, c = id - r * kc;
    const uint16_t* p = r < M ? x + (int64_t)r * K : w + (int64_t)(r - M) * K;
    return *reinterpret_cast<const uint4*>(p + 8 * c);
  };
  auto own_piece = [&](int id) -> uint4 {
    const int r = id / kc, c = id - r * kc;
    const uint16_t* p = r < 16 ? x + (int64_t)(m0 + r) * K : w + (int64_t)(n0 + r - 16) * K;
    return *reinterpret_cast<const uint4*>(p + 8 * c);
  };

  uint4 loc[kLocal];
#pragma unroll
  for (int u = 0; u < kLocal; ++u) {
    const int id = t + u * kLThreads;
    loc[u] = id < own ? own_piece(id) : make_uint4(0u, 0u, 0u, 0u);
  }
  // 1. amaxes. A lane's pieces are ids t, t + 256, ..
  uint32_t mx = 0, mw = 0;
  auto fold_max = [&](const uint4& v, int id) {
    const uint32_t m = mag_max8(v);
    if (id < M * kc) mx = max(mx, m);
    else mw = max(mw, m);
  };
  if constexpr (ALL) {
    uint4 v[kAll];
#pragma unroll
    for (int u = 0; u < kAll; ++u) {
      const int id = t + u * kLThreads;
      v[u] = id < pieces ? piece(id) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kAll; ++u) {
      const int id = t + u * kLThreads;
      if (id < pieces) fold_max(v[u], id);
    }
  } else {
    for (int id0 = t; id0 < pieces; id0 += kLThreads * kBatch) {
      uint4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int id = id0 + u * kLThreads;
        if (id < pieces) v[u] = piece(id);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (id0 + u * kLThreads < pieces) fold_max(v[u], id0 + u * kLThreads);
    }
  }
  mx = wave_max_u32(mx);
  mw = wave_max_u32(mw);
  if (lane == 0) {
    red[0][wave] = mx;
    red[1][wave] = mw;
  }
  __syncthreads();
  // 2. scales {sx, sw} and multipliers {sx_inv, sw_inv}
  if (t < 2) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < kLThreads / 64; ++i) m = max(m, red[t][i]);
    float s, si;
    scale_pair(__uint_as_float(m << 16), &s, &si);
    sc[t] = s;
    sc[2 + t] = si;
    if (blockIdx.x == 0) {
      scales[t] = s;
      scales[2 + t] = si;
    }
  }
  __syncthreads();
  // 3. casts of the tile's own rows
  const float mulx = sc[2], mulw = sc[3];
  uint8_t* const qxt = n0 == 0 ? qx : nullptr;
  uint8_t* const qwt = m0 == 0 ? qw : nullptr;
  auto cast = [&](const uint4& v, int id) {
    const int r = id / kc, c = id - r * kc;
    const bool isx = r < 16;
    const float s = isx ? mulx : mulw;
    const uint32_t lo = quant4(v.x, v.y, s, s, s, s), hi = quant4(v.z, v.w, s, s, s, s);
    const int ks = c / (kLStep / 8), cw = c % (kLStep / 8);   // 8-byte piece cw of step ks
    const int at = (ks * kTileRows + r) * kLStep + 16 * ((cw >> 1) ^ swz(r)) + 8 * (cw & 1);
    *reinterpret_cast<uint2*>(codes + at) = make_uint2(lo, hi);
    uint8_t* const q = isx ? qxt : qwt;
    if (q != nullptr)
      *reinterpret_cast<uint2*>(q + (int64_t)(isx ? m0 + r : n0 + r - 16) * K + 8 * c) =
          make_uint2(lo, hi);
  };
#pragma unroll
  for (int u = 0; u < kLocal; ++u) {
    const int id = t + u * kLThreads;
    if (id < own) cast(loc[u], id);
  }
  for (int id0 = t + kLocal * kLThreads; id0 < own; id0 += kLThreads * kBatch) {
    uint4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int id = id0 + u * kLThreads;
      if (id < own) v[u] = own_piece(id);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (id0 + u * kLThreads < own) cast(v[u], id0 + u * kLThreads);
  }
  __syncthreads();
  // 4. the tile: lane (r16, g) reads chunks 2 g, 2 g + 1 of row r16 of x's and of W's rows;
  // with W as the first operand its 4 results are columns 4 g .. 4 g + 3 of row r16.
  if (wave != 0) return;
  const int r16 = lane & 15, g = lane >> 4;
  auto frag = [&](int ks, int row) {
    const uint8_t* base = codes + (ks * kTileRows + row) * kLStep;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + 16 * ((2 * g) ^ swz(row)));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + 16 * ((2 * g + 1) ^ swz(row)));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
               (int)hi.w};
  };
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int ks = 0; ks < K / kLStep; ++ks)
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(frag(ks, 16 + r16), frag(ks, r16),
                                                           acc, 0, 0, 0, 0, 0, 0);
  const float scl = sc[0] * sc[1];
  const uint32_t p0 = pack_bf16x2(acc[0] * scl, acc[1] * scl);
  const uint32_t p1 = pack_bf16x2(acc[2] * scl, acc[3] * scl);
  *reinterpret_cast<uint2*>(y + (int64_t)(m0 + r16) * N + n0 + 4 * g) = make_uint2(p0, p1);
}

}  // namespace

hipError_t launch_linear_current_small(const uint16_t* x, const uint16_t* w, int M, int N, int K,
                                       uint16_t* y, float* scales, uint8_t* qx, uint8_t* qw,
                                       hipStream_t s) {
  const unsigned tiles = (unsigned)((M / 16) * (N / 16));
  if ((M + N) * (K / 8) <= kAll * kLThreads)
    hipLaunchKernelGGL(linear_current_small_kernel<true>, dim3(tiles), dim3(kLThreads), 0, s, x,
                       w, M, N, K, y, scales, qx, qw);
  else
    hipLaunchKernelGGL(linear_current_small_kernel<false>, dim3(tiles), dim3(kLThreads), 0, s, x,
                       w, M, N, K, y, scales, qx, qw);
  return hipGetLastError();
}

}  // namespace fp8lin
