// Current-scaling forward of a small linear in one launch.
//
// Dynamic (current) tensorwise scaling, as torchao's Float8Linear does it (SpecForge PR 2,
// Modifications): amax of x and of W, scale = max(amax, 1e-12)/448 and multiplier
// 448/max(amax, 1e-12) for each (AstrAI _update_delayed_scale with no delay), the casts,
// then y = bf16(sx sw Qx Qw^T). Done as separate passes, a small linear is a chain of
// launches whose overheads dwarf its arithmetic (the NeMo PR 15754 thread: on very small
// matmuls the scaling costs more than FP8 gains). Here one workgroup does all of it: the
// operands' codes stay in LDS between the cast and the matrix instructions.
//
// One workgroup of 256 lanes (4 waves):
//  1. amax of x and of W over 16-byte pieces (exact: a max of the 15-bit magnitudes of
//     the bf16 patterns, NaN above infinity), reduced by wave shuffles and LDS;
//  2. lanes 0 and 1 turn the two amaxes into scales and multipliers;
//  3. the casts, written to LDS in the fragment layout of the 16x16x128 FP8 matrix
//     instruction (and to qx, qw when asked for). Up to 16 pieces per lane stay in
//     registers from step 1; more are read again from memory (from the cache the first
//     pass filled), 8 per lane and step with the loads issued before any is used;
//  4. the GEMM: each wave takes work items in turn, a 16-row tile of y and 4 of its
//     16-column tiles, one MFMA per tile and 128 K bytes, and stores its 4 results per lane
//     and tile scaled by sx sw (one float32 product) and rounded to bf16.
#include "common.h"
#include "launch.h"

namespace fp8lin {

namespace {

constexpr int kLThreads = 256;
constexpr int kLStep = 128;              // K bytes per matrix instruction
constexpr int kBatch = 8;                // 16-byte pieces per lane and step of a pass
constexpr int kKeep = 16;                // pieces per lane held in registers (KEEP)
constexpr int kGroup = 4;                // 16-column tiles per GEMM work item

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// LDS layout of the codes: K step ks (128 K bytes), code row r (x rows 0..M-1, then W
// rows M..M+N-1) at (ks (M + N) + r) 128; 16-byte chunk c of the row at chunk
// c ^ swz(r), which spreads the 16 rows a fragment read touches over the banks (M is a
// multiple of 16, so a row's swizzle depends on its index within its 16-row tile only).
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

// KEEP: every lane holds its pieces (at most kKeep) in registers from the amax pass to the
// casts; otherwise the casts read them again (from the cache the first pass filled).
template <bool KEEP>
__global__ void __launch_bounds__(kLThreads)
linear_current_small_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                            int M, int N, int K, uint16_t* __restrict__ y,
                            float* __restrict__ scales, uint8_t* __restrict__ qx,
                            uint8_t* __restrict__ qw) {
  __shared__ __attribute__((aligned(16))) uint8_t codes[kSmallLinearCodes];
  __shared__ uint32_t red[2][kLThreads / 64];
  __shared__ float sc[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int R = M + N;
  const int kc = K / 8;                  // 16-byte pieces (8 values) per row
  const int pieces = R * kc;
  auto piece = [&](int id, int& r, int& c) -> uint4 {
    r = id / kc;
    c = id - r * kc;
    const uint16_t* p = r < M ? x + (int64_t)r * K : w + (int64_t)(r - M) * K;
    return *reinterpret_cast<const uint4*>(p + 8 * c);
  };

  // 1. amaxes. A lane's pieces are ids t, t + 256, ..; kBatch of them per step (all loads
  // issued before any is used), or with KEEP all of them at once.
  uint32_t mx = 0, mw = 0;
  uint4 held[KEEP ? kKeep : 1];
  auto fold_max = [&](const uint4& v, int r) {
    const uint32_t m = mag_max8(v);
    if (r < M) mx = max(mx, m);
    else mw = max(mw, m);
  };
  if constexpr (KEEP) {
#pragma unroll
    for (int u = 0; u < kKeep; ++u) {
      const int id = t + u * kLThreads;
      int r, c;
      held[u] = id < pieces ? piece(id, r, c) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kKeep; ++u) {
      const int id = t + u * kLThreads;
      if (id < pieces) fold_max(held[u], id / kc);
    }
  } else {
    for (int id0 = t; id0 < pieces; id0 += kLThreads * kBatch) {
      uint4 v[kBatch];
      int r[kBatch], c[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int id = id0 + u * kLThreads;
        if (id < pieces) v[u] = piece(id, r[u], c[u]);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (id0 + u * kLThreads < pieces) fold_max(v[u], r[u]);
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
    scales[t] = s;
    scales[2 + t] = si;
  }
  __syncthreads();
  // 3. casts
  const float mulx = sc[2], mulw = sc[3];
  auto cast = [&](const uint4& v, int r, int c) {
    const bool isx = r < M;
    const float s = isx ? mulx : mulw;
    const uint32_t lo = quant4(v.x, v.y, s, s, s, s), hi = quant4(v.z, v.w, s, s, s, s);
    const int ks = c / (kLStep / 8), cw = c % (kLStep / 8);   // 8-byte piece cw of step ks
    const int at = (ks * R + r) * kLStep + 16 * ((cw >> 1) ^ swz(r)) + 8 * (cw & 1);
    *reinterpret_cast<uint2*>(codes + at) = make_uint2(lo, hi);
    uint8_t* q = isx ? qx : qw;
    if (q != nullptr)
      *reinterpret_cast<uint2*>(q + (int64_t)(isx ? r : r - M) * K + 8 * c) = make_uint2(lo, hi);
  };
  if constexpr (KEEP) {
#pragma unroll
    for (int u = 0; u < kKeep; ++u) {
      const int id = t + u * kLThreads;
      if (id < pieces) cast(held[u], id / kc, id % kc);
    }
  } else {
    for (int id0 = t; id0 < pieces; id0 += kLThreads * kBatch) {
      uint4 v[kBatch];
      int r[kBatch], c[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int id = id0 + u * kLThreads;
        if (id < pieces) v[u] = piece(id, r[u], c[u]);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (id0 + u * kLThreads < pieces) cast(v[u], r[u], c[u]);
    }
  }
  __syncthreads();
  // 4. GEMM: lane (r16, g) reads chunks 2 g, 2 g + 1 of row r16 of a 16-row tile; with W
  // as the first operand its 4 results are columns 4 g .. 4 g + 3 of row r16. A work item
  // is one 16-row tile of y and kGroup of its 16-column tiles: per K step the A fragment
  // is read once, the B fragments together, and the kGroup matrix instructions run back
  // to back; the waves take the items in turn.
  const int r16 = lane & 15, g = lane >> 4;
  const float scl = sc[0] * sc[1];
  const int tm = M / 16, tn = N / 16, steps = K / kLStep;
  const int groups = (tn + kGroup - 1) / kGroup, items = tm * groups;
  auto frag = [&](int ks, int row) {
    const uint8_t* base = codes + (ks * R + row) * kLStep;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + 16 * ((2 * g) ^ swz(row)));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + 16 * ((2 * g + 1) ^ swz(row)));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
               (int)hi.w};
  };
  for (int it = wave; it < items; it += kLThreads / 64) {
    const int m0 = (it / groups) * 16, nt0 = (it % groups) * kGroup;
    v4f acc[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < steps; ++ks) {
      const v8i a = frag(ks, m0 + r16);
      v8i b[kGroup];
#pragma unroll
      for (int u = 0; u < kGroup; ++u)
        if (nt0 + u < tn) b[u] = frag(ks, M + 16 * (nt0 + u) + r16);
#pragma unroll
      for (int u = 0; u < kGroup; ++u)
        if (nt0 + u < tn)
          acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[u], a, acc[u], 0, 0, 0, 0,
                                                                    0, 0);
    }
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      if (nt0 + u >= tn) break;
      const int n0 = 16 * (nt0 + u);
      const uint32_t p0 = pack_bf16x2(acc[u][0] * scl, acc[u][1] * scl);
      const uint32_t p1 = pack_bf16x2(acc[u][2] * scl, acc[u][3] * scl);
      *reinterpret_cast<uint2*>(y + (int64_t)(m0 + r16) * N + n0 + 4 * g) = make_uint2(p0, p1);
    }
  }
}

}  // namespace

hipError_t launch_linear_current_small(const uint16_t* x, const uint16_t* w, int M, int N, int K,
                                       uint16_t* y, float* scales, uint8_t* qx, uint8_t* qw,
                                       hipStream_t s) {
  if ((M + N) * (K / 8) <= kKeep * kLThreads)
    hipLaunchKernelGGL(linear_current_small_kernel<true>, dim3(1), dim3(kLThreads), 0, s, x, w, M,
                       N, K, y, scales, qx, qw);
  else
    hipLaunchKernelGGL(linear_current_small_kernel<false>, dim3(1), dim3(kLThreads), 0, s, x, w, M,
                       N, K, y, scales, qx, qw);
  return hipGetLastError();
}

}  // namespace fp8lin
