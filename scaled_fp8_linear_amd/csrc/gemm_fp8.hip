// Scaled FP8 GEMM on the gfx950 matrix cores.
//
// What it computes (AstrAI, astrai/extension/fp8_state.py, module comment:
// "D = A_SCALE * B_SCALE * A * B" with per-tensor scales amax/448): e4m3
// operands multiplied as they are, float32 accumulation, and the scales
// folded in after accumulation:
//
//     D[m, n] = bf16_rne( (sa * sb) * sum_k A[m, k] * B[n, k] )
//
// Both operands keep the contraction index last. The layer's three GEMMs are
// all of this form because the quantize pass also writes transposed copies:
// forward (Qx, Qw), dgrad (Qg, Qw^T), wgrad (Qg^T, Qx^T).
//
// Block recipe (TE "recipe=block", NeMo PR 15754): the scales multiply each
// 128-wide partial sum, D = sum_kb sa[m,kb] * sb[n/b_rows, kb] * S_kb.
//
// Kernel design:
//  * macro tile BM x BN, contraction step BK = 128 bytes (= one block-scale
//    block), one barrier per step, two LDS stages (global loads for step
//    k+1 are in flight while step k is multiplied);
//  * each wavefront owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 output
//    tiles, computed with v_mfma_f32_32x32x64_f8f6f4 (OCP e4m3 x e4m3 ->
//    float32). The B fragment is given as the instruction's first operand,
//    so every lane ends up holding 4 consecutive n of one row m and the
//    epilogue writes 8-byte runs of bf16;
//  * the MFMA pairs A and B by lane and byte position, so any ordering of k
//    inside a 64-wide step is valid as long as A and B use the same one: each
//    lane takes 32 contiguous k (two 16-byte LDS reads);
//  * LDS rows are 128 bytes; 16-byte chunks are XOR-swizzled by the row so
//    that the 16-byte fragment reads of consecutive rows hit distinct banks;
//  * workgroups are dispatched round-robin over the 8 XCDs; the block index
//    is remapped so each XCD gets a contiguous range of tiles, walked in
//    groups of GROUP_M row tiles so that concurrently running tiles share A
//    and B panels in that XCD's L2.
#include <stdlib.h>

#include "common.h"
#include "launch.h"

namespace fp8lin {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;

template <int BM_, int BN_, int WM_, int WN_, int SWZ_, int GROUP_M_, bool BLOCK_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, SWZ = SWZ_, GROUP_M = GROUP_M_;
  static constexpr bool BLOCK = BLOCK_;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int kStageBytes = (BM + BN) * kBK;
  static constexpr int kLoadsA = BM * kBK / (kThreads * 16);
  static constexpr int kLoadsB = BN * kBK / (kThreads * 16);
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BM * kBK % (kThreads * 16) == 0 && BN * kBK % (kThreads * 16) == 0, "loads");
};

template <int SWZ>
__device__ __forceinline__ int swz_chunk(int row, int chunk) {
  return chunk ^ (SWZ == 0 ? (row & 7) : ((row >> 1) & 7));
}

// logical tile index -> (tile_m, tile_n), XCD-contiguous and grouped.
template <int GROUP_M>
__device__ __forceinline__ void tile_of(int bid, int nwg, int tiles_m, int tiles_n, int& tm,
                                        int& tn) {
  int lid = bid;
  if ((nwg & 7) == 0) lid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int per_group = GROUP_M * tiles_n;
  const int group = lid / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = lid - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

template <class C>
__global__ void __launch_bounds__(C::kThreads)
gemm_fp8_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                const float* __restrict__ sa, const float* __restrict__ sb,
                uint16_t* __restrict__ D, int M, int N, int K, int M_valid, int tiles_m,
                int tiles_n, int b_rows_per_scale) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::kStageBytes];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  int tm, tn;
  tile_of<C::GROUP_M>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  // ---- global -> register loads of one K step
  const int ld_chunk = t & 7;          // 16-byte chunk within a 128-byte row
  const int ld_row = t >> 3;           // first row handled by this lane
  constexpr int kRowsPerPass = C::kThreads / 8;
  uint4 ra[C::kLoadsA], rb[C::kLoadsB];

  auto load_step = [&](int k0) {
    const int kk = k0 + 16 * ld_chunk;
    const bool k_ok = kk < K;
#pragma unroll
    for (int i = 0; i < C::kLoadsA; ++i) {
      const int r = m0 + ld_row + i * kRowsPerPass;
      ra[i] = (k_ok && r < M) ? *reinterpret_cast<const uint4*>(A + (int64_t)r * K + kk)
                              : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::kLoadsB; ++i) {
      const int r = n0 + ld_row + i * kRowsPerPass;
      rb[i] = (k_ok && r < N) ? *reinterpret_cast<const uint4*>(B + (int64_t)r * K + kk)
                              : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_step = [&](int stage) {
    uint8_t* sA = smem + stage * C::kStageBytes;
    uint8_t* sB = sA + C::BM * kBK;
#pragma unroll
    for (int i = 0; i < C::kLoadsA; ++i) {
      const int r = ld_row + i * kRowsPerPass;
      *reinterpret_cast<uint4*>(sA + r * kBK + 16 * swz_chunk<C::SWZ>(r, ld_chunk)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::kLoadsB; ++i) {
      const int r = ld_row + i * kRowsPerPass;
      *reinterpret_cast<uint4*>(sB + r * kBK + 16 * swz_chunk<C::SWZ>(r, ld_chunk)) = rb[i];
    }
  };

  v16f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int fr = lane & 31;            // fragment row within a 32-row tile
  const int fg = lane >> 5;            // which 32-byte half of a 64-wide k step

  auto frag = [&](const uint8_t* s, int row, int h) -> v8i {
    const int c0 = 4 * h + 2 * fg;
    const uint4 lo = *reinterpret_cast<const uint4*>(s + row * kBK + 16 * swz_chunk<C::SWZ>(row, c0));
    const uint4 hi =
        *reinterpret_cast<const uint4*>(s + row * kBK + 16 * swz_chunk<C::SWZ>(row, c0 + 1));
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };

  const int nk = (K + kBK - 1) / kBK;
  load_step(0);
  store_step(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_step((kt + 1) * kBK);
    const uint8_t* sA = smem + (kt & 1) * C::kStageBytes;
    const uint8_t* sB = sA + C::BM * kBK;

    if constexpr (!C::BLOCK) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v8i af[C::TM], bf[C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i) af[i] = frag(sA, wm * C::WTM + 32 * i + fr, h);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) bf[j] = frag(sB, wn * C::WTN + 32 * j + fr, h);
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af[i], acc[i][j], 0,
                                                                          0, 0, 0, 0, 0);
      }
    } else {
      // Block recipe: per-128 partial sums, scaled and accumulated in float32.
      const int kb = kt;
      const int kblocks = (K + kBK - 1) / kBK;
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        v16f part[C::TN];
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) part[j][r] = 0.0f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v8i af = frag(sA, wm * C::WTM + 32 * i + fr, h);
#pragma unroll
          for (int j = 0; j < C::TN; ++j) {
            const v8i bfj = frag(sB, wn * C::WTN + 32 * j + fr, h);
            part[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfj, af, part[j], 0, 0, 0, 0,
                                                                      0, 0);
          }
        }
        const int m = m0 + wm * C::WTM + 32 * i + fr;
        const float s_a = (m < M) ? sa[(int64_t)m * kblocks + kb] : 0.0f;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int n = n0 + wn * C::WTN + 32 * j + 8 * (r >> 2) + 4 * fg + (r & 3);
            const float s_b = (n < N) ? sb[(int64_t)(n / b_rows_per_scale) * kblocks + kb] : 0.0f;
            acc[i][j][r] = fmaf(part[j][r], s_a * s_b, acc[i][j][r]);
          }
        }
      }
    }

    if (kt + 1 < nk) store_step((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: scale, round to bf16, write 4 consecutive n per lane
  const float s = C::BLOCK ? 1.0f : sa[0] * sb[0];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int m = m0 + wm * C::WTM + 32 * i + fr;
    if (m >= M) continue;
    const bool live = m < M_valid;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int n = n0 + wn * C::WTN + 32 * j + 8 * rq + 4 * fg;
        if (n >= N) continue;
        uint32_t p0 = 0, p1 = 0;
        if (live) {
          p0 = f32_to_bf16_bits(acc[i][j][4 * rq + 0] * s) |
               (f32_to_bf16_bits(acc[i][j][4 * rq + 1] * s) << 16);
          p1 = f32_to_bf16_bits(acc[i][j][4 * rq + 2] * s) |
               (f32_to_bf16_bits(acc[i][j][4 * rq + 3] * s) << 16);
        }
        *reinterpret_cast<uint2*>(D + (int64_t)m * N + n) = make_uint2(p0, p1);
      }
    }
  }
}

template <class C>
hipError_t run(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb, uint16_t* D,
               int M, int N, int K, int M_valid, int b_rows, hipStream_t s) {
  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  hipLaunchKernelGGL(gemm_fp8_kernel<C>, dim3((unsigned)tiles), dim3(C::kThreads), 0, s, A, B, sa,
                     sb, D, M, N, K, M_valid, tiles_m, tiles_n, b_rows);
  return hipGetLastError();
}

// Tile configurations. The default is chosen per shape; FP8LIN_GEMM_CFG
// (read once) forces one of them for tuning sweeps.
using CfgBig4 = Cfg<256, 256, 2, 2, 0, 8, false>;     // 4 waves, 128x128 per wave
using CfgBig8 = Cfg<256, 256, 2, 4, 0, 8, false>;     // 8 waves, 128x64 per wave
using CfgBig4S = Cfg<256, 256, 2, 2, 1, 8, false>;    // swizzle for 64 banks
using CfgMid = Cfg<128, 128, 2, 2, 0, 8, false>;      // small problems
using CfgBlk = Cfg<128, 128, 2, 2, 0, 8, true>;       // block recipe

int forced_cfg() {
  static int v = [] {
    const char* e = getenv("FP8LIN_GEMM_CFG");
    return e ? atoi(e) : -1;
  }();
  return v;
}

}  // namespace

hipError_t launch_gemm_fp8(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                           uint16_t* D, int64_t M, int64_t N, int64_t K, int64_t M_valid,
                           bool block_scaled, int b_rows_per_scale, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  const int m = (int)M, n = (int)N, k = (int)K, mv = (int)M_valid;
  if (block_scaled) return run<CfgBlk>(A, B, sa, sb, D, m, n, k, mv, b_rows_per_scale, s);
  int cfg = forced_cfg();
  if (cfg < 0) cfg = ((int64_t)M * N >= (int64_t)4096 * 4096) ? 0 : 3;
  switch (cfg) {
    case 1: return run<CfgBig8>(A, B, sa, sb, D, m, n, k, mv, 1, s);
    case 2: return run<CfgBig4S>(A, B, sa, sb, D, m, n, k, mv, 1, s);
    case 3: return run<CfgMid>(A, B, sa, sb, D, m, n, k, mv, 1, s);
    default: return run<CfgBig4>(A, B, sa, sb, D, m, n, k, mv, 1, s);
  }
}

}  // namespace fp8lin
