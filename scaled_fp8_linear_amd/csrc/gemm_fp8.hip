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
          p0 = pack_bf16x2(acc[i][j][4 * rq + 0] * s, acc[i][j][4 * rq + 1] * s);
          p1 = pack_bf16x2(acc[i][j][4 * rq + 2] * s, acc[i][j][4 * rq + 3] * s);
        }
        *reinterpret_cast<uint2*>(D + (int64_t)m * N + n) = make_uint2(p0, p1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tensorwise kernel: direct global->LDS loads into a ring of LDS stages.
//
// * A stage holds BM x 64 bytes of A and BN x 64 bytes of B (one 64-wide K
//   step = one v_mfma_f32_32x32x64_f8f6f4 per 32x32 output tile). Rows are
//   64 bytes = four 16-byte chunks, XOR-swizzled by the row.
// * Operand tiles go from memory straight into LDS with buffer loads carrying
//   the "lds" modifier (no VGPR staging, no ds_write). One wavefront
//   instruction fills 1 KiB = 16 rows; lane l writes LDS bytes [16 l, 16 l+16)
//   of that KiB, so each lane loads the global chunk that belongs there.
// * Rows past M (or N) read as zero through the buffer's size field; a K tail
//   is zeroed by pointing its lanes past the end of the buffer. Steps past the
//   last K step are loaded the same way (all zeros), which keeps the number of
//   loads in flight identical at every step and the loop free of branches.
// * STAGES separate LDS arrays and a K loop unrolled by STAGES keep every LDS
//   address static, so the compiler waits only for the load that fills the
//   stage being read. Per step: wait until this wave's loads for the step have
//   landed, one barrier (all waves' loads landed, and every wave is done with
//   the stage that is refilled next), refill that stage, then multiply.
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit dwords
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBKS = 64;                   // K bytes per stage

typedef int v4i __attribute__((ext_vector_type(4)));

// Buffer resource of a raw byte buffer of `bytes` bytes (reads at or past the end return 0).
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = kRsrcWord3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_ptr)p;
}

// One 16-byte-per-lane buffer load written straight to LDS at lds + 16 * lane. Issued
// through inline asm so that the compiler does not guard later LDS reads of other
// stages with waits on it; the kernel waits for these loads itself (vmcnt) before the
// barrier that publishes a stage.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane((int)lds))
               : "memory", "m0");
}

template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int SWZ_, int GROUP_M_>
struct PCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_, SWZ = SWZ_;
  static constexpr int GROUP_M = GROUP_M_;
  static constexpr int kWaves = WM * WN, kThreads = kWaves * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  static constexpr int kStageBytes = (BM + BN) * kBKS;
  static constexpr int kInstA = BM / (16 * kWaves), kInstB = BN / (16 * kWaves);
  static constexpr int kLoadsPerStage = kInstA + kInstB;
  static_assert(BM % (16 * kWaves) == 0 && BN % (16 * kWaves) == 0, "dma rows");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(STAGES >= 2 && STAGES <= 5, "stages");
  static_assert(kLoadsPerStage * (STAGES - 2) <= 63, "vmcnt range");
};

// 64-byte rows: chunk c (0..3) of row r sits at c ^ f(r).
template <int SWZ>
__device__ __forceinline__ int swz64(int row, int chunk) {
  return chunk ^ (SWZ == 0 ? ((row >> 1) & 3) : ((row >> 2) & 3));
}

template <int S, int STAGES>
__device__ __forceinline__ uint8_t* pick(uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3,
                                         uint8_t* s4) {
  constexpr int i = S % STAGES;
  if constexpr (i == 0) return s0;
  else if constexpr (i == 1) return s1;
  else if constexpr (i == 2) return s2;
  else if constexpr (i == 3) return s3;
  else return s4;
}

template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  // this wave's loads older than the newest N have landed; LDS reads are done
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

template <class C>
__global__ void __launch_bounds__(C::kThreads, 1)
gemm_fp8_pipe_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                     const float* __restrict__ sa, const float* __restrict__ sb,
                     uint16_t* __restrict__ D, int M, int N, int K, int M_valid, int tiles_m,
                     int tiles_n) {
  constexpr int SB = C::kStageBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t s0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[C::STAGES > 2 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[C::STAGES > 3 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t s4[C::STAGES > 4 ? SB : 16];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;

  int tm, tn;
  tile_of<C::GROUP_M>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  const v4i rsA = make_rsrc(A, (uint32_t)(M * K));
  const v4i rsB = make_rsrc(B, (uint32_t)(N * K));

  // Load plan: instruction i of this wave fills rows 16 (W i + wave) .. +16; lane l
  // takes row l / 4 of them and physical chunk l % 4. Row steps between instructions
  // are multiples of 64, so the lane's logical chunk is the same for all of them.
  const int lr = lane >> 2, lp = lane & 3;
  const int r0 = 16 * wave + lr;
  const int ch = swz64<C::SWZ>(r0, lp);
  const uint32_t baseA = (uint32_t)(m0 + r0) * (uint32_t)K + 16u * ch;
  const uint32_t baseB = (uint32_t)(n0 + r0) * (uint32_t)K + 16u * ch;
  const uint32_t step_rows = (uint32_t)(16 * C::kWaves) * (uint32_t)K;

  auto issue = [&](uint8_t* stage, int kstep) {
    const int k0 = kstep * kBKS;
    // offsets stay below 2^31 (operands hold fewer than 2^31 bytes): setting bit 31
    // puts a lane past the end of the buffer, which reads zeros
    const uint32_t oob = (k0 + 16 * ch < K) ? 0u : kOutOfRange;
    const uint32_t lds = lds_addr(stage) + (uint32_t)(16 * wave * kBKS);
#pragma unroll
    for (int i = 0; i < C::kInstA; ++i)
      dma16(rsA, (baseA + i * step_rows + (uint32_t)k0) | oob,
            lds + (uint32_t)(16 * C::kWaves * i * kBKS));
#pragma unroll
    for (int i = 0; i < C::kInstB; ++i)
      dma16(rsB, (baseB + i * step_rows + (uint32_t)k0) | oob,
            lds + (uint32_t)(C::BM * kBKS + 16 * C::kWaves * i * kBKS));
  };

  // fragment of one 32-row tile for a 64-wide K step: lane (fr, fg) holds k bytes
  // [32 fg, 32 fg + 32) of row fr, i.e. chunks 2 fg and 2 fg + 1
  const int fr = lane & 31;
  const int fg = lane >> 5;
  const int c_lo = swz64<C::SWZ>(fr, 2 * fg) * 16;
  const int c_hi = swz64<C::SWZ>(fr, 2 * fg + 1) * 16;
  auto frag = [&](const uint8_t* base, int row) -> v8i {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + row * kBKS + c_lo);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + row * kBKS + c_hi);
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };

  v16f acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute = [&](const uint8_t* stage) {
    const uint8_t* sA = stage + (wm * C::WTM + fr) * kBKS;
    const uint8_t* sB = stage + C::BM * kBKS + (wn * C::WTN + fr) * kBKS;
    v8i b[C::TN];
#pragma unroll
    for (int j = 0; j < C::TN; ++j) b[j] = frag(sB, 32 * j);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const v8i a = frag(sA, 32 * i);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a, acc[i][j], 0, 0, 0,
                                                                    0, 0, 0);
    }
  };

  constexpr int kWaitN = C::kLoadsPerStage * (C::STAGES - 2);
  auto step = [&](uint8_t* cur, uint8_t* refill, int kstep) {
    wait_vm_lgkm<kWaitN>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(refill, kstep + C::STAGES - 1);
    compute(cur);
  };

  const int nk = (K + kBKS - 1) / kBKS;
  // prologue: steps 0 .. STAGES-2 in flight
  issue(s0, 0);
  if constexpr (C::STAGES > 2) issue(s1, 1);
  if constexpr (C::STAGES > 3) issue(s2, 2);
  if constexpr (C::STAGES > 4) issue(s3, 3);
  for (int kt = 0; kt < nk; kt += C::STAGES) {
    step(pick<0, C::STAGES>(s0, s1, s2, s3, s4), pick<C::STAGES - 1, C::STAGES>(s0, s1, s2, s3, s4), kt);
    step(pick<1, C::STAGES>(s0, s1, s2, s3, s4), pick<C::STAGES, C::STAGES>(s0, s1, s2, s3, s4), kt + 1);
    if constexpr (C::STAGES > 2)
      step(pick<2, C::STAGES>(s0, s1, s2, s3, s4), pick<C::STAGES + 1, C::STAGES>(s0, s1, s2, s3, s4), kt + 2);
    if constexpr (C::STAGES > 3)
      step(pick<3, C::STAGES>(s0, s1, s2, s3, s4), pick<C::STAGES + 2, C::STAGES>(s0, s1, s2, s3, s4), kt + 3);
    if constexpr (C::STAGES > 4)
      step(pick<4, C::STAGES>(s0, s1, s2, s3, s4), pick<C::STAGES + 3, C::STAGES>(s0, s1, s2, s3, s4), kt + 4);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: scale, round to bf16, write 4 consecutive n per lane
  const float s = sa[0] * sb[0];
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
          p0 = pack_bf16x2(acc[i][j][4 * rq + 0] * s, acc[i][j][4 * rq + 1] * s);
          p1 = pack_bf16x2(acc[i][j][4 * rq + 2] * s, acc[i][j][4 * rq + 3] * s);
        }
        *reinterpret_cast<uint2*>(D + (int64_t)m * N + n) = make_uint2(p0, p1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent variant: each workgroup walks a list of tiles as ONE stream of
// 64-wide K steps, so the loads for the next tile are already in flight while
// the current tile's epilogue runs (no pipeline drain between tiles).
//
// * Workgroup b runs on XCD b % 8 (round-robin dispatch). The tiles are split
//   into 8 contiguous chunks of the grouped tile order, one per XCD, and the
//   workgroups of an XCD take the tiles of its chunk in turn, so the tiles
//   that run at the same time on one XCD are neighbours and share A and B
//   panels in that XCD's L2.
// * The epilogue packs 4 bf16 per lane and pairs lanes l and l + 32 with
//   v_permlane32_swap, so that every lane stores 16 contiguous bytes.
// * Stores count in vmcnt like the loads. The per-step wait keeps its steady
//   count: a step needs its own loads, and the only newer operations allowed
//   to stay in flight are the loads of the STAGES - 2 later steps; loads
//   complete in order among themselves, so reaching that count means the
//   step's loads have landed whatever the epilogue's stores are doing (for a
//   few steps after an epilogue the wait simply also covers some stores).
template <class C>
struct Persist {
  static constexpr int kStoresPerLane = C::TM * C::TN * 2;   // 16-byte stores per lane
};

bool xcd_split_enabled();

template <class C>
__device__ __forceinline__ void tile_coords(int lid, int tiles_m, int tiles_n, int& m0, int& n0) {
  const int per_group = C::GROUP_M * tiles_n;
  const int group = lid / per_group;
  const int first_m = group * C::GROUP_M;
  const int gsize = min(tiles_m - first_m, C::GROUP_M);
  const int in_group = lid - group * per_group;
  m0 = (first_m + in_group % gsize) * C::BM;
  n0 = (in_group / gsize) * C::BN;
}

template <class C>
__global__ void __launch_bounds__(C::kThreads, 1)
gemm_fp8_persist_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                        const float* __restrict__ sa, const float* __restrict__ sb,
                        uint16_t* __restrict__ D, int M, int N, int K, int M_valid, int tiles_m,
                        int tiles_n, int split_m, int split_n) {
  constexpr int SB = C::kStageBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t s0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[C::STAGES > 2 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[C::STAGES > 3 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t s4[C::STAGES > 4 ? SB : 16];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;

  // ---- this workgroup's tiles: i-th tile = (bm0 + lm, bn0 + ln) of its XCD's block
  // With split_m * split_n = 8 the tile grid is cut into 8 rectangles, one per XCD
  // (workgroup b runs on XCD b % 8); the workgroups of an XCD take the rectangle's
  // tiles in turn, in groups of GROUP_M rows, so the tiles running at the same time
  // on an XCD are neighbours in both directions. split_m == 0: one rectangle.
  const int nwg = gridDim.x;
  int bm0 = 0, bn0 = 0, bmc = tiles_m, bnc = tiles_n, slot = blockIdx.x, nslots = nwg;
  if (split_m > 0) {
    const int xcd = blockIdx.x & 7;
    const int rm = (tiles_m + split_m - 1) / split_m, rn = (tiles_n + split_n - 1) / split_n;
    const int bx = xcd / split_n, by = xcd % split_n;
    bm0 = bx * rm;
    bn0 = by * rn;
    bmc = max(0, min(tiles_m, bm0 + rm) - bm0);
    bnc = max(0, min(tiles_n, bn0 + rn) - bn0);
    slot = blockIdx.x >> 3;
    nslots = nwg >> 3;
  }
  const int block_tiles = bmc * bnc;
  const int count = slot < block_tiles ? (block_tiles - slot + nslots - 1) / nslots : 0;
  auto tile_mn = [&](int ti, int& m0, int& n0) {
    const int lid = slot + ti * nslots;
    const int per_group = C::GROUP_M * bnc;
    const int group = lid / per_group;
    const int first_m = group * C::GROUP_M;
    const int gsize = min(bmc - first_m, C::GROUP_M);
    const int in_group = lid - group * per_group;
    m0 = (bm0 + first_m + in_group % gsize) * C::BM;
    n0 = (bn0 + in_group / gsize) * C::BN;
  };
  const int nk = (K + kBKS - 1) / kBKS;

  const v4i rsA = make_rsrc(A, (uint32_t)(M * K));
  const v4i rsB = make_rsrc(B, (uint32_t)(N * K));
  const int lr = lane >> 2, lp = lane & 3;
  const int r0 = 16 * wave + lr;
  const int ch = swz64<C::SWZ>(r0, lp);
  const uint32_t step_rows = (uint32_t)(16 * C::kWaves) * (uint32_t)K;

  // Row offsets (K step 0) of tile ti of this workgroup, or "out of range" past the last.
  struct TileBase { uint32_t a, b; };
  auto tile_base = [&](int ti) -> TileBase {
    if (ti >= count) return {kOutOfRange, kOutOfRange};
    int m0, n0;
    tile_mn(ti, m0, n0);
    return {(uint32_t)(m0 + r0) * (uint32_t)K + 16u * ch, (uint32_t)(n0 + r0) * (uint32_t)K + 16u * ch};
  };
  auto issue = [&](uint8_t* stage, TileBase tb, int kstep) {
    const int k0 = kstep * kBKS;
    const bool ok = (tb.a != kOutOfRange) && (k0 + 16 * ch < K);
    const uint32_t lds = lds_addr(stage) + (uint32_t)(16 * wave * kBKS);
#pragma unroll
    for (int i = 0; i < C::kInstA; ++i)
      dma16(rsA, ok ? tb.a + i * step_rows + (uint32_t)k0 : kOutOfRange,
            lds + (uint32_t)(16 * C::kWaves * i * kBKS));
#pragma unroll
    for (int i = 0; i < C::kInstB; ++i)
      dma16(rsB, ok ? tb.b + i * step_rows + (uint32_t)k0 : kOutOfRange,
            lds + (uint32_t)(C::BM * kBKS + 16 * C::kWaves * i * kBKS));
  };

  const int fr = lane & 31;
  const int fg = lane >> 5;
  const int c_lo = swz64<C::SWZ>(fr, 2 * fg) * 16;
  const int c_hi = swz64<C::SWZ>(fr, 2 * fg + 1) * 16;
  auto frag = [&](const uint8_t* base, int row) -> v8i {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + row * kBKS + c_lo);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + row * kBKS + c_hi);
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };

  v16f acc[C::TM][C::TN];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  };
  zero_acc();

  auto compute = [&](const uint8_t* stage) {
    const uint8_t* sA = stage + (wm * C::WTM + fr) * kBKS;
    const uint8_t* sB = stage + C::BM * kBKS + (wn * C::WTN + fr) * kBKS;
    v8i b[C::TN];
#pragma unroll
    for (int j = 0; j < C::TN; ++j) b[j] = frag(sB, 32 * j);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const v8i a = frag(sA, 32 * i);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a, acc[i][j], 0, 0, 0,
                                                                    0, 0, 0);
    }
  };

  const float s = sa[0] * sb[0];
  auto epilogue = [&](int ti) {
    int m0, n0;
    tile_mn(ti, m0, n0);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int m = m0 + wm * C::WTM + 32 * i + fr;
      const bool live = m < M_valid;
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          // rq = 2p (lanes 0..31 keep it) and rq = 2p + 1 (lanes 32..63 take it)
          uint32_t q[2][2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int rq = 2 * p + h;
            q[h][0] = pack_bf16x2(acc[i][j][4 * rq + 0] * s, acc[i][j][4 * rq + 1] * s);
            q[h][1] = pack_bf16x2(acc[i][j][4 * rq + 2] * s, acc[i][j][4 * rq + 3] * s);
          }
          const auto w0 = __builtin_amdgcn_permlane32_swap(q[0][0], q[1][0], false, false);
          const auto w1 = __builtin_amdgcn_permlane32_swap(q[0][1], q[1][1], false, false);
          const int n = n0 + wn * C::WTN + 32 * j + 8 * (2 * p + fg);
          if (m < M && n < N) {
            uint4 o = make_uint4(w0[0], w1[0], w0[1], w1[1]);
            if (!live) o = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(D + (int64_t)m * N + n) = o;
          }
        }
      }
    }
  };

  constexpr int kWaitN = C::kLoadsPerStage * (C::STAGES - 2);
  // step kk + S of the loop body: refill the stage read S - 1 steps ago with K step
  // kk + S + STAGES - 1 of this tile, or of the next tile near the end of this one
  TileBase cur_tb = tile_base(0), next_tb = tile_base(1);
  auto step = [&](uint8_t* cur, uint8_t* refill, int kk_refill) {
    wait_vm_lgkm<kWaitN>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kk_refill < nk) issue(refill, cur_tb, kk_refill);
    else issue(refill, next_tb, kk_refill - nk);
    compute(cur);
  };

  // nk is a multiple of STAGES (the host checks), so every tile starts on stage 0
  issue(s0, cur_tb, 0);
  if constexpr (C::STAGES > 2) issue(s1, cur_tb, 1);
  if constexpr (C::STAGES > 3) issue(s2, cur_tb, 2);
  if constexpr (C::STAGES > 4) issue(s3, cur_tb, 3);
  constexpr int R = C::STAGES - 1;
  for (int ti = 0; ti < count; ++ti) {
    for (int kk = 0; kk < nk; kk += C::STAGES) {
      step(pick<0, C::STAGES>(s0, s1, s2, s3, s4), pick<R, C::STAGES>(s0, s1, s2, s3, s4), kk + R);
      step(pick<1, C::STAGES>(s0, s1, s2, s3, s4), pick<R + 1, C::STAGES>(s0, s1, s2, s3, s4), kk + R + 1);
      if constexpr (C::STAGES > 2)
        step(pick<2, C::STAGES>(s0, s1, s2, s3, s4), pick<R + 2, C::STAGES>(s0, s1, s2, s3, s4), kk + R + 2);
      if constexpr (C::STAGES > 3)
        step(pick<3, C::STAGES>(s0, s1, s2, s3, s4), pick<R + 3, C::STAGES>(s0, s1, s2, s3, s4), kk + R + 3);
      if constexpr (C::STAGES > 4)
        step(pick<4, C::STAGES>(s0, s1, s2, s3, s4), pick<R + 4, C::STAGES>(s0, s1, s2, s3, s4), kk + R + 4);
    }
    epilogue(ti);
    zero_acc();
    cur_tb = next_tb;
    next_tb = tile_base(ti + 2);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <class C>
hipError_t run_pipe(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                    uint16_t* D, int M, int N, int K, int M_valid, hipStream_t s) {
  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  hipLaunchKernelGGL(gemm_fp8_pipe_kernel<C>, dim3((unsigned)tiles), dim3(C::kThreads), 0, s, A,
                     B, sa, sb, D, M, N, K, M_valid, tiles_m, tiles_n);
  return hipGetLastError();
}

template <class C>
hipError_t run_persist(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                       uint16_t* D, int M, int N, int K, int M_valid, int max_wg, hipStream_t s) {
  if (((K + kBKS - 1) / kBKS) % C::STAGES != 0)
    return run_pipe<C>(A, B, sa, sb, D, M, N, K, M_valid, s);
  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  const int tiles = tiles_m * tiles_n;
  int grid = tiles < max_wg ? tiles : max_wg;
  // one rectangle of tiles per XCD: the split with the fewest A+B panel rows per XCD
  int split_m = 0, split_n = 0;
  if (grid == max_wg && (max_wg & 7) == 0 && xcd_split_enabled()) {
    int best = 1 << 30;
    for (int pm = 1; pm <= 8; pm *= 2) {
      const int pn = 8 / pm;
      if (tiles_m % pm || tiles_n % pn) continue;
      const int cost = (tiles_m / pm) * C::BM + (tiles_n / pn) * C::BN;
      if (cost < best) { best = cost; split_m = pm; split_n = pn; }
    }
  }
  hipLaunchKernelGGL(gemm_fp8_persist_kernel<C>, dim3((unsigned)grid), dim3(C::kThreads), 0, s, A,
                     B, sa, sb, D, M, N, K, M_valid, tiles_m, tiles_n, split_m, split_n);
  return hipGetLastError();
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

bool xcd_split_enabled() {
  static bool v = [] {
    const char* e = getenv("FP8LIN_GEMM_XCD_SPLIT");
    return e ? atoi(e) != 0 : true;
  }();
  return v;
}

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
  if (cfg < 0) cfg = ((int64_t)M * N >= (int64_t)4096 * 4096) ? 16 : 3;
  switch (cfg) {
    case 4: return run_pipe<PCfg<256, 256, 2, 2, 4, 0, 8>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 5: return run_pipe<PCfg<256, 256, 2, 4, 4, 0, 8>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 6: return run_pipe<PCfg<256, 256, 2, 2, 4, 1, 8>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 7: return run_pipe<PCfg<256, 256, 2, 4, 4, 1, 8>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 8: return run_pipe<PCfg<256, 256, 2, 2, 3, 0, 8>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 9: return run_pipe<PCfg<256, 256, 2, 4, 5, 0, 8>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 16: return run_persist<PCfg<256, 256, 2, 4, 4, 0, 8>>(A, B, sa, sb, D, m, n, k, mv, 256, s);
    case 18: return run_persist<PCfg<256, 256, 2, 4, 5, 0, 8>>(A, B, sa, sb, D, m, n, k, mv, 256, s);
    case 19: return run_persist<PCfg<256, 256, 2, 4, 4, 0, 4>>(A, B, sa, sb, D, m, n, k, mv, 256, s);
    case 10: return run_pipe<PCfg<128, 256, 2, 2, 4, 1, 8>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 11: return run_pipe<PCfg<256, 128, 2, 2, 4, 1, 8>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 12: return run_pipe<PCfg<128, 256, 2, 4, 4, 1, 8>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 13: return run_pipe<PCfg<256, 256, 2, 2, 5, 1, 8>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 14: return run_pipe<PCfg<256, 256, 2, 2, 4, 1, 4>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 15: return run_pipe<PCfg<256, 256, 2, 2, 4, 1, 16>>(A, B, sa, sb, D, m, n, k, mv, s);
    case 1: return run<CfgBig8>(A, B, sa, sb, D, m, n, k, mv, 1, s);
    case 2: return run<CfgBig4S>(A, B, sa, sb, D, m, n, k, mv, 1, s);
    case 3: return run<CfgMid>(A, B, sa, sb, D, m, n, k, mv, 1, s);
    default: return run<CfgBig4>(A, B, sa, sb, D, m, n, k, mv, 1, s);
  }
}

}  // namespace fp8lin
