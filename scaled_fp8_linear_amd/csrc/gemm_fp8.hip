// Scaled FP8 GEMM on the gfx950 matrix cores.
//
// What it computes (AstrAI, astrai/extension/fp8_state.py, module comment:
// "D = A_SCALE * B_SCALE * A * B" with per-tensor scales amax/448): e4m3
// operands multiplied as they are, float32 accumulation, the scales folded in
// after accumulation, bf16 out:
//
//     D[m, n] = bf16_rne( (sa * sb) * sum_k A[m, k] * B[n, k] )
//
// Both operands keep the contraction index last. The layer's three GEMMs are
// all of this form because the quantize pass also writes transposed copies:
// forward (Qx, Qw), dgrad (Qg, Qw^T), wgrad (Qg^T, Qx^T).
//
// Block recipe (TE "recipe=block", named in NeMo PR 15754): the scales
// multiply each 128-wide partial sum,
//     D[m, n] = bf16_rne( sum_kb sa[m, kb] * sb[n / b_rows, kb] * S_kb[m, n] ),
// with b_rows = 128 for weight tiles and 1 for 1x128 tiles.
//
// Kernels:
//  * gemm_fp8_mx16_kernel (tensorwise, K of at least 512): 256x256 tiles, 4 waves of
//    128x128 on v_mfma_f32_16x16x128_f8f6f4, 128-byte K stages in two LDS slots, one
//    barrier per stage, the epilogue split across the tile boundary; described at the
//    kernel;
//  * gemm_fp8_mx16bw_kernel (block recipe, K of at least 512, outputs of at least 256
//    tiles): 256x256 tiles, 8 waves of 128x64 with the accumulators in VGPRs;
//  * gemm_fp8_mx16b_kernel (block recipe, K of at least 512, other shapes): 256x128
//    tiles, 8 waves of 64x64;
//  * gemm_fp8_persist_kernel (small outputs and K): macro tile
//    BM x BN, K advances 64 bytes per step (one v_mfma_f32_32x32x64_f8f6f4 per 32x32
//    output tile and step), a ring of STAGES LDS arrays, one wait + barrier per step;
//  * gemm_fp8_pipe_kernel: one tile per workgroup, for K step counts the persistent
//    kernel's unrolled loop cannot divide.
// Shared by all of them:
//  * operand tiles go from memory straight into LDS with buffer loads that carry the
//    "lds" modifier (no VGPR staging, no ds_write), issued through inline asm so the
//    compiler does not add waits; the kernels wait (vmcnt) before the barrier that
//    publishes a stage; rows past M or N, K tails and "no tile" read zeros through
//    the buffer range check;
//  * LDS rows XOR-swizzled by 16-byte chunk, so fragment reads are free of bank
//    conflicts; the B fragment is the instruction's first operand, so each lane holds
//    consecutive n of one row m; the MFMA pairs A and B by lane and byte, so any
//    ordering of k within a step is valid as long as both operands use it;
//  * persistent kernels: one workgroup per CU walks its tiles as one stream of K steps
//    (the next tile's loads overlap this tile's epilogue); each XCD gets a rectangle of
//    output tiles (workgroups are dispatched round-robin over the 8 XCDs), so tiles
//    that run together share A and B panels in that XCD's L2;
//  * epilogue: v_cvt_pk_bf16_f32 packs, a lane permute pairs results so that every
//    lane stores 16 contiguous bytes through a buffer resource (pieces outside D are
//    dropped by its range check); rows at or past M_valid are written as zeros (by the
//    kernel, or for gemm_fp8_mx16_kernel by a fill kernel its launcher runs).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace fp8lin {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit dwords
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBKS = 64;                   // K bytes per step
constexpr int kScaleBlock = 128;           // block recipe: K per scale

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

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row for the 16x16x128 kernels: row r
// stores logical chunk c at physical chunk c ^ row_swizzle(r). A fragment read is a
// ds_read_b128 where lane l takes chunk 2 (l / 16) (+ 1) of row l % 16. gfx950's LDS (64
// banks of 4 bytes, a row pair per 256 bytes) serves such a read in four cycles, one per
// group of 16 lanes; measured with bank-conflict counters, a group is the lanes of one
// half-wave whose bits 2-4 have the same parity ({0-3, 12-15, 20-23, 24-27},
// {4-7, 8-11, 16-19, 28-31}, and those plus 32). This swizzle gives the 16 lanes of each
// group 16 distinct bank quads for both chunks of the fragment (swizzling by (r / 2) % 8,
// right for groups of 16 consecutive lanes, costs a second cycle per read here).
__device__ __forceinline__ int row_swizzle(int r) { return (r >> 1) & 5; }

// bias epilogue: 4 consecutive bf16 bias values (8 bytes at column n, n a multiple of 4)
// as floats; columns past N read as 0 (their outputs are dropped anyway)
__device__ __forceinline__ v4f bias4(const uint16_t* bias, int n, int N) {
  if (n >= N) return v4f{0.f, 0.f, 0.f, 0.f};
  const uint2 b = *reinterpret_cast<const uint2*>(bias + n);
  return v4f{__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
             __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u)};
}

// 16-byte LDS read at an LDS byte address (a base register plus a constant folds into the
// instruction's offset field)
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(3))) v4u lds_v4u;
__device__ __forceinline__ v4u lds16(uint32_t a) { return *(lds_v4u*)(uintptr_t)a; }

// One 16-byte-per-lane buffer load written straight to LDS at lds + 16 * lane. Issued
// through inline asm so that the compiler does not guard later LDS reads of other
// stages with waits on it; the kernels wait for these loads themselves (vmcnt) before
// the barrier that publishes a stage. Loads complete in order, which keeps every
// compiler-inserted vmcnt wait for ordinary loads correct (at worst stricter).
// The LDS address goes in M0, which the compiler treats as reserved (it warns that the
// clobber may be ignored): no code generated for these kernels reads or writes M0 itself
// (the LDS instructions of gfx950 do not use it), so only these loads set it.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane((int)lds))
               : "memory", "m0");
}

// As dma16, with a wave-uniform byte offset in an SGPR added to the lane's. Callers put
// the whole row offset in the lane's operand (the one the buffer range check is sure to
// test) and only an offset that stays inside a row in the SGPR.
__device__ __forceinline__ void dma16_so(v4i rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(__builtin_amdgcn_readfirstlane((int)lds))
               : "memory", "m0");
}

// One 4-byte-per-lane buffer load written straight to LDS at lds + 4 * lane.
__device__ __forceinline__ void dma4(v4i rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane((int)lds))
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  // this wave's loads older than the newest N have landed
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  // this wave's loads older than the newest N have landed; its LDS reads are done
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// Tile configuration. BROWS: 0 tensorwise, 1 or 128 block recipe (rows per B scale).
// AFMT: format of the A codes as the f8f6f4 MFMAs number it (0 OCP e4m3, 1 OCP e5m2);
// B is always e4m3. The block recipe takes e4m3 only.
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int SWZ_, int GROUP_M_, int BROWS_,
          int AFMT_ = 0>
struct PCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_, SWZ = SWZ_;
  static constexpr int GROUP_M = GROUP_M_, BROWS = BROWS_, AFMT = AFMT_;
  static constexpr bool BLOCK = BROWS_ != 0;
  static constexpr int kWaves = WM * WN, kThreads = kWaves * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  static constexpr int kStageBytes = (BM + BN) * kBKS;
  static constexpr int kInstA = BM / (16 * kWaves), kInstB = BN / (16 * kWaves);
  static constexpr int kLoadsPerStage = kInstA + kInstB;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  static_assert(STAGES >= 2 && STAGES <= 5, "stages");
  static_assert(!BLOCK || (STAGES % 2 == 0 && (BROWS == 1 || BN % 128 == 0)), "block recipe");
  static_assert(!BLOCK || BROWS == 1 || WTN <= 128, "one weight scale row per wave");
  static_assert(!BLOCK || AFMT == 0, "block recipe: e4m3 operands");
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

template <int V>
using IC = std::integral_constant<int, V>;

// ---------------------------------------------------------------------------
// State and per-step work of one workgroup, shared by both kernels.
template <class C>
struct Tile {
  // the 32x32x64 kernels: 16 rows per load instruction, 32x32 output tiles
  static_assert(C::BM % (16 * C::kWaves) == 0 && C::BN % (16 * C::kWaves) == 0, "dma rows");
  static_assert(C::WTM % 32 == 0 && C::WTN % 32 == 0, "wave tile");
  static_assert(C::kLoadsPerStage * (C::STAGES - 2) <= 63, "vmcnt range");
  const float* sa;
  const float* sb;
  uint16_t* D;
  int M, N, K, M_valid, nk;
  v4i rsA, rsB;
  __amdgpu_buffer_rsrc_t rsD;   // D as a raw buffer: stores at offsets past its end are dropped
  int wave, wm, wn, fr, fg, ch, r0, c_lo, c_hi;
  uint32_t step_rows;
  float s_tensor;   // tensorwise: sa * sb (wave-uniform)
  const uint16_t* bias = nullptr;   // tensorwise: bf16 [N] added after scaling, or none

  v16f acc[C::TM][C::TN];
  v16f part[C::BLOCK ? C::TM : 1][C::BLOCK ? C::TN : 1];
  float scl_a[C::TM];                                 // block recipe: sa of the lane's rows
  float scl_b[C::BLOCK && C::BROWS == 1 ? C::TN : 1][C::BLOCK && C::BROWS == 1 ? 16 : 1];
  float scl_bw;                                       // block recipe with 128-row B scales

  __device__ void init(const uint8_t* A, const uint8_t* B, const float* sa_, const float* sb_,
                       uint16_t* D_, int M_, int N_, int K_, int M_valid_) {
    sa = sa_; sb = sb_; D = D_;
    M = M_; N = N_; K = K_; M_valid = M_valid_;
    nk = (K + kBKS - 1) / kBKS;
    rsA = make_rsrc(A, (uint32_t)(M * K));
    rsB = make_rsrc(B, (uint32_t)(N * K));
    rsD = __builtin_amdgcn_make_buffer_rsrc(D_, 0, M * N * 2, kRsrcWord3);
    const int t = threadIdx.x, lane = t & 63;
    wave = __builtin_amdgcn_readfirstlane(t >> 6);
    wm = wave / C::WN;
    wn = wave % C::WN;
    fr = lane & 31;
    fg = lane >> 5;
    // load plan: instruction i of this wave fills rows 16 (W i + wave) .. +16; lane l
    // takes row l / 4 of them and physical chunk l % 4. Row steps between instructions
    // are multiples of 64, so the lane's logical chunk is the same for all of them.
    const int lr = lane >> 2, lp = lane & 3;
    r0 = 16 * wave + lr;
    ch = swz64<C::SWZ>(r0, lp);
    step_rows = (uint32_t)(16 * C::kWaves) * (uint32_t)K;
    // fragment of a 32-row tile for one step: lane (fr, fg) holds k bytes
    // [32 fg, 32 fg + 32) of row fr, i.e. chunks 2 fg and 2 fg + 1
    c_lo = swz64<C::SWZ>(fr, 2 * fg) * 16;
    c_hi = swz64<C::SWZ>(fr, 2 * fg + 1) * 16;
    s_tensor = C::BLOCK ? 1.0f
                        : __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                        __builtin_bit_cast(int, sa[0] * sb[0])));
    zero_acc();
  }

  __device__ void zero_acc() {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  }

  struct Base { uint32_t a, b; };
  // row offsets of K step 0 of the tile at (m0, n0); kOutOfRange for "no tile"
  __device__ Base base(bool valid, int m0, int n0) const {
    if (!valid) return {kOutOfRange, kOutOfRange};
    return {(uint32_t)(m0 + r0) * (uint32_t)K + 16u * ch,
            (uint32_t)(n0 + r0) * (uint32_t)K + 16u * ch};
  }

  // loads of K step `kstep` of a tile into `stage`. Rows past M (N) read zeros through the
  // buffer size; a K tail and "no tile" read zeros through an offset past the end.
  __device__ void issue(uint8_t* stage, Base tb, int kstep) const {
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
  }

  __device__ v8i frag(const uint8_t* base, int row) const {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + row * kBKS + c_lo);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + row * kBKS + c_hi);
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  }

  // block recipe: load the scales of 128-wide K block kb of the tile at (m0, n0)
  __device__ void load_scales(int m0, int n0, int kb) {
    const int kblocks = K / kScaleBlock;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int m = min(m0 + wm * C::WTM + 32 * i + fr, M - 1);
      scl_a[i] = sa[(int64_t)m * kblocks + kb];
    }
    if constexpr (C::BROWS == 1) {
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = min(n0 + wn * C::WTN + 32 * j + 8 * (r >> 2) + 4 * fg + (r & 3), N - 1);
          scl_b[j][r] = sb[(int64_t)n * kblocks + kb];
        }
    } else {
      const int nb = __builtin_amdgcn_readfirstlane(min(n0 + wn * C::WTN, N - 1) / C::BROWS);
      scl_bw = sb[(int64_t)nb * kblocks + kb];
    }
  }

  // one K step on `stage`. Block recipe: even steps start a 128-wide partial sum, odd
  // steps finish it and add it to the accumulators with its scale.
  template <int ODD>
  __device__ void compute(const uint8_t* stage) {
    const uint8_t* pA = stage + (wm * C::WTM + fr) * kBKS;
    const uint8_t* pB = stage + C::BM * kBKS + (wn * C::WTN + fr) * kBKS;
    v8i b[C::TN];
#pragma unroll
    for (int j = 0; j < C::TN; ++j) b[j] = frag(pB, 32 * j);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const v8i a = frag(pA, 32 * i);
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        if constexpr (!C::BLOCK) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a, acc[i][j], 0,
                                                                      C::AFMT, 0, 0, 0, 0);
        } else if constexpr (!ODD) {
          const v16f z = {};
          part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a, z, 0, 0, 0, 0,
                                                                       0, 0);
        } else {
          part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a, part[i][j], 0,
                                                                       0, 0, 0, 0, 0);
        }
      }
    }
    if constexpr (C::BLOCK && ODD) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float sbv;
            if constexpr (C::BROWS == 1) sbv = scl_b[j][r];
            else sbv = scl_bw;
            acc[i][j][r] = fmaf(part[i][j][r], scl_a[i] * sbv, acc[i][j][r]);
          }
    }
  }

  // write the tile at (m0, n0): scale, round to bf16, 16 bytes per lane. Every lane
  // issues exactly 2 TM TN buffer stores; pieces outside D get an offset past its end,
  // which the buffer range check drops.
  // With a bias, value 4 rq + c of the lane holds column 32 j + 8 rq + 4 fg + c of its
  // 32x32 tile; the bias is added in float32 after the scale, before the one rounding.
  __device__ void epilogue(int m0, int n0) {
    const float s = s_tensor;
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
            if (bias != nullptr) {
              const v4f b = bias4(bias, n0 + wn * C::WTN + 32 * j + 8 * rq + 4 * fg, N);
              q[h][0] = pack_bf16x2(acc[i][j][4 * rq + 0] * s + b[0],
                                    acc[i][j][4 * rq + 1] * s + b[1]);
              q[h][1] = pack_bf16x2(acc[i][j][4 * rq + 2] * s + b[2],
                                    acc[i][j][4 * rq + 3] * s + b[3]);
            } else {
              q[h][0] = pack_bf16x2(acc[i][j][4 * rq + 0] * s, acc[i][j][4 * rq + 1] * s);
              q[h][1] = pack_bf16x2(acc[i][j][4 * rq + 2] * s, acc[i][j][4 * rq + 3] * s);
            }
          }
          const auto w0 = __builtin_amdgcn_permlane32_swap(q[0][0], q[1][0], false, false);
          const auto w1 = __builtin_amdgcn_permlane32_swap(q[0][1], q[1][1], false, false);
          const int n = n0 + wn * C::WTN + 32 * j + 8 * (2 * p + fg);
          v4i o = {(int)w0[0], (int)w1[0], (int)w0[1], (int)w1[1]};
          if (!live) o = v4i{0, 0, 0, 0};
          const uint32_t off = (m < M && n < N) ? ((uint32_t)m * (uint32_t)N + (uint32_t)n) * 2u
                                                : kOutOfRange;
          __builtin_amdgcn_raw_buffer_store_b128(o, rsD, off, 0, 0);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Persistent kernel: a workgroup walks its tiles as one stream of K steps.
// The K step count is a multiple of STAGES (the host checks), so every tile
// starts on stage 0 and the unrolled loop body knows each step's stage.
template <class C>
__global__ void __launch_bounds__(C::kThreads, 1)
gemm_fp8_persist_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                        const float* __restrict__ sa, const float* __restrict__ sb,
                        const uint16_t* __restrict__ bias, uint16_t* __restrict__ D, int M,
                        int N, int K, int M_valid, int tiles_m, int tiles_n, int split_m,
                        int split_n) {
  constexpr int SB = C::kStageBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t s0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[C::STAGES > 2 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[C::STAGES > 3 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t s4[C::STAGES > 4 ? SB : 16];

  Tile<C> T;
  T.init(A, B, sa, sb, D, M, N, K, M_valid);
  T.bias = bias;

  // ---- this workgroup's tiles. With split_m * split_n = 8 the tile grid is cut into
  // 8 rectangles, one per XCD (workgroup b runs on XCD b % 8); the workgroups of an
  // XCD take the rectangle's tiles in turn, in groups of GROUP_M rows, so the tiles
  // running at the same time on an XCD are neighbours in both directions.
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
  auto tile_base = [&](int ti) {
    int m0 = 0, n0 = 0;
    if (ti < count) tile_mn(ti, m0, n0);
    return T.base(ti < count, m0, n0);
  };

  constexpr int kWaitN = C::kLoadsPerStage * (C::STAGES - 2);
  const int nk = T.nk;
  auto cur_tb = tile_base(0), next_tb = tile_base(1);
  int cm0 = 0, cn0 = 0;
  // one step (index S within the loop body) on stage `cur`: wait for its loads, publish
  // it, refill the stage read one step ago with K step kk_refill (of this tile, or of the
  // next one near the end of this tile), multiply.
  auto step = [&](auto S_, uint8_t* cur, uint8_t* refill, int kk, int kk_refill) {
    constexpr int S = decltype(S_)::value;
    wait_vm_lgkm<kWaitN>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kk_refill < nk) T.issue(refill, cur_tb, kk_refill);
    else T.issue(refill, next_tb, kk_refill - nk);
    // block recipe: the scales of the 128-wide K block finished at the odd step are
    // loaded at its start; that step's MFMAs cover the load latency
    if constexpr (C::BLOCK && (S % 2) == 1) T.load_scales(cm0, cn0, (kk + S) / 2);
    T.template compute<S % 2>(cur);
  };

  T.issue(s0, cur_tb, 0);
  if constexpr (C::STAGES > 2) T.issue(s1, cur_tb, 1);
  if constexpr (C::STAGES > 3) T.issue(s2, cur_tb, 2);
  if constexpr (C::STAGES > 4) T.issue(s3, cur_tb, 3);
  constexpr int R = C::STAGES - 1;
  // ring[i] = stage of step i of the loop body (i < 2 STAGES)
#define FP8LIN_P(i) pick<i, C::STAGES>(s0, s1, s2, s3, s4)
  uint8_t* const ring[10] = {FP8LIN_P(0), FP8LIN_P(1), FP8LIN_P(2), FP8LIN_P(3), FP8LIN_P(4),
                             FP8LIN_P(5), FP8LIN_P(6), FP8LIN_P(7), FP8LIN_P(8), FP8LIN_P(9)};
#undef FP8LIN_P
  for (int ti = 0; ti < count; ++ti) {
    tile_mn(ti, cm0, cn0);
    for (int kk = 0; kk < nk; kk += C::STAGES) {
      step(IC<0>{}, ring[0], ring[R], kk, kk + R);
      step(IC<1>{}, ring[1], ring[R + 1], kk, kk + R + 1);
      if constexpr (C::STAGES > 2) step(IC<2>{}, ring[2], ring[R + 2], kk, kk + R + 2);
      if constexpr (C::STAGES > 3) step(IC<3>{}, ring[3], ring[R + 3], kk, kk + R + 3);
      if constexpr (C::STAGES > 4) step(IC<4>{}, ring[4], ring[R + 4], kk, kk + R + 4);
    }
    T.epilogue(cm0, cn0);
    T.zero_acc();
    cur_tb = next_tb;
    next_tb = tile_base(ti + 2);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may land after exit
}

// ---------------------------------------------------------------------------
constexpr int kStageK = 128;   // K bytes per LDS stage of gemm_fp8_mx16_kernel

// ---------------------------------------------------------------------------
// 16x16x128 kernel (tensorwise scaling): 256x256 tiles (or 224x256 / 256x224), 4 waves
// of 128x128 (112x128 / 128x112), each wave an RT x CT grid of v_mfma_f32_16x16x128_f8f6f4
// tiles (the 16x16 form keeps the matrix cores busier than 32x32x64 when LDS reads run
// alongside, and moves half as many accumulator bytes per FLOP). An LDS stage holds 128
// K bytes of the tile's A and B rows (64 KB at 256x256), in two slots, loaded straight
// to LDS: a 64-byte K step would fetch each 128-byte line in two halves, one step apart,
// which halves the L2 -> CU throughput. One MFMA covers a whole stage's K, so per stage
// a wave runs RT x CT MFMAs (rows i of 16x16 tiles, all CT columns j each):
//   first half  (rows 0 .. RT/2-1): A fragments of rows 1 .. RT-1 are read in between;
//   mid-stage:  the wave waits for its loads of stage s + 1; a barrier publishes them
//               and frees this stage's slot (all its reads are done by then);
//   second half (the other rows, tile column by tile column): the loads of stage s + 2
//               go into this slot, and stage s + 1's A row 0 is read, and its B fragment
//               j right after this stage's last MFMA with B fragment j (one set of B
//               registers).
// Fragment of a 16-row tile: lane l holds 32 bytes of row l % 16 at K offset
// 32 (l / 16); the instruction pairs A and B by lane and byte, so this K order is as
// good as any. The B tile goes in as the first operand, so a lane's 4 results are 4
// consecutive n of row m = l % 16.
template <class C, bool TAIL, bool BIAS>
__global__ void __launch_bounds__(C::kThreads, 1)
gemm_fp8_mx16_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                     const float* __restrict__ sa, const float* __restrict__ sb,
                     const uint16_t* __restrict__ bias, uint16_t* __restrict__ D, int M, int N,
                     int K, int M_valid, int tiles_m, int tiles_n, int split_m, int split_n) {
  static_assert(!C::BLOCK, "tensorwise only");
  constexpr int SB = (C::BM + C::BN) * kStageK;
  constexpr int kRowsPerInst = 1024 / kStageK;               // 8 rows of 128 bytes
  constexpr int kInstA = C::BM / (kRowsPerInst * C::kWaves);  // per wave and stage
  constexpr int kInstB = C::BN / (kRowsPerInst * C::kWaves);
  constexpr int kDma = kInstA + kInstB;
  constexpr int RT = C::WTM / 16, CT = C::WTN / 16;           // 16x16 tiles per wave
  constexpr int RH = RT / 2, RS = RT - RH;                    // rows in the two halves
  // epilogue stores per lane: one per pair of tiles, and one per row for an odd last tile
  constexpr int kStores = RT * (CT / 2) + (CT % 2 ? RT : 0);
  static_assert(RH >= 1 && kDma <= 63 && kStores <= 63, "plan");
  static_assert(C::BM % (kRowsPerInst * C::kWaves) == 0 &&
                C::BN % (kRowsPerInst * C::kWaves) == 0, "load instructions");
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[SB];
  // STAGED (wave tiles 128 outputs wide, no bias): the output passes through 4 KB of LDS
  // per wave so that every store writes whole 128-byte lines (see op_emit)
  constexpr bool kStaged = C::WTN == 128 && !BIAS;
  __shared__ __attribute__((aligned(1024))) uint8_t stg_mem[kStaged ? 4096 * C::kWaves : 16];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const v4i rsA = make_rsrc(A, (uint32_t)(M * K));
  const v4i rsB = make_rsrc(B, (uint32_t)(N * K));
  // D as a raw buffer over the valid rows: stores to rows at or past M_valid are dropped
  const __amdgpu_buffer_rsrc_t rsD =
      __builtin_amdgcn_make_buffer_rsrc(D, 0, M_valid * N * 2, kRsrcWord3);
  const float scl = __builtin_bit_cast(
      float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sa[0] * sb[0])));

  // tile assignment: as in gemm_fp8_persist_kernel (one rectangle of tiles per XCD)
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

  // load plan: instruction i of wave w fills rows
  // 8 (W i + w) .. + 8; lane l writes 16 bytes at 16 l: row l / 8, physical chunk l % 8,
  // which holds logical chunk (l % 8) ^ row_swizzle(row)
  const int lrow = kRowsPerInst * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ row_swizzle(lrow);
  const uint32_t inst_rows = (uint32_t)(kRowsPerInst * C::kWaves) * (uint32_t)K;
  // the lane's part of its row offsets (the same for A and B)
  const uint32_t lane_off = (uint32_t)lrow * (uint32_t)K + 16u * lchunk;
  struct Rows { uint32_t a, b; };      // wave-uniform: the tile's first row times K
  auto rows_of = [&](int ti) -> Rows {
    if (ti >= count) return {kOutOfRange, kOutOfRange};
    int m0, n0;
    tile_mn(ti, m0, n0);
    return {(uint32_t)m0 * (uint32_t)K, (uint32_t)n0 * (uint32_t)K};
  };
  // load d (0 .. kDma) of stage kb of the tile whose rows are r, into slot_mem. The lane's
  // whole row offset goes in the VGPR operand, which the buffer range check tests, so
  // rows past M or N read zeros; only the K block's offset (which stays inside a row)
  // goes in the SGPR operand.
  auto dma = [&](int d, uint8_t* slot_mem, Rows r, int kb) {
    const uint32_t k0 = (uint32_t)kb * kStageK;
    const uint32_t lds = lds_addr(slot_mem) + 1024u * wave;
    uint32_t off = d < kInstA ? lane_off + (r.a + d * inst_rows)
                              : lane_off + (r.b + (d - kInstA) * inst_rows);
    // TAIL (K not a multiple of 256): the K tail, or a padding stage, reads zeros, chunk
    // by chunk (K is a multiple of 16)
    if constexpr (TAIL) off = k0 + 16u * lchunk < (uint32_t)K ? off : kOutOfRange;
    if (d < kInstA)
      dma16_so(rsA, off, k0, lds + 1024u * C::kWaves * d);
    else
      dma16_so(rsB, off, k0, lds + C::BM * kStageK + 1024u * C::kWaves * (d - kInstA));
  };
  // fragments: lane (r16 = l % 16, g = l / 16) reads logical chunks 2 g, 2 g + 1 of its row;
  // rows 16 apart share the swizzle
  const int r16 = lane & 15, g4 = lane >> 4;
  const int sw = row_swizzle(r16);
  const uint32_t fo0 = r16 * kStageK + 16 * ((2 * g4) ^ sw);
  const uint32_t fo1 = r16 * kStageK + 16 * ((2 * g4 + 1) ^ sw);
  auto rd = [&](const uint8_t* p) {
    const uint4 lo = *reinterpret_cast<const uint4*>(p + fo0);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + fo1);
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };
  auto rdA = [&](const uint8_t* sm, int i) { return rd(sm + (wm * C::WTM + 16 * i) * kStageK); };
  auto rdB = [&](const uint8_t* sm, int j) {
    return rd(sm + (C::BM + wn * C::WTN + 16 * j) * kStageK);
  };

  v4f acc[RT][CT];
  // B fragments (one set: fragment j of stage s + 1 replaces stage s's after its last
  // MFMA); A rows 0 .. RH-1 and RH .. RT-1 of this stage. Only B and A row 0 are read a
  // stage ahead: rows 1 .. RT-1 are read during the stage's first half, which keeps the
  // register peak down.
  v8i Bf[CT], Alo[RH], Ahi[RS];

  // stages per tile: K / 128 rounded up to an even count of at least 4; stages past K
  // (the tail of a K that is not a multiple of 256) load zeros
  const int ns = max(4, (((K + kStageK - 1) / kStageK) + 1) & ~1);
  Rows cur = rows_of(0), nxt = rows_of(1);

  // ---- epilogue pieces: scale, round to bf16, 16-byte stores. Store op o of row i of the
  // wave's 16x16 tiles: for o < kPairs the tiles j = 2 o, 2 o + 1 (after v_permlane16_swap
  // lane group g = l / 16 holds 8 consecutive n, columns 8 (g / 2) .. + 8 of tile j + g % 2);
  // with an odd CT, op kPairs is the last tile alone, 8 bytes (4 consecutive n) per lane.
  // Rows at or past M_valid lie past the end of D's buffer range (rsD covers the valid rows
  // only) and are dropped there; the launcher writes their zeros.
  constexpr int kPairs = CT / 2, kOps = kPairs + CT % 2;   // store ops per row
  static_assert(kStores == RT * kOps, "store count");
  static_assert(!kStaged || kOps == 4, "a staged row is 4 ops: 2 chunk columns of 2 pairs");
  typedef int v2i __attribute__((ext_vector_type(2)));
  // BIAS: tile j's 4 columns of the lane are n0 + wn WTN + 16 j + 4 g .. + 3 (packed bf16;
  // columns past N read as 0)
  uint2 bj[BIAS ? CT : 1];
  auto load_bias = [&](int n0) {
    if constexpr (BIAS) {
#pragma unroll
      for (int j = 0; j < CT; ++j) {
        const int n = n0 + wn * C::WTN + 16 * j + 4 * g4;
        bj[j] = n < N ? *reinterpret_cast<const uint2*>(bias + n) : make_uint2(0u, 0u);
      }
    }
  };
  // the packed output of op o of row i (BIAS: the float32 bias added after the scale,
  // before the one rounding)
  auto op_value = [&](int i, int o) -> v4i {
    const float si = scl;
    auto val = [&](int j, int r) {
      if constexpr (BIAS) {
        const uint32_t w = r < 2 ? bj[j].x : bj[j].y;
        return acc[i][j][r] * si + __uint_as_float(r % 2 ? (w & 0xFFFF0000u) : (w << 16));
      } else {
        return acc[i][j][r] * si;
      }
    };
    if (o < kPairs) {
      const int j = 2 * o;
      const uint32_t p0j = pack_bf16x2(val(j, 0), val(j, 1));
      const uint32_t p1j = pack_bf16x2(val(j, 2), val(j, 3));
      const uint32_t p0k = pack_bf16x2(val(j + 1, 0), val(j + 1, 1));
      const uint32_t p1k = pack_bf16x2(val(j + 1, 2), val(j + 1, 3));
      const auto w0 = __builtin_amdgcn_permlane16_swap(p0j, p0k, false, false);
      const auto w1 = __builtin_amdgcn_permlane16_swap(p1j, p1k, false, false);
      return v4i{(int)w0[0], (int)w1[0], (int)w0[1], (int)w1[1]};
    }
    constexpr int j = CT - 1;
    return v4i{(int)pack_bf16x2(val(j, 0), val(j, 1)), (int)pack_bf16x2(val(j, 2), val(j, 3)),
               0, 0};
  };
  // the lane's part of its output offsets (bytes): its row in the workgroup tile times N
  // plus its first column in the op; an op adds the tile origin, its 16 i rows and 32 o
  // columns, all wave-uniform. The launcher keeps every row below M + BM + 1 inside 2^31
  // bytes, so a row at or past M_valid lands at or past the end of rsD's range, where the
  // store is dropped; a column past N would land in the next row, so such a piece gets an
  // offset past the end.
  const int lcol_p = wn * C::WTN + 16 * (g4 & 1) + 8 * (g4 >> 1);
  const int lcol_s = wn * C::WTN + 16 * (CT - 1) + 4 * g4;
  const uint32_t lrow_off = (uint32_t)(wm * C::WTM + r16) * (uint32_t)N * 2u;
  const uint32_t loff_p = lrow_off + 2u * (uint32_t)lcol_p;
  const uint32_t loff_s = lrow_off + 2u * (uint32_t)lcol_s;
  auto op_store = [&](int i, int o, v4i v, int m0, int n0) {
    const uint32_t base = ((uint32_t)(m0 + 16 * i) * (uint32_t)N + (uint32_t)n0) * 2u;
    if (o < kPairs) {
      const bool in = lcol_p < N - n0 - 32 * o;
      __builtin_amdgcn_raw_buffer_store_b128(v, rsD, in ? base + 64u * o + loff_p : kOutOfRange,
                                             0, 0);
    } else {
      const bool in = lcol_s < N - n0;
      __builtin_amdgcn_raw_buffer_store_b64(v2i{v[0], v[1]}, rsD, in ? base + loff_s : kOutOfRange,
                                            0, 0);
    }
  };

  // STAGED. An op's 16 bytes per lane are 8 outputs of ITS row (l % 16), 4 lanes per row, so
  // a direct store writes 16 rows of 64 bytes: half lines, which cost the memory pipeline
  // about as many cycles as whole ones. Staged, op o of row i writes its piece into the
  // wave's 16 staging rows of 256 bytes (row r16, 16-byte chunk c = 4 o + 2 (g % 2) + g / 2,
  // the piece's 8 columns / 8); a row's chunk c (h = c % 2: rows 8 h .. 8 h + 7; q = c / 2:
  // columns 64 q .. 64 q + 63, complete once pairs 2 q and 2 q + 1 are written) is read back
  // so that lane l holds row 8 h + l / 8, columns 64 q + 8 (l % 8), and stored: 8 rows of
  // 128 bytes. Op k of a half reads and stores the chunk two ops behind it (row i's chunk
  // o - 2, or the row before's chunk o + 2) before it computes its own piece, which hides
  // the read's latency; the half's last op also stores its row's chunks 2 and 3. Pairs 0
  // and 1 of a row overwrite chunks 0 to 7 of the staging rows only after the row before's
  // chunks 2 and 3 (16-byte chunks 8 to 15) were read. Each row still takes kOps stores, so
  // the waits that count stores in flight stay exact. A wave reads only what it wrote and
  // its LDS operations complete in order: no barrier. 16-byte chunk c of staging row r
  // sits at c ^ sw(r), sw(r) = ((r % 8) + 8 r1) ^ 6 r3 (ri: bit i of r), chosen for how
  // gfx950 serves 16-byte LDS accesses (measured with the bank-conflict counter): a write in
  // groups of 8 consecutive lanes over 128 bytes of banks, so the 8 rows of a group need
  // distinct sw(r) % 8; a read in groups of 16 lanes over 256 bytes ({0-3, 12-15, 20-23,
  // 24-27}, {4-7, 8-11, 16-19, 28-31}, and those + 32), which r1 in bit 3 spreads over all
  // 64 banks. The 6 r3 term changes no bank but keeps the kernels free of register spills.
  auto stg_sw = [](int r) { return ((r & 7) | (((r >> 1) & 1) << 3)) ^ (6 * ((r >> 3) & 1)); };
  const uint32_t stg = lds_addr(stg_mem) + 4096u * (uint32_t)wave;
  // the lane's staging addresses for op 0 (write) and for chunk 0 (read); an op or chunk
  // flips chunk bits only (XOR inside the 256-byte row), since sw(8 h + r) = sw(r) ^ 6 h
  const uint32_t stg_w =
      stg + 256u * (uint32_t)r16 + 16u * (uint32_t)((2 * (g4 & 1) + (g4 >> 1)) ^ stg_sw(r16));
  const uint32_t stg_r =
      stg + 256u * (uint32_t)(lane >> 3) + 16u * (uint32_t)((lane & 7) ^ stg_sw(lane >> 3));
  const int fcol = wn * C::WTN + 8 * (lane & 7);
  const uint32_t frow_off =
      (uint32_t)(wm * C::WTM + (lane >> 3)) * (uint32_t)N * 2u + 2u * (uint32_t)fcol;
  typedef __attribute__((address_space(3))) v4i lds_v4i;
  // op k of a half that starts at row i0 and has kn ops
  auto op_emit = [&](int k, int i0, int kn, int m0, int n0) {
    const int i = i0 + k / kOps, o = k % kOps;
    if constexpr (!kStaged) {
      op_store(i, o, op_value(i, o), m0, n0);
    } else {
      auto chunk_read = [&](int c) {
        const int h = c & 1, q = c >> 1;
        return *(lds_v4i*)(uintptr_t)((stg_r ^ (128u * q + 96u * h)) + 2048u * h);
      };
      auto chunk_store = [&](v4i w, int row, int c) {
        const int h = c & 1, q = c >> 1;
        const uint32_t base = ((uint32_t)(m0 + 16 * row) * (uint32_t)N + (uint32_t)n0) * 2u;
        __builtin_amdgcn_raw_buffer_store_b128(
            w, rsD,
            fcol + 64 * q < N - n0 ? base + frow_off + 16u * (uint32_t)N * h + 128u * q
                                   : kOutOfRange,
            0, 0);
      };
      const bool behind = k >= 2;
      const int prow = o >= 2 ? i : i - 1, pc = o >= 2 ? o - 2 : o + 2;
      v4i w;
      if (behind) w = chunk_read(pc);
      *(lds_v4i*)(uintptr_t)(stg_w ^ (64u * (uint32_t)o)) = op_value(i, o);
      if (behind) chunk_store(w, prow, pc);
      if (k == kn - 1) {
        chunk_store(chunk_read(2), i, 2);
        chunk_store(chunk_read(3), i, 3);
      }
    }
  };

  // One stage. Bf and Alo[0]: this stage's B fragments and A row 0 (read before); the
  // next stage's are read in the second half, B fragment j into Bf[j] right after this
  // stage's last MFMA with it (the second half runs tile column by tile column).
  // FIRST: the tile's first stage (sums start at zero). LAST: the tile's last stage, which
  // reads no fragments of the next stage (they are read after it, so that they hold no
  // registers through it).
  // The epilogue of a tile runs in the shadow of the matrix cores, in two halves:
  // EPI = 1 (the LAST stage): after the first half, rows 0 .. RH-1 are final; their store
  //   ops run during the second half. All loads of that half (the next tile's stage 1) go
  //   out first, one per MFMA, and the ops (value and store) are spread over the MFMAs
  //   left.
  // EPI = 2 (every tile's FIRST stage): the first half's MFMAs write rows 0 .. RH-1 only,
  //   so the previous tile's rows RH .. RT-1 (at em0, en0) go out in between. With those of
  //   EPI = 1, exactly kStores stores then follow the stage-1 loads, and the wait in the
  //   middle of the stage lets them stay in flight: loads and stores retire in order, and
  //   the loads it waits for were issued before them. Before the first tile there is no
  //   previous tile (em0 = M): no stores, and the wait covers every load.
  auto stage = [&](auto FIRST_, auto LAST_, auto EPI_, int s, uint8_t* mine, uint8_t* other,
                   int em0, int en0) {
    constexpr bool FIRST = decltype(FIRST_)::value != 0, LAST = decltype(LAST_)::value != 0;
    constexpr int EPI = decltype(EPI_)::value;
    static_assert(EPI != 1 || LAST, "the first epilogue half runs in a last stage");
    static_assert(EPI != 2 || FIRST, "the second epilogue half runs in a first stage");
    const v4f z = {};
    // first half: rows 0 .. RH-1; A rows 1 .. RT-1 are read in between (row i is first
    // needed by MFMA i CT, and is read among the first ones)
    if constexpr (LAST) load_bias(en0);
#pragma unroll
    for (int i = 1; i < RH; ++i) Alo[i] = rdA(mine, i);
#pragma unroll
    for (int i = 0; i < RS; ++i) Ahi[i] = rdA(mine, RH + i);
    if constexpr (EPI == 2) {
      // RS kOps ops of the previous tile spread over the RH CT MFMAs, in a pinned order
      constexpr int kMf = RH * CT, kEp = RS * kOps;
#pragma unroll
      for (int x = 0; x < kMf; ++x) {
        const int i = x / CT, j = x % CT;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Bf[j], Alo[i], z, 0,
                                                                     C::AFMT, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (em0 < M) {             // false before the first tile: nothing to store
#pragma unroll
          for (int k = x * kEp / kMf; k < (x + 1) * kEp / kMf; ++k)
            op_emit(k, RH, kEp, em0, en0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < RH; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Bf[j], Alo[i],
                                                                       FIRST ? z : acc[i][j], 0,
                                                                       C::AFMT, 0, 0, 0, 0);
#pragma unroll
      for (int x = 0; x < RH * CT; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (x % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // stage s + 1 landed (own loads), own LDS reads done; then for every wave. In the first
    // tile no stores follow the stage-1 loads.
    if constexpr (EPI == 2) {
      if (em0 >= M) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kStores) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // second half: rows RH .. RT-1, with the loads of stage s + 2 (into `mine`) and the
    // reads of stage s + 1's fragments (from `other`) in between, in a pinned order
    const int gs = s + 2;
    const Rows r = gs < ns ? cur : nxt;
    const int kb = gs < ns ? gs : gs - ns;
    constexpr int kSecond = RS * CT;                 // MFMAs in the second half
    constexpr int kLeadA = CT - 1;                   // see the reads below
    constexpr int kEpLo = RH * kOps;                 // EPI = 1: store ops of rows 0 .. RH-1
    static_assert(EPI != 1 || kDma < kSecond, "the loads go out before the stores");
#pragma unroll
    for (int x = 0; x < kSecond; ++x) {
      const int i = RH + x % RS, j = x / RS;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Bf[j], Ahi[i - RH],
                                                                   FIRST ? z : acc[i][j], 0,
                                                                   C::AFMT, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (EPI == 1) {
        // the loads first (one per MFMA), then the store ops spread over the MFMAs left
        if (x < kDma) dma(x, mine, r, kb);
#pragma unroll
        for (int k = 0; k < kEpLo; ++k)
          if (kDma + k * (kSecond - kDma) / kEpLo == x)
            op_emit(k, 0, kEpLo, em0, en0);
      } else {
        if (x * kDma / kSecond != (x + 1) * kDma / kSecond) dma(x * kDma / kSecond, mine, r, kb);
        // the next stage's B fragment j after this stage's last MFMA with it (CT - 1 MFMAs
        // or more before the next stage's first use of it), and its A row 0 kLeadA MFMAs
        // before the stage ends (early enough that the next stage's first MFMA does not
        // wait for it)
        if constexpr (!LAST) {
          if (x % RS == RS - 1) Bf[j] = rdB(other, j);
          if (x == kSecond - kLeadA) Alo[0] = rdA(other, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

#pragma unroll
  for (int d = 0; d < kDma; ++d) dma(d, slot0, cur, 0);
#pragma unroll
  for (int d = 0; d < kDma; ++d) dma(d, slot1, ns > 1 ? cur : nxt, ns > 1 ? 1 : 0);
  wait_vm<kDma>();                     // stage 0 landed
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // stage 0 of a tile: its B fragments and A rows 0 .. RH-1 (slot 0, published)
  auto first_frags = [&]() {
#pragma unroll
    for (int j = 0; j < CT; ++j) Bf[j] = rdB(slot0, j);
    Alo[0] = rdA(slot0, 0);
  };
  first_frags();
  // the previous tile (its rows RH .. RT-1 still to go); a row origin of M: none
  int pm0 = M, pn0 = 0;
  for (int ti = 0; ti < count; ++ti) {
    int cm0, cn0;
    tile_mn(ti, cm0, cn0);
    // stages 0, 1 | 2 .. ns - 3 | ns - 2, ns - 1 (ns is even and at least 4)
    stage(IC<1>{}, IC<0>{}, IC<2>{}, 0, slot0, slot1, pm0, pn0);
    stage(IC<0>{}, IC<0>{}, IC<0>{}, 1, slot1, slot0, 0, 0);
    for (int s = 2; s < ns - 2; s += 2) {
      stage(IC<0>{}, IC<0>{}, IC<0>{}, s, slot0, slot1, 0, 0);
      stage(IC<0>{}, IC<0>{}, IC<0>{}, s + 1, slot1, slot0, 0, 0);
    }
    stage(IC<0>{}, IC<0>{}, IC<0>{}, ns - 2, slot0, slot1, 0, 0);
    stage(IC<0>{}, IC<1>{}, IC<1>{}, ns - 1, slot1, slot0, cm0, cn0);
    first_frags();                     // the next tile's stage 0, published at stage ns - 1
    pm0 = cm0;
    pn0 = cn0;
    cur = nxt;
    nxt = rows_of(ti + 2);
  }
  if (count > 0) {
    // the last tile's rows RH .. RT-1
#pragma unroll
    for (int k = 0; k < RS * kOps; ++k)
      op_emit(k, RH, RS * kOps, pm0, pn0);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // no load may land after exit
}

// ---------------------------------------------------------------------------
// Block-recipe 16x16x128 kernel: 256x128 tiles, 8 waves (two per SIMD) of 64x64, each a
// 4x4 grid of 16x16 tiles. A 16x16x128 MFMA covers exactly one 128-wide K block, so
// each one, started from zero, is that block's partial sum P, and the lane folds it in
//     acc += P * (sa[m, kb] * sb[n / b_rows, kb])
// with the accumulators in VGPRs (64 per wave, which is what lets P and the fragments
// stay in VGPRs as well: each MFMA then has its own result registers and the folds of
// one MFMA overlap the next). Stages of 128 K bytes as in gemm_fp8_mx16_kernel, but in
// three LDS slots: the barrier in the middle of stage s publishes stage s + 1 and frees
// slot s % 3, which takes the loads of stage s + 3, so two stages are in flight while
// one is multiplied (with one, the load latency, not the matrix cores, sets the pace).
// The slot index is computed at run time (the compiler sees no LDS writes: the loads
// are asm). A slot also holds the stage's scales, loaded with the operands by 4-byte
// LDS loads into one region indexed by p = 64 w + l (wave w, lane l):
//   p in [0, BM):       sa of tile row wm WTM + 16 (p % RT) + (p % WTM) / RT, for
//                       p = wm WTM + (row % 16) RT + i: a lane's RT row scales are
//                       contiguous;
//   p in [BM, BM + BN): with one scale per B row, sb of tile column
//                       wn WTN + 16 j + 4 g + r at p - BM = wn WTN + g 4 CT + 4 j + r
//                       (a lane's 4 CT column scales are contiguous); with one scale
//                       per 128 B rows, the single value at p = BM.
// Every wave issues the same loads per stage (lanes with nothing to load read out of
// range), so the memory counts stay uniform.
template <class C, bool PAD>
__global__ void __launch_bounds__(C::kThreads, 1)
gemm_fp8_mx16b_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                      const float* __restrict__ sa, const float* __restrict__ sb,
                      uint16_t* __restrict__ D, int M, int N, int K, int M_valid, int tiles_m,
                      int tiles_n, int split_m, int split_n) {
  static_assert(C::BLOCK, "block recipe");
  constexpr int BROWS = C::BROWS;
  constexpr int RT = C::WTM / 16, CT = C::WTN / 16;
  constexpr int RH = RT / 2;
  constexpr int kTileBytes = (C::BM + C::BN) * kStageK;
  constexpr int kScaleLanes = 64 * C::kWaves;
  constexpr int kSaOff = kTileBytes, kSbOff = kTileBytes + 4 * C::BM;
  constexpr int SB = kTileBytes + 4 * kScaleLanes;
  constexpr int kRowsPerInst = 1024 / kStageK;
  constexpr int kInstA = C::BM / (kRowsPerInst * C::kWaves);
  constexpr int kInstB = C::BN / (kRowsPerInst * C::kWaves);
  constexpr int kDma = kInstA + kInstB + 1;                   // + one scale piece
  constexpr int kStores = RT * CT / 2;
  static_assert(RT % 2 == 0 && CT % 2 == 0 && 2 * kDma + kStores <= 63, "plan");
  static_assert(C::BM + C::BN <= kScaleLanes, "one scale load per wave and stage");
  static_assert(C::BM % (kRowsPerInst * C::kWaves) == 0 &&
                C::BN % (kRowsPerInst * C::kWaves) == 0, "load instructions");
  static_assert(BROWS == 1 || C::BN % BROWS == 0, "one weight scale row per tile");
  constexpr int kSlots = 3;             // two stages in flight while one is multiplied
  static_assert(kSlots * SB <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSlots * SB];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int kblocks = K / kStageK;
  const v4i rsA = make_rsrc(A, (uint32_t)(M * K));
  const v4i rsB = make_rsrc(B, (uint32_t)(N * K));
  const v4i rsSa = make_rsrc(sa, (uint32_t)(M * kblocks * 4));
  const v4i rsSb = make_rsrc(sb, (uint32_t)(((N + BROWS - 1) / BROWS) * kblocks * 4));
  const __amdgpu_buffer_rsrc_t rsD = __builtin_amdgcn_make_buffer_rsrc(D, 0, M * N * 2, kRsrcWord3);

  // tile assignment: as in gemm_fp8_persist_kernel (one rectangle of tiles per XCD)
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

  // operand load plan: as gemm_fp8_mx16_kernel
  const int lrow = kRowsPerInst * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ row_swizzle(lrow);
  const uint32_t inst_rows = (uint32_t)(kRowsPerInst * C::kWaves) * (uint32_t)K;
  // scale load plan (see above)
  const int p = 64 * wave + lane;
  // the lane's parts of its offsets: operand rows (the same for A and B) and its scale
  // (tile row or column times the scale grid's row bytes; kOutOfRange: nothing to load)
  const uint32_t lane_off = (uint32_t)lrow * (uint32_t)K + 16u * lchunk;
  // the scale piece of wave w reads from sa (waves holding p < BM) or sb
  const bool sc_from_a = 64 * wave < C::BM;
  static_assert(C::BM % 64 == 0, "a wave's scale lanes come from one grid");
  uint32_t sc_lane = kOutOfRange;
  if (p < C::BM) {
    const int q = p % C::WTM;
    const int row = (p / C::WTM) * C::WTM + 16 * (q % RT) + q / RT;
    sc_lane = (uint32_t)row * (uint32_t)kblocks * 4u;
  } else if constexpr (BROWS == 1) {
    if (p < C::BM + C::BN) {
      const int q = p - C::BM, qw = q % C::WTN;
      const int col = (q / C::WTN) * C::WTN + 16 * ((qw % (4 * CT)) / 4) + 4 * (qw / (4 * CT)) +
                      (qw % 4);
      sc_lane = (uint32_t)col * (uint32_t)kblocks * 4u;
    }
  } else {
    if (p == C::BM) sc_lane = 0;
  }
  struct Rows { uint32_t a, b, sc; };   // wave-uniform parts for the tile (K block 0)
  auto rows_of = [&](int ti) -> Rows {
    if (ti >= count) return {kOutOfRange, kOutOfRange, kOutOfRange};
    int m0, n0;
    tile_mn(ti, m0, n0);
    uint32_t sc;
    if (sc_from_a) sc = (uint32_t)m0 * (uint32_t)kblocks * 4u;
    else if constexpr (BROWS == 1) sc = (uint32_t)n0 * (uint32_t)kblocks * 4u;
    else sc = (uint32_t)(n0 / BROWS) * (uint32_t)kblocks * 4u;
    return {(uint32_t)m0 * (uint32_t)K, (uint32_t)n0 * (uint32_t)K, sc};
  };
  // load d of stage kb: whole row offsets in the VGPR operand, which the buffer range
  // check tests (rows past M or N read zeros); only the K block's offset, which stays
  // inside a row, in the SGPR operand
  auto dma = [&](int d, uint8_t* slot_mem, Rows r, int kb) {
    const uint32_t k0 = (uint32_t)kb * kStageK;
    // PAD (an odd count of K blocks): the padding stage reads zeros, its scales too
    const bool kin = !PAD || kb < kblocks;
    const uint32_t lds = lds_addr(slot_mem);
    if (d < kInstA)
      dma16_so(rsA, kin ? lane_off + (r.a + d * inst_rows) : kOutOfRange, k0,
               lds + 1024u * wave + 1024u * C::kWaves * d);
    else if (d < kInstA + kInstB)
      dma16_so(rsB, kin ? lane_off + (r.b + (d - kInstA) * inst_rows) : kOutOfRange, k0,
               lds + C::BM * kStageK + 1024u * wave + 1024u * C::kWaves * (d - kInstA));
    else
      dma4(sc_from_a ? rsSa : rsSb,
           (!kin || sc_lane == kOutOfRange || r.sc == kOutOfRange) ? kOutOfRange
                                                                    : sc_lane + r.sc + 4u * kb,
           lds + kSaOff + 256u * wave);
  };
  const int r16 = lane & 15, g4 = lane >> 4;
  const int sw = row_swizzle(r16);
  // the lane's two 16-byte pieces of its fragment row, as offsets into a slot, with the
  // wave's first A row and first B row folded in: a read then adds the slot's base (one
  // add per slot and stage) and a constant that fits the instruction's offset field
  const uint32_t fa0 = (uint32_t)(wm * C::WTM + r16) * kStageK + 16 * ((2 * g4) ^ sw);
  const uint32_t fa1 = (uint32_t)(wm * C::WTM + r16) * kStageK + 16 * ((2 * g4 + 1) ^ sw);
  const uint32_t fb0 = fa0 + (uint32_t)(C::BM + wn * C::WTN - wm * C::WTM) * kStageK;
  const uint32_t fb1 = fa1 + (uint32_t)(C::BM + wn * C::WTN - wm * C::WTM) * kStageK;
  static_assert((C::BM + C::BN) * kStageK < 65536, "row offsets fit the LDS offset field");
  auto rd = [&](uint32_t lo_at, uint32_t hi_at) {
    const v4u lo = lds16(lo_at);
    const v4u hi = lds16(hi_at);
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };
  // a slot's read bases (computed once per stage, opaque to the compiler, so that each
  // read is base + constant and the constant goes in the offset field)
  struct Bases { uint32_t a0, a1, b0, b1; };
  auto slot_addr = [&](const uint8_t* sm) {   // the slot's LDS address, one SGPR
    uint32_t b = lds_addr(sm);
    asm volatile("" : "+s"(b));
    return b;
  };
  auto bases = [&](const uint8_t* sm) {
    const uint32_t b = slot_addr(sm);
    Bases r{b + fa0, b + fa1, b + fb0, b + fb1};
    asm volatile("" : "+v"(r.a0), "+v"(r.a1), "+v"(r.b0), "+v"(r.b1));
    return r;
  };
  auto rdA = [&](const Bases& q, int i) {
    return rd(q.a0 + 16u * i * kStageK, q.a1 + 16u * i * kStageK);
  };
  auto rdB = [&](const Bases& q, int j) {
    return rd(q.b0 + 16u * j * kStageK, q.b1 + 16u * j * kStageK);
  };
  // this stage's scales: fa[i] = sa of the lane's row in tile row i (times sb when B has one
  // scale per tile), fb the lane's column scales when B has one per row
  float fa[RT];
  float fb[BROWS == 1 ? CT * 4 : 1];
  const uint32_t fsa = kSaOff + 4u * (uint32_t)(wm * C::WTM + r16 * RT);
  const uint32_t fsb = kSbOff + 4u * (uint32_t)(wn * C::WTN + g4 * 4 * CT);
  auto rd_scales = [&](const uint8_t* sm) {
    static_assert(RT % 4 == 0, "row scales by 16 bytes");
    uint32_t ba = slot_addr(sm) + fsa;
    asm volatile("" : "+v"(ba));
#pragma unroll
    for (int v = 0; v < RT / 4; ++v) {
      const v4u a4 = lds16(ba + 16u * v);
      fa[4 * v + 0] = __uint_as_float(a4.x); fa[4 * v + 1] = __uint_as_float(a4.y);
      fa[4 * v + 2] = __uint_as_float(a4.z); fa[4 * v + 3] = __uint_as_float(a4.w);
    }
    if constexpr (BROWS == 1) {
      uint32_t bb = slot_addr(sm) + fsb;
      asm volatile("" : "+v"(bb));
#pragma unroll
      for (int j = 0; j < CT; ++j) {
        const v4u b4 = lds16(bb + 16u * j);
        fb[4 * j + 0] = __uint_as_float(b4.x); fb[4 * j + 1] = __uint_as_float(b4.y);
        fb[4 * j + 2] = __uint_as_float(b4.z); fb[4 * j + 3] = __uint_as_float(b4.w);
      }
    } else {
      fb[0] = *reinterpret_cast<const float*>(sm + kSbOff);
    }
  };

  v4f acc[RT][CT];
  v8i Bf0[CT], Bf1[CT], Alo[RH], Ahi[RH];
  // stages per tile: K / 128 rounded up to an even count of at least 4; stages past K
  // (the tail of a K that is not a multiple of 256) load zeros
  const int ns = max(4, (((K + kStageK - 1) / kStageK) + 1) & ~1);
  Rows cur = rows_of(0), nxt = rows_of(1);

  // MFMA x of the stage (x = i CT + j) gives the block's partial sum P; fold() adds it in
  // with its scale. Software-pipelined: MFMA x is issued before the fold of MFMA x - L,
  // L = 2 where registers allow (with L = 1 the fold waits on the matrix core's result;
  // the kernel with a scale per B row holds 16 more scales and keeps L = 1).
  constexpr int L = BROWS == 1 ? 1 : 2;
  auto mfma_x = [&](int x, const v8i* Bc) {
    const int i = x / CT, j = x % CT;
    const v4f z = {};
    const v8i& a = i < RH ? Alo[i] : Ahi[i - RH];
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Bc[j], a, z, 0, 0, 0, 0, 0, 0);
  };
  auto fold = [&](auto FIRST_, int x, const v4f& P) {
    constexpr bool FIRST = decltype(FIRST_)::value != 0;
    const int i = x / CT, j = x % CT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float f;
      if constexpr (BROWS == 1) f = fa[i] * fb[4 * j + r];
      else f = fa[i];                   // sb is folded into fa once per stage
      acc[i][j][r] = FIRST ? P[r] * f : fmaf(P[r], f, acc[i][j][r]);
    }
  };

  auto stage = [&](auto FIRST_, auto LAST_, int s, uint8_t* mine, uint8_t* other, v8i* Bc,
                   v8i* Bn, bool after) {
    constexpr bool LAST = decltype(LAST_)::value != 0;
    constexpr bool FIRST = decltype(FIRST_)::value != 0;
    constexpr int kHalf = RH * CT;       // MFMAs per half stage
    static_assert(kHalf >= L, "fold lag");
    v4f P[L + 1];
    // first half: rows 0 .. RH-1; this stage's scales, then A rows RH .. RT-1, are read
    const Bases qm = bases(mine);
    rd_scales(mine);
#pragma unroll
    for (int i = 0; i < RH; ++i) Ahi[i] = rdA(qm, RH + i);
    if constexpr (BROWS != 1) {
#pragma unroll
      for (int i = 0; i < RT; ++i) fa[i] *= fb[0];
    }
#pragma unroll
    for (int x = 0; x < kHalf; ++x) {
      P[x % (L + 1)] = mfma_x(x, Bc);
      __builtin_amdgcn_sched_barrier(0);
      if (x >= L) fold(FIRST_, x - L, P[(x - L) % (L + 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // own loads of stage s + 1 landed (those of stage s + 2, and after a previous tile
    // its stores, which were issued later, may stay in flight: they retire in order)
    if (FIRST && after)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kDma + kStores) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kDma) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // second half: rows RH .. RT-1, with the loads of stage s + 3 (into `mine`) and the
    // reads of stage s + 1's first fragments in between
    const int gs = s + kSlots;
    const Rows r = gs < ns ? cur : nxt;
    const int kb = gs < ns ? gs : gs - ns;
    constexpr int kReads = CT + RH;
    Bases qo{};
    if constexpr (!LAST) qo = bases(other);
#pragma unroll
    for (int y = 0; y < kHalf; ++y) {
      const int x = kHalf + y;
      P[x % (L + 1)] = mfma_x(x, Bc);
      __builtin_amdgcn_sched_barrier(0);
      fold(FIRST_, x - L, P[(x - L) % (L + 1)]);
#pragma unroll
      for (int d = y * kDma / kHalf; d < (y + 1) * kDma / kHalf; ++d) dma(d, mine, r, kb);
#pragma unroll
      for (int f = y * kReads / kHalf; f < (y + 1) * kReads / kHalf; ++f) {
        if constexpr (!LAST) {
          if (f < CT) Bn[f] = rdB(qo, f);
          else Alo[f - CT] = rdA(qo, f - CT);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int x = 2 * kHalf - L; x < 2 * kHalf; ++x) fold(FIRST_, x, P[x % (L + 1)]);
  };

  // epilogue: as gemm_fp8_mx16_kernel's (the block scales are already applied)
  auto epilogue = [&](int m0, int n0) {
    const int mrow = m0 + wm * C::WTM + r16;
    const int ncol = n0 + wn * C::WTN + 16 * (g4 & 1) + 8 * (g4 >> 1);
    const uint32_t base = ((uint32_t)mrow * (uint32_t)N + (uint32_t)ncol) * 2u;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int m = mrow + 16 * i;
      const bool live = m < M_valid;   // rows past it are written as zeros, whatever
                                       // their sums hold (a select, not a product)
#pragma unroll
      for (int jp = 0; jp < CT / 2; ++jp) {
        const int j = 2 * jp;
        const uint32_t p0j = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        const uint32_t p1j = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        const uint32_t p0k = pack_bf16x2(acc[i][j + 1][0], acc[i][j + 1][1]);
        const uint32_t p1k = pack_bf16x2(acc[i][j + 1][2], acc[i][j + 1][3]);
        const auto w0 = __builtin_amdgcn_permlane16_swap(p0j, p0k, false, false);
        const auto w1 = __builtin_amdgcn_permlane16_swap(p1j, p1k, false, false);
        v4i o = {(int)w0[0], (int)w1[0], (int)w0[1], (int)w1[1]};
        if (!live) o = v4i{0, 0, 0, 0};
        const bool in = m < M && ncol + 32 * jp < N;
        const uint32_t off =
            in ? base + (uint32_t)(16 * i) * (uint32_t)N * 2u + 64u * jp : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(o, rsD, off, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // global stage counter g: stage g lives in slot g % 3
  auto slot_of = [&](int g) { return smem + (g % kSlots) * SB; };
#pragma unroll
  for (int d = 0; d < kDma; ++d) dma(d, smem, cur, 0);
#pragma unroll
  for (int d = 0; d < kDma; ++d) dma(d, smem + SB, cur, 1);
#pragma unroll
  for (int d = 0; d < kDma; ++d) dma(d, smem + 2 * SB, cur, 2);
  wait_vm<2 * kDma>();                 // stage 0 landed
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  int g = 0;                           // global index of the tile's first stage
  auto first_frags = [&]() {
    const Bases q = bases(slot_of(g));
#pragma unroll
    for (int j = 0; j < CT; ++j) Bf0[j] = rdB(q, j);
#pragma unroll
    for (int i = 0; i < RH; ++i) Alo[i] = rdA(q, i);
  };
  first_frags();
  for (int ti = 0; ti < count; ++ti) {
    int cm0, cn0;
    tile_mn(ti, cm0, cn0);
    const bool after = ti > 0;
    // stages 0, 1 | 2 .. ns - 3 | ns - 2, ns - 1 (ns is even and at least 4)
    stage(IC<1>{}, IC<0>{}, 0, slot_of(g), slot_of(g + 1), Bf0, Bf1, after);
    stage(IC<0>{}, IC<0>{}, 1, slot_of(g + 1), slot_of(g + 2), Bf1, Bf0, false);
    for (int s = 2; s < ns - 2; s += 2) {
      stage(IC<0>{}, IC<0>{}, s, slot_of(g + s), slot_of(g + s + 1), Bf0, Bf1, false);
      stage(IC<0>{}, IC<0>{}, s + 1, slot_of(g + s + 1), slot_of(g + s + 2), Bf1, Bf0, false);
    }
    stage(IC<0>{}, IC<0>{}, ns - 2, slot_of(g + ns - 2), slot_of(g + ns - 1), Bf0, Bf1, false);
    stage(IC<0>{}, IC<1>{}, ns - 1, slot_of(g + ns - 1), slot_of(g + ns), Bf1, Bf0, false);
    epilogue(cm0, cn0);
    g += ns;
    first_frags();                     // the next tile's stage 0, published at stage ns - 1
    cur = nxt;
    nxt = rows_of(ti + 2);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // no load may land after exit
}

// ---------------------------------------------------------------------------
// Block-recipe kernel for one weight scale per 128 x 128 block (forward and input
// gradient): 256x256 tiles, 8 waves (two per SIMD) of 128x64, each an 8x4 grid of 16x16
// tiles. gemm_fp8_mx16b_kernel's 256x128 tile is bound by its operand loads; this tile
// loads a third fewer bytes per product. The folds are that kernel's (acc += P * sa * sb
// after every 16x16x128 MFMA, the accumulators in VGPRs); what gives is the fragment
// storage: a wave holds its stage's 4 B fragments and streams the 8 A rows through a ring
// of 4 registers sets, two rows ahead, and replaces each B fragment by the next stage's
// right after its last MFMA.
// Two LDS slots. The barrier comes after 24 of a stage's 32 MFMAs, once every wave has
// read all of the stage's A rows: it publishes stage s + 1 (whose first A rows and B
// fragments are read during the last 8 MFMAs) and frees stage s's slot for the loads of
// stage s + 2, issued during those same 8 MFMAs.
// Scales: lane p = 64 w + l of the workgroup loads the scales of one tile row for p < 256
// and, for p = 256 + c, the weight scale of the tile's column block c.
// SG (a count of K blocks divisible by 4): lane p < 256 loads row p's scales of 4
// consecutive K blocks (16 bytes) once per 4 stages into one of two LDS regions (a quarter
// of the requests of one 4-byte load per stage: the scale loads are scattered, one row
// apart). Else the stage's scales are 4-byte loads behind its operands in the slot, lane p
// holding row 128 (p / 128) + 16 (p % 8) + (p % 128) / 8, so that a lane's 8 row scales
// are neighbours.
template <int BROWS, bool PAD, bool SG>
__global__ void __launch_bounds__(512, 1)
gemm_fp8_mx16bw_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                       const float* __restrict__ sa, const float* __restrict__ sb,
                       uint16_t* __restrict__ D, int M, int N, int K, int M_valid, int tiles_m,
                       int tiles_n, int split_m, int split_n) {
  static_assert(!(PAD && SG), "grouped scales need a K block count divisible by 4");
  static_assert(BROWS == 128 || (BROWS == 1 && SG), "per-row weight scales: grouped loads only");
  constexpr int BM = 256, BN = 256, WM = 2, WN = 4, kWaves = WM * WN, GROUP_M = 8;
  constexpr int WTM = BM / WM, WTN = BN / WN;           // 128 x 64
  constexpr int RT = WTM / 16, CT = WTN / 16;           // 8 x 4
  constexpr int kRing = 4;                              // A row registers
  constexpr int kTileBytes = (BM + BN) * kStageK;       // 64 KB
  constexpr int kScaleOff = kTileBytes;                 // !SG: 4 bytes per lane
  constexpr int SB = kTileBytes + (SG ? 0 : 4 * 64 * kWaves);
  constexpr int kRegion = 16 * 64 * kWaves;             // SG: 16 bytes per lane
  constexpr int kRowsPerInst = 1024 / kStageK;          // 8 rows of 128 bytes
  constexpr int kInstA = BM / (kRowsPerInst * kWaves);  // 4
  constexpr int kInstB = BN / (kRowsPerInst * kWaves);  // 4
  constexpr int kDma = kInstA + kInstB + (SG ? 0 : 1);  // + the stage's scale piece
  constexpr int kStores = RT * CT / 2;
  constexpr int kMf = RT * CT;                          // MFMAs per stage
  constexpr int kBarrierAt = (RT - 2) * CT;             // MFMAs before the barrier
  constexpr int kTail = kMf - kBarrierAt;
  constexpr int L = 2;                                  // fold lag (MFMAs)
  constexpr int kGroup = 4;                             // SG: stages per scale load
  static_assert(kDma + 1 + kStores <= 63, "memory counts");
  static_assert(2 * SB + (SG ? 2 * kRegion : 0) <= 160 * 1024, "LDS");
  static_assert(WTN <= 128 && 128 % WTN == 0, "one weight scale per wave");
  static_assert(kRing == 4 && RT % kRing == 0, "ring slots: row i in i % 4, and so the next "
                "stage's rows 0 and 1 go where rows RT - 4 and RT - 3 were");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * SB + (SG ? 2 * kRegion : 0)];
  uint8_t* const slot0 = smem;
  uint8_t* const slot1 = smem + SB;
  uint8_t* const regions = smem + 2 * SB;               // SG

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int kblocks = K / kStageK;
  const v4i rsA = make_rsrc(A, (uint32_t)(M * K));
  const v4i rsB = make_rsrc(B, (uint32_t)(N * K));
  const v4i rsSa = make_rsrc(sa, (uint32_t)(M * kblocks * 4));
  const v4i rsSb = make_rsrc(sb, (uint32_t)(((N + BROWS - 1) / BROWS) * kblocks * 4));
  const __amdgpu_buffer_rsrc_t rsD = __builtin_amdgcn_make_buffer_rsrc(D, 0, M * N * 2, kRsrcWord3);

  // tile assignment: as in gemm_fp8_persist_kernel (one rectangle of tiles per XCD)
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
    const int per_group = GROUP_M * bnc;
    const int group = lid / per_group;
    const int first_m = group * GROUP_M;
    const int gsize = min(bmc - first_m, GROUP_M);
    const int in_group = lid - group * per_group;
    m0 = (bm0 + first_m + in_group % gsize) * BM;
    n0 = (bn0 + in_group / gsize) * BN;
  };

  // operand load plan: as gemm_fp8_mx16_kernel's
  const int lrow = kRowsPerInst * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ row_swizzle(lrow);
  const uint32_t inst_rows = (uint32_t)(kRowsPerInst * kWaves) * (uint32_t)K;
  const uint32_t lane_off = (uint32_t)lrow * (uint32_t)K + 16u * lchunk;
  // scale load plan (see above): waves 0 .. 3 read sa, wave 4 the two weight scales
  const int p = 64 * wave + lane;
  const bool sc_from_a = wave < BM / 64;
  uint32_t sc_lane = kOutOfRange;
  if (p < BM) {
    const int row = SG ? p : (p / WTM) * WTM + 16 * (p % RT) + (p % WTM) / RT;
    sc_lane = (uint32_t)row * (uint32_t)kblocks * 4u;
  } else if (p < BM + (BN + BROWS - 1) / BROWS) {
    sc_lane = (uint32_t)(p - BM) * (uint32_t)kblocks * 4u;
  }
  struct Rows { uint32_t a, b, sc; };   // wave-uniform parts for the tile (K block 0)
  auto rows_of = [&](int ti) -> Rows {
    if (ti >= count) return {kOutOfRange, kOutOfRange, kOutOfRange};
    int m0, n0;
    tile_mn(ti, m0, n0);
    const uint32_t sc = sc_from_a ? (uint32_t)m0 * (uint32_t)kblocks * 4u
                                  : (uint32_t)(n0 / BROWS) * (uint32_t)kblocks * 4u;
    return {(uint32_t)m0 * (uint32_t)K, (uint32_t)n0 * (uint32_t)K, sc};
  };
  auto sc_off = [&](Rows r, int kb) {
    return (sc_lane == kOutOfRange || r.sc == kOutOfRange) ? kOutOfRange
                                                           : sc_lane + r.sc + 4u * kb;
  };
  // load d of stage kb (whole row offsets in the VGPR operand, which the buffer range check
  // tests: rows past M or N read zeros; the K block's offset in the SGPR operand)
  auto dma = [&](int d, uint8_t* slot_mem, Rows r, int kb) {
    const uint32_t k0 = (uint32_t)kb * kStageK;
    // PAD (an odd count of K blocks): the padding stage reads zeros, its scales too
    const bool kin = !PAD || kb < kblocks;
    const uint32_t lds = lds_addr(slot_mem);
    if (d < kInstA)
      dma16_so(rsA, kin ? lane_off + (r.a + d * inst_rows) : kOutOfRange, k0,
               lds + 1024u * wave + 1024u * kWaves * d);
    else if (d < kInstA + kInstB)
      dma16_so(rsB, kin ? lane_off + (r.b + (d - kInstA) * inst_rows) : kOutOfRange, k0,
               lds + BM * kStageK + 1024u * wave + 1024u * kWaves * (d - kInstA));
    else if constexpr (!SG)
      dma4(sc_from_a ? rsSa : rsSb, kin ? sc_off(r, kb) : kOutOfRange,
           lds + kScaleOff + 256u * wave);
  };
  // SG: the scales of K blocks kb .. kb + 3 (kb % 4 == 0) into region `rg` (0 or 1)
  auto dma_scales = [&](int rg, Rows r, int kb) {
    dma16(sc_from_a ? rsSa : rsSb, sc_off(r, kb),
          lds_addr(regions) + (uint32_t)(rg * kRegion) + 1024u * wave);
  };

  const int r16 = lane & 15, g4 = lane >> 4;
  const int sw = row_swizzle(r16);
  // the lane's two 16-byte pieces of its fragment row, as offsets into a slot
  const uint32_t fa0 = (uint32_t)(wm * WTM + r16) * kStageK + 16 * ((2 * g4) ^ sw);
  const uint32_t fa1 = (uint32_t)(wm * WTM + r16) * kStageK + 16 * ((2 * g4 + 1) ^ sw);
  const uint32_t fb0 = fa0 + (uint32_t)(BM + wn * WTN - wm * WTM) * kStageK;
  const uint32_t fb1 = fa1 + (uint32_t)(BM + wn * WTN - wm * WTM) * kStageK;
  static_assert((BM + BN) * kStageK <= 65536, "row offsets fit the LDS offset field");
  auto rd = [&](uint32_t lo_at, uint32_t hi_at) {
    const v4u lo = lds16(lo_at);
    const v4u hi = lds16(hi_at);
    v8i v;
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    return v;
  };
  struct Bases { uint32_t a0, a1, b0, b1; };
  auto slot_addr = [&](const uint8_t* sm) {   // the slot's LDS address, one SGPR
    uint32_t b = lds_addr(sm);
    asm volatile("" : "+s"(b));
    return b;
  };
  auto bases = [&](const uint8_t* sm) {
    const uint32_t b = slot_addr(sm);
    Bases q{b + fa0, b + fa1, b + fb0, b + fb1};
    asm volatile("" : "+v"(q.a0), "+v"(q.a1), "+v"(q.b0), "+v"(q.b1));
    return q;
  };
  auto rdA = [&](const Bases& q, int i) {
    return rd(q.a0 + 16u * i * kStageK, q.a1 + 16u * i * kStageK);
  };
  auto rdB = [&](const Bases& q, int j) {
    return rd(q.b0 + 16u * j * kStageK, q.b1 + 16u * j * kStageK);
  };
  // this stage's scales: fa[i] = sa of the lane's row in tile row i, times the wave's
  // weight scale when B has one per 128x128 block; with one per B row (BROWS = 1),
  // fb[4 j + r] = sb of the lane's column 4 g + r of tile column j
  // PF (grouped scales, one weight scale per 128x128 block): a stage's scales are read in
  // the previous stage's tail, after its barrier, into the other of two register sets, so
  // that the stage's first folds do not wait for them
  constexpr bool PF = SG && BROWS == 128;
  float fa[RT];
  float fa2[PF ? RT : 1];
  float fb[BROWS == 1 ? 4 * CT : 1];
  const int pa = wm * WTM + r16 * (SG ? 1 : RT);   // the lane's first row-scale lane
  const int pb = BROWS == 1 ? BM + wn * WTN + 4 * g4 : BM + (wn * WTN) / 128;
  auto rd_scales = [&](float* fs, const uint8_t* sm, int rg, int q) {
    static_assert(RT % 4 == 0, "row scales by 16 bytes");
    float fbw;
    if constexpr (SG) {
      // lane p's 4 K blocks at 16 p .. 16 p + 15 of the region; this stage's is the q-th.
      // Tile row i of the lane is lane pa + 16 i, so the 16 rows a read serves lie 16
      // bytes apart: 16 distinct banks.
      typedef const __attribute__((address_space(3))) float lds_f32;
      uint32_t ba = slot_addr(regions) + (uint32_t)(rg * kRegion) + 16u * pa + 4u * q;
      asm volatile("" : "+v"(ba));
#pragma unroll
      for (int i = 0; i < RT; ++i) fs[i] = *(lds_f32*)(uintptr_t)(ba + 256u * i);
      uint32_t bb = slot_addr(regions) + (uint32_t)(rg * kRegion) + 16u * pb + 4u * q;
      asm volatile("" : "+v"(bb));
      if constexpr (BROWS == 1) {
        // column 16 j + 4 g + r of the wave at 16 (BM + wn WTN + 16 j + 4 g + r) + 4 q: the 4
        // lane groups read 4 addresses 64 bytes apart, the 16 lanes of a group one address
#pragma unroll
        for (int j = 0; j < CT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) fb[4 * j + r] = *(lds_f32*)(uintptr_t)(bb + 256u * j + 16u * r);
        return;
      } else {
        fbw = *(lds_f32*)(uintptr_t)bb;
      }
    } else {
      uint32_t ba = slot_addr(sm) + kScaleOff + 4u * pa;
      asm volatile("" : "+v"(ba));
#pragma unroll
      for (int v = 0; v < RT / 4; ++v) {
        const v4u a4 = lds16(ba + 16u * v);
        fs[4 * v + 0] = __uint_as_float(a4.x); fs[4 * v + 1] = __uint_as_float(a4.y);
        fs[4 * v + 2] = __uint_as_float(a4.z); fs[4 * v + 3] = __uint_as_float(a4.w);
      }
      fbw = *reinterpret_cast<const float*>(sm + kScaleOff + 4 * pb);
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) fs[i] *= fbw;
  };

  v4f acc[RT][CT];
  v8i Bq[CT], Aq[kRing];
  const int ns = max(4, (kblocks + 1) & ~1);   // stages per tile: even, at least 4
  Rows cur = rows_of(0), nxt = rows_of(1);
  int gq = 0;                                  // SG: scale groups begun before this tile

  auto fold = [&](auto FIRST_, int x, const v4f& P, const float* fs) {
    constexpr bool FIRST = decltype(FIRST_)::value != 0;
    const int i = x / CT, j = x % CT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float f = BROWS == 1 ? fs[i] * fb[4 * j + r] : fs[i];
      acc[i][j][r] = FIRST ? P[r] * f : fmaf(P[r], f, acc[i][j][r]);
    }
  };

  // stage s from slot `mine`; `other` receives stage s + 1 (published by this stage's
  // barrier). On entry Bq holds the stage's B fragments and Aq[0], Aq[1] its A rows 0, 1.
  // AFTER: the first stage after a tile's epilogue, whose stores were issued after the
  // loads of stage s + 1 and may stay in flight at the barrier. SG: Q = s % 4; the tail of a
  // stage with Q = 0 loads the scales of stages s + 4 .. s + 7 into the other region, the
  // one that stages s - 4 .. s - 1 read (done by every wave at this stage's barrier).
  auto stage = [&](auto FIRST_, auto Q_, int s, uint8_t* mine, uint8_t* other, bool after) {
    constexpr int Q = decltype(Q_)::value;
    const v4f z = {};
    v4f P[L + 1];
    const Bases qm = bases(mine);
    const int rg = (gq + s / kGroup) & 1;
    float* const fs = (PF && Q % 2 == 1) ? fa2 : fa;     // this stage's scales
    if constexpr (!PF) rd_scales(fa, mine, rg, Q);
    const int gs = s + 2;
    const Rows r = gs < ns ? cur : nxt;
    const int kb = gs < ns ? gs : gs - ns;
    const int gs4 = s + kGroup;
    const Rows r4 = gs4 < ns ? cur : nxt;
    const int kb4 = gs4 < ns ? gs4 : gs4 - ns;
    Bases qo{};
#pragma unroll
    for (int x = 0; x < kMf; ++x) {
      const int i = x / CT, j = x % CT;
      P[x % (L + 1)] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Bq[j], Aq[i % kRing], z,
                                                                        0, 0, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (x >= L) fold(FIRST_, x - L, P[(x - L) % (L + 1)], fs);
      // this stage's A rows, two ahead
      if (j == 0 && i + 2 < RT) Aq[(i + 2) % kRing] = rdA(qm, i + 2);
      if (x == kBarrierAt - 1) {
        // every A row of this stage read; stage s + 1 landed (own loads); then for all
        if (after) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kStores) : "memory");
        else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        qo = bases(other);
      }
      if (x >= kBarrierAt) {
        const int y = x - kBarrierAt;
        // the loads of stage s + 2 into this stage's slot
#pragma unroll
        for (int d = y * kDma / kTail; d < (y + 1) * kDma / kTail; ++d) dma(d, mine, r, kb);
        if constexpr (SG && Q == 0)
          if (y == kTail - 1) dma_scales(rg ^ 1, r4, kb4);
        // PF: the next stage's scales (the next group's region after Q = 3)
        if constexpr (PF)
          if (y == 1) rd_scales(Q % 2 == 1 ? fa : fa2, nullptr, Q == 3 ? rg ^ 1 : rg, (Q + 1) % 4);
        // the next stage's A rows 0 and 1, into the ring slots of rows RT - 4, RT - 3
        if (y == 0) Aq[0] = rdA(qo, 0);
        if (y == CT) Aq[1] = rdA(qo, 1);
        // B fragment j after its last MFMA
        if (i == RT - 1) Bq[j] = rdB(qo, j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int x = kMf - L; x < kMf; ++x) fold(FIRST_, x, P[x % (L + 1)], fs);
  };

  auto epilogue = [&](int m0, int n0) {
    const int mrow = m0 + wm * WTM + r16;
    const int ncol = n0 + wn * WTN + 16 * (g4 & 1) + 8 * (g4 >> 1);
    const uint32_t base = ((uint32_t)mrow * (uint32_t)N + (uint32_t)ncol) * 2u;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int m = mrow + 16 * i;
      const bool live = m < M_valid;   // rows past it are written as zeros, whatever
                                       // their sums hold (a select, not a product)
#pragma unroll
      for (int jp = 0; jp < CT / 2; ++jp) {
        const int j = 2 * jp;
        const uint32_t p0j = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        const uint32_t p1j = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        const uint32_t p0k = pack_bf16x2(acc[i][j + 1][0], acc[i][j + 1][1]);
        const uint32_t p1k = pack_bf16x2(acc[i][j + 1][2], acc[i][j + 1][3]);
        const auto w0 = __builtin_amdgcn_permlane16_swap(p0j, p0k, false, false);
        const auto w1 = __builtin_amdgcn_permlane16_swap(p1j, p1k, false, false);
        v4i o = {(int)w0[0], (int)w1[0], (int)w0[1], (int)w1[1]};
        if (!live) o = v4i{0, 0, 0, 0};
        const bool in = m < M && ncol + 32 * jp < N;
        const uint32_t off =
            in ? base + (uint32_t)(16 * i) * (uint32_t)N * 2u + 64u * jp : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(o, rsD, off, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (SG) dma_scales(0, cur, 0);
#pragma unroll
  for (int d = 0; d < kDma; ++d) dma(d, slot0, cur, 0);
#pragma unroll
  for (int d = 0; d < kDma; ++d) dma(d, slot1, cur, 1);
  wait_vm<kDma>();                     // stage 0 landed (and SG: the first scale group)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  {
    const Bases q = bases(slot0);
#pragma unroll
    for (int j = 0; j < CT; ++j) Bq[j] = rdB(q, j);
    Aq[0] = rdA(q, 0);
    Aq[1] = rdA(q, 1);
    if constexpr (PF) rd_scales(fa, nullptr, 0, 0);   // stage 0 of the first tile
  }
  for (int ti = 0; ti < count; ++ti) {
    int cm0, cn0;
    tile_mn(ti, cm0, cn0);
    if constexpr (SG) {
      // stages in fours (ns is a multiple of 4)
      stage(IC<1>{}, IC<0>{}, 0, slot0, slot1, ti > 0);
      stage(IC<0>{}, IC<1>{}, 1, slot1, slot0, false);
      stage(IC<0>{}, IC<2>{}, 2, slot0, slot1, false);
      stage(IC<0>{}, IC<3>{}, 3, slot1, slot0, false);
      for (int s = 4; s < ns; s += 4) {
        stage(IC<0>{}, IC<0>{}, s, slot0, slot1, false);
        stage(IC<0>{}, IC<1>{}, s + 1, slot1, slot0, false);
        stage(IC<0>{}, IC<2>{}, s + 2, slot0, slot1, false);
        stage(IC<0>{}, IC<3>{}, s + 3, slot1, slot0, false);
      }
      gq += ns / kGroup;
    } else {
      // stages 0, 1 | 2 .. ns - 1 in pairs (ns is even and at least 4)
      stage(IC<1>{}, IC<0>{}, 0, slot0, slot1, ti > 0);
      stage(IC<0>{}, IC<0>{}, 1, slot1, slot0, false);
      for (int s = 2; s < ns; s += 2) {
        stage(IC<0>{}, IC<0>{}, s, slot0, slot1, false);
        stage(IC<0>{}, IC<0>{}, s + 1, slot1, slot0, false);
      }
    }
    epilogue(cm0, cn0);
    cur = nxt;
    nxt = rows_of(ti + 2);
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");   // no load may land after exit
}

// ---------------------------------------------------------------------------
// One tile per workgroup; K steps past the end are zero loads, so the loop body
// (unrolled by STAGES) needs no branches. Tensorwise scaling only.
template <class C>
__global__ void __launch_bounds__(C::kThreads, 1)
gemm_fp8_pipe_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                     const float* __restrict__ sa, const float* __restrict__ sb,
                     const uint16_t* __restrict__ bias, uint16_t* __restrict__ D, int M, int N,
                     int K, int M_valid, int tiles_n) {
  static_assert(!C::BLOCK, "tensorwise only");
  constexpr int SB = C::kStageBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t s0[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[SB];
  __shared__ __attribute__((aligned(1024))) uint8_t s2[C::STAGES > 2 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t s3[C::STAGES > 3 ? SB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t s4[C::STAGES > 4 ? SB : 16];

  Tile<C> T;
  T.init(A, B, sa, sb, D, M, N, K, M_valid);
  T.bias = bias;
  const int m0 = (blockIdx.x / tiles_n) * C::BM;
  const int n0 = (blockIdx.x % tiles_n) * C::BN;
  const auto tb = T.base(true, m0, n0);
  constexpr int kWaitN = C::kLoadsPerStage * (C::STAGES - 2);
  auto step = [&](uint8_t* cur, uint8_t* refill, int kk_refill) {
    wait_vm_lgkm<kWaitN>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    T.issue(refill, tb, kk_refill);
    T.template compute<0>(cur);
  };
  T.issue(s0, tb, 0);
  if constexpr (C::STAGES > 2) T.issue(s1, tb, 1);
  if constexpr (C::STAGES > 3) T.issue(s2, tb, 2);
  if constexpr (C::STAGES > 4) T.issue(s3, tb, 3);
  constexpr int R = C::STAGES - 1;
  // ring[i] = stage of step i of the loop body (i < 2 STAGES)
#define FP8LIN_P(i) pick<i, C::STAGES>(s0, s1, s2, s3, s4)
  uint8_t* const ring[10] = {FP8LIN_P(0), FP8LIN_P(1), FP8LIN_P(2), FP8LIN_P(3), FP8LIN_P(4),
                             FP8LIN_P(5), FP8LIN_P(6), FP8LIN_P(7), FP8LIN_P(8), FP8LIN_P(9)};
#undef FP8LIN_P
  for (int kk = 0; kk < T.nk; kk += C::STAGES) {
    step(ring[0], ring[R], kk + R);
    step(ring[1], ring[R + 1], kk + R + 1);
    if constexpr (C::STAGES > 2) step(ring[2], ring[R + 2], kk + R + 2);
    if constexpr (C::STAGES > 3) step(ring[3], ring[R + 3], kk + R + 3);
    if constexpr (C::STAGES > 4) step(ring[4], ring[R + 4], kk + R + 4);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  T.epilogue(m0, n0);
}

// ---------------------------------------------------------------------------
// One rectangle of output tiles per XCD (workgroups are dispatched round-robin over the 8
// XCDs): of the splits of the tile grid into pm x pn = 8 equal rectangles, the one whose
// rectangle spans the fewest A + B panel rows, so the tiles running together on an XCD
// share the most operand bytes in its L2. No split (0, 0) if none divides the grid.
void xcd_split(int tiles_m, int tiles_n, int bm, int bn, int& split_m, int& split_n) {
  int best = 1 << 30;
  split_m = split_n = 0;
  for (int pm = 1; pm <= 8; pm *= 2) {
    const int pn = 8 / pm;
    if (tiles_m % pm || tiles_n % pn) continue;
    const int cost = (tiles_m / pm) * bm + (tiles_n / pn) * bn;
    if (cost < best) { best = cost; split_m = pm; split_n = pn; }
  }
}

template <class C>
hipError_t run_pipe(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                    const uint16_t* bias, uint16_t* D, int M, int N, int K, int M_valid,
                    hipStream_t s) {
  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  const int64_t tiles = (int64_t)tiles_m * tiles_n;
  hipLaunchKernelGGL(gemm_fp8_pipe_kernel<C>, dim3((unsigned)tiles), dim3(C::kThreads), 0, s, A,
                     B, sa, sb, bias, D, M, N, K, M_valid, tiles_n);
  return hipGetLastError();
}

// One workgroup per CU at most (the LDS ring takes most of a CU).
constexpr int kMaxWorkgroups = 256;

template <class C>
hipError_t run_persist(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                       const uint16_t* bias, uint16_t* D, int M, int N, int K, int M_valid,
                       hipStream_t s) {
  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  const int tiles = tiles_m * tiles_n;
  const int grid = tiles < kMaxWorkgroups ? tiles : kMaxWorkgroups;
  // one rectangle of tiles per XCD: the split with the fewest A+B panel rows per XCD
  int split_m = 0, split_n = 0;
  if (grid == kMaxWorkgroups) xcd_split(tiles_m, tiles_n, C::BM, C::BN, split_m, split_n);
  hipLaunchKernelGGL(gemm_fp8_persist_kernel<C>, dim3((unsigned)grid), dim3(C::kThreads), 0, s, A,
                     B, sa, sb, bias, D, M, N, K, M_valid, tiles_m, tiles_n, split_m, split_n);
  return hipGetLastError();
}

// Tensorwise: 256x256 tiles, 8 waves of 128x64 (four 32 KiB stages) for large problems;
// 128x128 tiles, 4 waves of 64x64 for small ones. Two-stage variants take step counts
// that are even but not multiples of four.
template <int AF> using TwBig = PCfg<256, 256, 2, 4, 4, 0, 8, 0, AF>;
template <int AF> using TwBig2 = PCfg<256, 256, 2, 4, 2, 0, 8, 0, AF>;
template <int AF> using TwSmall = PCfg<128, 128, 2, 2, 4, 0, 8, 0, AF>;
template <int AF> using TwSmall2 = PCfg<128, 128, 2, 2, 2, 0, 8, 0, AF>;
// 16x16x128 kernel: 256x256 tiles, 4 waves of 128x128 (its own LDS plan); 224-row or
// 224-column tiles where they split the output into whole rounds of 256 tiles better.
template <int AF> using TwMx16 = PCfg<256, 256, 2, 2, 2, 0, 8, 0, AF>;
template <int AF> using TwMx16M224 = PCfg<224, 256, 2, 2, 2, 0, 8, 0, AF>;
template <int AF> using TwMx16N224 = PCfg<256, 224, 2, 2, 2, 0, 8, 0, AF>;
// Block recipe: the partial sums need a second set of accumulators, so 256x128 tiles.
// With one weight scale per 128 rows, 8 waves of 64x64; with a B scale per row (wgrad),
// 8 waves of 128x32, so that a lane needs 16 B scales per 128-wide K block, not 32.
template <int BROWS> using Blk4 =
    PCfg<256, 128, BROWS == 1 ? 2 : 4, BROWS == 1 ? 4 : 2, 4, 0, 8, BROWS>;
template <int BROWS> using Blk2 =
    PCfg<256, 128, BROWS == 1 ? 2 : 4, BROWS == 1 ? 4 : 2, 2, 0, 8, BROWS>;

template <class C>
hipError_t run_mx16(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                    const uint16_t* bias, uint16_t* D, int M, int N, int K, int M_valid,
                    hipStream_t s) {
  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  const int tiles = tiles_m * tiles_n;
  const int grid = tiles < kMaxWorkgroups ? tiles : kMaxWorkgroups;
  int split_m = 0, split_n = 0;
  if (grid == kMaxWorkgroups) xcd_split(tiles_m, tiles_n, C::BM, C::BN, split_m, split_n);
  const dim3 g((unsigned)grid), b(C::kThreads);
  const bool tail = K % (2 * kStageK) != 0;
  // the kernel leaves rows at or past M_valid alone (they are past its output range):
  // their zeros come from a fill kernel
  if (M_valid < M) {
    const hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(D + (int64_t)M_valid * N), 0u,
                                         (int64_t)(M - M_valid) * N / 2, s);
    if (e != hipSuccess) return e;
  }
  if (bias == nullptr && !tail)
    hipLaunchKernelGGL((gemm_fp8_mx16_kernel<C, false, false>), g, b, 0, s, A, B, sa, sb, bias, D,
                       M, N, K, M_valid, tiles_m, tiles_n, split_m, split_n);
  else if (bias == nullptr)
    hipLaunchKernelGGL((gemm_fp8_mx16_kernel<C, true, false>), g, b, 0, s, A, B, sa, sb, bias, D,
                       M, N, K, M_valid, tiles_m, tiles_n, split_m, split_n);
  else if constexpr (C::AFMT != 0)
    return hipErrorInvalidValue;   // the host never asks for a bias with e5m2 codes
  else if (!tail)
    hipLaunchKernelGGL((gemm_fp8_mx16_kernel<C, false, true>), g, b, 0, s, A, B, sa, sb, bias, D,
                       M, N, K, M_valid, tiles_m, tiles_n, split_m, split_n);
  else
    hipLaunchKernelGGL((gemm_fp8_mx16_kernel<C, true, true>), g, b, 0, s, A, B, sa, sb, bias, D,
                       M, N, K, M_valid, tiles_m, tiles_n, split_m, split_n);
  return hipGetLastError();
}

template <class C4, class C2>
hipError_t run_tensorwise(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                          const uint16_t* bias, uint16_t* D, int M, int N, int K, int M_valid,
                          hipStream_t s) {
  const int nk = (K + kBKS - 1) / kBKS;
  if (nk % 4 == 0) return run_persist<C4>(A, B, sa, sb, bias, D, M, N, K, M_valid, s);
  if (nk % 2 == 0) return run_persist<C2>(A, B, sa, sb, bias, D, M, N, K, M_valid, s);
  return run_pipe<C2>(A, B, sa, sb, bias, D, M, N, K, M_valid, s);
}

template <class C>
hipError_t run_mx16b(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                     uint16_t* D, int M, int N, int K, int M_valid, hipStream_t s) {
  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  const int tiles = tiles_m * tiles_n;
  const int grid = tiles < kMaxWorkgroups ? tiles : kMaxWorkgroups;
  int split_m = 0, split_n = 0;
  if (grid == kMaxWorkgroups) xcd_split(tiles_m, tiles_n, C::BM, C::BN, split_m, split_n);
  // an odd count of K blocks ends each tile with a padding stage (stages come in pairs)
  if ((K / kStageK) % 2 == 0)
    hipLaunchKernelGGL((gemm_fp8_mx16b_kernel<C, false>), dim3((unsigned)grid), dim3(C::kThreads),
                       0, s, A, B, sa, sb, D, M, N, K, M_valid, tiles_m, tiles_n, split_m,
                       split_n);
  else
    hipLaunchKernelGGL((gemm_fp8_mx16b_kernel<C, true>), dim3((unsigned)grid), dim3(C::kThreads),
                       0, s, A, B, sa, sb, D, M, N, K, M_valid, tiles_m, tiles_n, split_m,
                       split_n);
  return hipGetLastError();
}

// block recipe on the 16x16x128 kernel: 256x128 tiles, 8 waves of 64x64
template <int BROWS> using BlkMx16 = PCfg<256, 128, 4, 2, 2, 0, 8, BROWS>;

// the 256x256 block-recipe kernel loads scales 4 K blocks (16 bytes) at a time
bool bw_grouped(const float* sa, const float* sb, int K) {
  return (K / kStageK) % 4 == 0 &&
         ((reinterpret_cast<uintptr_t>(sa) | reinterpret_cast<uintptr_t>(sb)) & 15) == 0;
}

template <int BROWS>
hipError_t run_mx16bw(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                      uint16_t* D, int M, int N, int K, int M_valid, hipStream_t s) {
  const int tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
  const int tiles = tiles_m * tiles_n;
  const int grid = tiles < kMaxWorkgroups ? tiles : kMaxWorkgroups;
  int split_m = 0, split_n = 0;
  if (grid == kMaxWorkgroups) xcd_split(tiles_m, tiles_n, 256, 256, split_m, split_n);
  // a count of K blocks divisible by 4 (and 16-byte aligned scale grids): scales in groups
  // of 4 stages; an odd count ends each tile with a padding stage (stages come in pairs)
  const dim3 g((unsigned)grid), b(512);
  if (bw_grouped(sa, sb, K))
    hipLaunchKernelGGL((gemm_fp8_mx16bw_kernel<BROWS, false, true>), g, b, 0, s, A, B, sa, sb, D, M,
                       N, K, M_valid, tiles_m, tiles_n, split_m, split_n);
  else if constexpr (BROWS == 1)
    return hipErrorInvalidValue;   // the host takes this kernel only with grouped scales
  else if ((K / kStageK) % 2 == 0)
    hipLaunchKernelGGL((gemm_fp8_mx16bw_kernel<BROWS, false, false>), g, b, 0, s, A, B, sa, sb, D,
                       M, N, K, M_valid, tiles_m, tiles_n, split_m, split_n);
  else
    hipLaunchKernelGGL((gemm_fp8_mx16bw_kernel<BROWS, true, false>), g, b, 0, s, A, B, sa, sb, D, M,
                       N, K, M_valid, tiles_m, tiles_n, split_m, split_n);
  return hipGetLastError();
}

template <int BROWS>
hipError_t run_block(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                     uint16_t* D, int M, int N, int K, int M_valid, hipStream_t s) {
  // K is a multiple of 128 (checked on the host), so the step count is even
  // (the per-row B scale variant keeps two stages: four run out of registers)
  if (K >= 4 * kStageK) {
    // enough 256x256 tiles to fill the chip: the wide-tile kernel (with one scale per B row
    // only when the scales load in groups of 4 K blocks)
    if ((int64_t)((M + 255) / 256) * ((N + 255) / 256) >= kMaxWorkgroups &&
        (BROWS == 128 || bw_grouped(sa, sb, K)))
      return run_mx16bw<BROWS>(A, B, sa, sb, D, M, N, K, M_valid, s);
    return run_mx16b<BlkMx16<BROWS>>(A, B, sa, sb, D, M, N, K, M_valid, s);
  }
  const int nk = K / kBKS;
  if constexpr (BROWS != 1)
    if (nk % 4 == 0)
      return run_persist<Blk4<BROWS>>(A, B, sa, sb, nullptr, D, M, N, K, M_valid, s);
  return run_persist<Blk2<BROWS>>(A, B, sa, sb, nullptr, D, M, N, K, M_valid, s);
}

// Tensorwise dispatch for one A format.
// The 16x16x128 kernel for K of at least 512 when the output spans at least 64 of its
// tiles; else the 32x32x64 persistent kernel with 256x256 tiles, or 128x128 tiles for
// small outputs.
template <int AF>
hipError_t run_tensorwise_fmt(const uint8_t* A, const uint8_t* B, const float* sa,
                              const float* sb, const uint16_t* bias, uint16_t* D, int m, int n,
                              int k, int mv, hipStream_t s) {
  // the 16x16x128 kernel's output offsets are 32-bit for rows up to M + 257
  const bool mx16_ok = k >= 4 * kStageK && ((int64_t)m + 257) * n * 2 < ((int64_t)1 << 31);
  const bool big = (int64_t)m * n >= (int64_t)2048 * 2048;
  if (big && mx16_ok) {
    // Beyond one round of 256x256 tiles, the tile shape with the shortest makespan:
    // rounds of kMaxWorkgroups tiles times the tile's area (896 tiles of 256x256 take 4
    // rounds, the last half empty; 1024 of 224x256 take 4 full ones, each 7/8 as long).
    auto cost = [&](int bm, int bn) {
      const int64_t tiles = (int64_t)((m + bm - 1) / bm) * ((n + bn - 1) / bn);
      return ((tiles + kMaxWorkgroups - 1) / kMaxWorkgroups) * bm * bn;
    };
    const int64_t c0 = cost(256, 256), cm = cost(224, 256), cn = cost(256, 224);
    if (c0 > 256 * 256) {
      if (cm < c0 && cm <= cn)
        return run_mx16<TwMx16M224<AF>>(A, B, sa, sb, bias, D, m, n, k, mv, s);
      if (cn < c0) return run_mx16<TwMx16N224<AF>>(A, B, sa, sb, bias, D, m, n, k, mv, s);
    }
    return run_mx16<TwMx16<AF>>(A, B, sa, sb, bias, D, m, n, k, mv, s);
  }
  if (!big)
    return run_tensorwise<TwSmall<AF>, TwSmall2<AF>>(A, B, sa, sb, bias, D, m, n, k, mv, s);
  return run_tensorwise<TwBig<AF>, TwBig2<AF>>(A, B, sa, sb, bias, D, m, n, k, mv, s);
}

}  // namespace

hipError_t launch_gemm_fp8(const uint8_t* A, const uint8_t* B, const float* sa, const float* sb,
                           const uint16_t* bias, uint16_t* D, int64_t M, int64_t N, int64_t K,
                           int64_t M_valid, bool block_scaled, int b_rows_per_scale, bool a_e5m2,
                           hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  // an empty contraction (e.g. a weight gradient over no tokens): every sum is +0, so the
  // valid rows hold the bias (if any)
  if (K == 0) {
    if (bias != nullptr) return launch_bias_rows(bias, D, M, N, M_valid, s);
    return launch_fill_u32(reinterpret_cast<uint32_t*>(D), 0u, M * N / 2, s);
  }
  const int m = (int)M, n = (int)N, k = (int)K, mv = (int)M_valid;
  if (block_scaled) {
    if (a_e5m2) return hipErrorInvalidValue;
    if (b_rows_per_scale == 1) return run_block<1>(A, B, sa, sb, D, m, n, k, mv, s);
    return run_block<128>(A, B, sa, sb, D, m, n, k, mv, s);
  }
  if (a_e5m2) {
    if (bias != nullptr) return hipErrorInvalidValue;
    return run_tensorwise_fmt<1>(A, B, sa, sb, nullptr, D, m, n, k, mv, s);
  }
  return run_tensorwise_fmt<0>(A, B, sa, sb, bias, D, m, n, k, mv, s);
}

}  // namespace fp8lin
