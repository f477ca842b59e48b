// Device helpers shared by the gfx950 kernels of the scaled FP8 linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8lin {

constexpr float kE4M3Max = 448.0f;     // largest finite OCP e4m3 value
constexpr float kE5M2Max = 57344.0f;   // largest finite OCP e5m2 value (1.75 * 2^15)
constexpr uint32_t kF32InfBits = 0x7F800000u;
constexpr float kAmaxFloor = 1e-12f;   // lower clamp of amax before 448/amax

// Streaming (non-temporal) 16/8-byte loads and stores: the quantize pass reads and
// writes every byte once, so it keeps them out of the caches' reuse set.
typedef unsigned fp8lin_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned fp8lin_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const fp8lin_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const fp8lin_u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_stream16(void* p, uint4 v) {
  const fp8lin_u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<fp8lin_u32x4*>(p));
}
__device__ __forceinline__ void st_stream8(void* p, uint32_t a, uint32_t b) {
  const fp8lin_u32x2 w = {a, b};
  __builtin_nontemporal_store(w, reinterpret_cast<fp8lin_u32x2*>(p));
}

// bf16 pair packed in a dword -> two floats (exact).
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Clamp to +-448 (the e4m3 range; +-inf too) with one median-of-three, so the hardware
// converter only ever sees values inside the range and its own overflow behaviour never
// matters. A NaN comes out of the clamp as some finite value: quant4 marks NaN products
// itself.
__device__ __forceinline__ float sat_e4m3(float v) {
  return __builtin_amdgcn_fmed3f(v, -kE4M3Max, kE4M3Max);
}

// Four floats -> four codes in one dword (a in the low byte). gfx950's
// v_cvt_pk_fp8_f32 converts to the OCP E4M3 format, rounding to nearest even.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(a), sat_e4m3(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(c), sat_e4m3(d), lo, true);
}

// OCP e5m2 (sign, 5 exponent bits with bias 15, 2 mantissa bits; 0x7C is infinity,
// 0x7D..0x7F NaN), used for gradients in the hybrid format. Clamped to +-57344 as e4m3
// is to +-448.
__device__ __forceinline__ float sat_e5m2(float v) {
  return __builtin_amdgcn_fmed3f(v, -kE5M2Max, kE5M2Max);
}

// Four floats -> four OCP e5m2 codes in one dword (a in the low byte); gfx950's
// v_cvt_pk_bf8_f32 rounds to nearest even.
__device__ __forceinline__ uint32_t cvt4_e5m2(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_bf8_f32(sat_e5m2(a), sat_e5m2(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(sat_e5m2(c), sat_e5m2(d), lo, true);
}

// Sign bits of four bf16 values (elements 0,1 in d0, 2,3 in d1) placed at
// bit 7 of bytes 0..3.
__device__ __forceinline__ uint32_t sign_bytes(uint32_t d0, uint32_t d1) {
  return ((d0 >> 8) & 0x80u) | ((d0 >> 16) & 0x8000u) | ((d1 << 8) & 0x800000u) |
         (d1 & 0x80000000u);
}

// Four bf16 inputs (packed in d0, d1) times their multipliers -> four codes in the format
// FMT (0 e4m3, 1 e5m2). A NaN product (a NaN input, or a multiplier that makes one) is
// encoded as 0x7F with the sign of its input; the test is one compare per product, and
// the fix-up runs only in lanes that have one.
template <int FMT>
__device__ __forceinline__ uint32_t quant4_fmt(uint32_t d0, uint32_t d1, float s0, float s1,
                                               float s2, float s3) {
  const float a = bf16_lo(d0) * s0, b = bf16_hi(d0) * s1;
  const float c = bf16_lo(d1) * s2, d = bf16_hi(d1) * s3;
  uint32_t codes = FMT == 0 ? cvt4_e4m3(a, b, c, d) : cvt4_e5m2(a, b, c, d);
  const bool na = __builtin_isnan(a), nb = __builtin_isnan(b);
  const bool nc = __builtin_isnan(c), nd = __builtin_isnan(d);
  if (__builtin_expect(na | nb | nc | nd, 0)) {
    const uint32_t m = (na ? 0xFFu : 0u) | (nb ? 0xFF00u : 0u) | (nc ? 0xFF0000u : 0u) |
                       (nd ? 0xFF000000u : 0u);
    codes = (codes & ~m) | (m & (0x7F7F7F7Fu | sign_bytes(d0, d1)));
  }
  return codes;
}

__device__ __forceinline__ uint32_t quant4(uint32_t d0, uint32_t d1, float s0, float s1, float s2,
                                           float s3) {
  return quant4_fmt<0>(d0, d1, s0, s1, s2, s3);
}

// Two floats -> two bf16 in one dword (a in the low half), round to nearest even
// (gfx950's v_cvt_pk_bf16_f32).
typedef __bf16 fp8lin_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const fp8lin_bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// float -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > kF32InfBits) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Scale pair from an amax: a = max(amax, 1e-12) keeping NaN, then two IEEE
// divisions (this translation unit is built without fast-math, so '/' is the
// correctly rounded float32 division).
// fmax is the format's largest finite value (448 for e4m3, 57344 for e5m2).
__device__ __forceinline__ void scale_pair(float amax, float* scale, float* scale_inv,
                                           float fmax = kE4M3Max) {
  float a = (amax < kAmaxFloor) ? kAmaxFloor : amax;   // NaN < x is false: NaN kept
  *scale = a / fmax;
  *scale_inv = fmax / a;
}

// Wavefront (64 lanes) max of an unsigned value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

}  // namespace fp8lin
