// Delayed-scaling bookkeeping on the device (no host synchronization).
//
// AstrAI, astrai/extension/fp8_state.py:
//  * _update_delayed_scale: a = clamp_min(amax, 1e-12); scale = a/448,
//    scale_inv = 448/a, written for the next call;
//  * FP8TensorMeta.record: hist[idx] = amax (the host keeps idx);
//  * FP8TensorMeta.refresh: m = max(hist); if m > 0: scale = m/448,
//    scale_inv = 448/m.
// Each quotient is one correctly rounded float32 division (no fast-math in
// this translation unit, so '/' lowers to the IEEE division sequence). For
// gradients kept in e5m2 the format maximum 57344 takes the place of 448.
#include "common.h"
#include "launch.h"

namespace fp8lin {

namespace {

// clear: amax[0] = +0 once read (the next quantize pass folds its max into it)
__global__ void scale_from_amax_kernel(float* __restrict__ amax, float* __restrict__ scale,
                                       float* __restrict__ scale_inv, int clear, float fmax) {
  const float a = amax[0];
  float s, si;
  scale_pair(a, &s, &si, fmax);
  scale[0] = s;
  scale_inv[0] = si;
  if (clear) amax[0] = 0.0f;
}

__global__ void record_kernel(float* __restrict__ amax, float* __restrict__ hist, int pos,
                              int clear) {
  hist[pos] = amax[0];
  if (clear) amax[0] = 0.0f;
}

// One wavefront; len is small (16 for the pages' schedule).
__global__ void refresh_kernel(const float* __restrict__ hist, int len, float* __restrict__ scale,
                               float* __restrict__ scale_inv, float fmax) {
  const int lane = threadIdx.x;
  // max with NaN propagation, as torch.max does: track NaN separately
  float m = 0.0f;
  bool any = false, nan = false;
  for (int i = lane; i < len; i += 64) {
    float v = hist[i];
    nan |= (v != v);
    m = any ? fmaxf(m, v) : v;
    any = true;
  }
  // reduce across the wavefront (lanes with no entry contribute -inf)
  float r = any ? m : -__builtin_inff();
  for (int off = 32; off > 0; off >>= 1) r = fmaxf(r, __shfl_xor(r, off, 64));
  int anynan = __any(nan);
  if (lane == 0 && !anynan && r > 0.0f) {
    scale[0] = r / fmax;
    scale_inv[0] = fmax / r;
  }
}

}  // namespace

hipError_t launch_scale_update(int mode, float* amax, bool clear_amax, float* hist, int32_t len,
                               int32_t pos, float* scale, float* scale_inv, bool e5m2,
                               hipStream_t s) {
  const float fmax = e5m2 ? kE5M2Max : kE4M3Max;
  switch (mode) {
    case 0:
      hipLaunchKernelGGL(scale_from_amax_kernel, dim3(1), dim3(1), 0, s, amax, scale, scale_inv,
                         (int)clear_amax, fmax);
      break;
    case 1:
      hipLaunchKernelGGL(record_kernel, dim3(1), dim3(1), 0, s, amax, hist, (int)pos,
                         (int)clear_amax);
      break;
    case 2:
      hipLaunchKernelGGL(refresh_kernel, dim3(1), dim3(64), 0, s, (const float*)hist, (int)len,
                         scale, scale_inv, fmax);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fp8lin
