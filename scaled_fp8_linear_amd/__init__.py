"""MI355X (gfx950) scaled FP8 linear layer.

The compute path is ``libfp8lin.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fp8lin.h``); this package is its thin Python binding
(``_abi``) plus the host-side delayed-scaling schedule (``state``). PyTorch is
used for device memory and streams only. Importing works without the built
library; calling any entry point without it raises.
"""
from ._abi import (FP8_A_E5M2, FP8_AMAX_ACCUMULATE, FP8_BLOCK_1x128, FP8_E5M2, FP8_BLOCK_128x128, FP8_SCALE_CLEAR_AMAX,
                   FP8_SCALE_FROM_AMAX, FP8_SCALE_RECORD, FP8_SCALE_REFRESH, FP8_TENSORWISE,
                   FP8_LAYOUT_BSHD, FP8_LAYOUT_THD, Fp8Error, Slot, fp8_align_multiple,
                   fp8_bias_grad, fp8_last_error, fp8_pad_varlen, fp8_unpad_varlen,
                   fp8_linear_dgrad, fp8_linear_fwd, fp8_linear_fwd_current, fp8_linear_wgrad,
                   fp8_pad_tokens,
                   fp8_quantize_amax, fp8_scale_update, fp8_version, load)
from .autograd import Fp8Linear, fp8_autocast, fp8_state
from .state import DelayedScalingLinear

__all__ = ["fp8_quantize_amax", "fp8_scale_update", "fp8_linear_fwd", "fp8_linear_dgrad",
           "fp8_linear_fwd_current",
           "fp8_bias_grad",
           "fp8_linear_wgrad", "fp8_pad_tokens", "fp8_last_error", "fp8_version", "load",
           "Fp8Error", "Slot", "DelayedScalingLinear", "FP8_TENSORWISE", "FP8_BLOCK_1x128",
           "FP8_BLOCK_128x128", "FP8_SCALE_FROM_AMAX", "FP8_SCALE_RECORD", "FP8_SCALE_REFRESH",
           "FP8_AMAX_ACCUMULATE", "FP8_SCALE_CLEAR_AMAX", "FP8_E5M2", "FP8_A_E5M2",
           "Fp8Linear", "fp8_autocast", "fp8_align_multiple", "fp8_pad_varlen",
           "fp8_unpad_varlen", "FP8_LAYOUT_THD", "FP8_LAYOUT_BSHD",
           "fp8_state"]
