"""Tensorwise quantize + amax (test infrastructure only).

What is computed (AstrAI ``fp8_state.py``):

* the module comment fixes the GEMM layout ``D = A_SCALE * B_SCALE * A * B``
  with per-tensor scales amax/448, and says quantization divides by the scale,
  i.e. multiplies by ``1/scale`` -- the stored ``scale_inv``;
* ``fp8_linear_forward``'s docstring says the quantize kernel emits the
  current amax of its input ("free atomic amax", no extra abs/max reduce).

So, for a bf16 tensor X and the float32 multiplier ``scale_inv``:

* ``Q[r, c] = e4m3(float32(X[r, c]) * scale_inv)`` -- one float32 multiply
  (round to nearest even), then the E4M3 encoder of ``oracle.e4m3``;
* a NaN product (a NaN input, or an invalid multiplier) gives the NaN code
  0x7F with the SIGN OF THE INPUT x: IEEE 754 does not fix the sign of a NaN
  that an operation returns, so the input's sign is the one portable choice;
* ``Q_t`` is the byte-for-byte transpose of ``Q`` (the copy the backward
  GEMMs read; a reading of the hot path, not printed on the pages);
* ``amax = max |X[r, c]|`` over the valid rows, as float32. bf16 -> float32 is
  exact, so the maximum is exact; it is 0 for an all-zero input and NaN if any
  valid element is NaN (reading: NaN propagates, as ``torch.max`` does).

The gradients of the hybrid format are coded in E5M2 (``oracle.e5m2``) by
the same steps, with the multiplier 57344/amax.

Rows ``r >= rows_valid`` are padding (NeMo PR 15754 review thread: tokens
appended by ``pad = (-T) % seq_multiple``): they are not read, do not enter
amax, and their codes are written as 0x00.
"""
from __future__ import annotations

import numpy as np

from . import e4m3, e5m2

CODECS = {"e4m3": e4m3, "e5m2": e5m2}


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: bf16 is the top half of float32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def amax(x_bits: np.ndarray, rows_valid: int | None = None) -> np.float32:
    """max |x| over rows < rows_valid of a bf16 [rows, cols] tensor."""
    x = bf16_to_f32(x_bits)
    if rows_valid is not None:
        x = x[:rows_valid]
    if x.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(x)))


def encode_product(x: np.ndarray, v: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """Codes of the float32 products ``v`` of inputs ``x`` (float32, same shape):
    the format's encoder, except that a NaN product takes the sign of its input."""
    codec = CODECS[fmt]
    code = codec.encode(v)
    nan_code = np.where(np.signbit(x), codec.NAN_CODE | codec.SIGN_BIT, codec.NAN_CODE)
    return np.where(np.isnan(v), nan_code, code).astype(np.uint8)


def quantize_values(x_bits: np.ndarray, scale_inv, fmt: str = "e4m3") -> np.ndarray:
    """Codes (``fmt`` "e4m3" or "e5m2") of float32(x) * scale_inv, elementwise."""
    x = bf16_to_f32(x_bits)
    with np.errstate(invalid="ignore", over="ignore"):
        v = x * np.float32(scale_inv)            # float32 * float32 -> float32 (RNE)
    return encode_product(x, v, fmt)


def quantize_tensorwise(x_bits: np.ndarray, scale_inv, rows_valid: int | None = None,
                        fmt: str = "e4m3"):
    """Return ``(q, q_t, amax)`` for a bf16 [rows, cols] tensor.

    ``q`` is uint8 [rows, cols], ``q_t`` uint8 [cols, rows], ``amax`` float32;
    ``fmt`` "e5m2" codes the hybrid format's gradients.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows = x_bits.shape[0]
    rv = rows if rows_valid is None else int(rows_valid)
    q = np.zeros(x_bits.shape, dtype=np.uint8)
    q[:rv] = quantize_values(x_bits[:rv], scale_inv, fmt)
    return q, np.ascontiguousarray(q.T), amax(x_bits, rv)
