"""The bias of the linear layer, in float64 (test infrastructure only).

Source: AstrAI ``fp8_state.py``, ``fp8_linear_forward(x, w, bias)``: the bias goes to the
scaled forward kernel together with the operands; ``fp8_linear_backward``'s ``masks``
select the bias gradient among the outputs.

Reading (the pages print no formula for either): the forward output is the scaled product
plus the bias broadcast over the rows, ``y[m, n] = D[m, n] + bias[n]`` for the valid rows
(padded rows stay 0), rounded once to bf16; the bias gradient is the column sum of the
output gradient over the valid rows, ``db[n] = sum_{m < rows_valid} g[m, n]``.

Tolerances for the GPU (bf16 output, float32 arithmetic):
* forward: the GEMM bound of ``gemm.error_bound`` plus ``2**-8 |bias[n]|`` (the one bf16
  rounding of D + bias, whose share for D the GEMM bound already covers);
* bias gradient: ``2**-8 |db[n]|`` for the bf16 rounding plus
  ``(rows_valid + 32) 2**-24 sum_m |g[m, n]|`` for float32 sums of that many terms.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def add_bias(D: np.ndarray, bias_bits: np.ndarray, rows_valid: int | None = None) -> np.ndarray:
    """``D + bias`` over the valid rows; rows past ``rows_valid`` are 0."""
    y = np.asarray(D, dtype=np.float64) + bf16_to_f64(bias_bits)[None, :]
    if rows_valid is not None:
        y[int(rows_valid):] = 0.0
    return y


def bias_bound(bias_bits: np.ndarray) -> np.ndarray:
    """Extra forward tolerance per column: ``2**-8 |bias[n]|``."""
    return np.abs(bf16_to_f64(bias_bits)) * 2.0 ** -8


def bias_grad(g_bits: np.ndarray, rows_valid: int | None = None) -> np.ndarray:
    """``db[n] = sum over the valid rows m of g[m, n]`` in float64."""
    g = bf16_to_f64(g_bits)
    rv = g.shape[0] if rows_valid is None else int(rows_valid)
    return g[:rv].sum(axis=0) if rv > 0 else np.zeros(g.shape[1])


def bias_grad_bound(g_bits: np.ndarray, rows_valid: int | None = None) -> np.ndarray:
    """GPU tolerance per column for ``bias_grad``."""
    g = bf16_to_f64(g_bits)
    rv = g.shape[0] if rows_valid is None else int(rows_valid)
    s_abs = np.abs(g[:rv]).sum(axis=0) if rv > 0 else np.zeros(g.shape[1])
    return np.abs(bias_grad(g_bits, rv)) * 2.0 ** -8 + (rv + 32) * 2.0 ** -24 * s_abs
