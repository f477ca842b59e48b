"""Block-scaled recipe: 1x128 activation/gradient tiles, 128x128 weight tiles.

Test infrastructure only.

Sources: NeMo PR 15754 (its 2-GPU run uses TransformerEngine's FP8
"recipe=block"; the review thread contrasts the block/current recipes with
delayed scaling). The pages give no formulas for the block recipe beyond its
name, so the readings below restate the tensorwise rules of AstrAI
``fp8_state.py`` per tile:

* every tile has its own float32 scale ``max(tile_amax, 1e-12) / 448`` and
  multiplier ``448 / max(tile_amax, 1e-12)``, computed from the tile's own
  amax in the same pass (current scaling, no delay);
* activations and gradients use 1x128 tiles that run along the GEMM's
  contraction index; a transposed copy (the wgrad operands, which contract
  over tokens) is therefore quantized again with 1x128 tiles along the token
  index; weights use 128x128 tiles, and their transposed copy reuses the same
  tiles (the codes transpose, the scale grid transposes);
* the GEMM applies the scales per 128-wide contraction block:
  ``D[m, n] = sum_kb sA[m, kb] * sB[n, kb] * sum_{k in kb} A[m, k] * B[n, k]``.

Padded rows (``r >= rows_valid``) are not read, do not enter any tile amax and
are written as 0x00.
"""
from __future__ import annotations

import numpy as np

from . import e4m3
from .quantize import bf16_to_f32, encode_product
from .scaling import AMAX_FLOOR, E4M3_MAX

BLOCK = 128


def tile_scales(tile_amax: np.ndarray):
    """Vectorized scale_from_amax for a grid of tile amaxes (float32 IEEE)."""
    a = np.asarray(tile_amax, dtype=np.float32)
    a = np.where(np.isnan(a) | (a >= AMAX_FLOOR), a, AMAX_FLOOR).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        scale = (a / E4M3_MAX).astype(np.float32)
        scale_inv = (E4M3_MAX / a).astype(np.float32)
    return scale, scale_inv


def _valid_mask(rows: int, cols: int, rows_valid: int | None) -> np.ndarray:
    rv = rows if rows_valid is None else int(rows_valid)
    return (np.arange(rows) < rv)[:, None] & np.ones((1, cols), dtype=bool)


def _quantize_row_tiles(xf: np.ndarray, valid: np.ndarray):
    """1x128 tiles along the last index of a float32 [R, C] array."""
    R, C = xf.shape
    assert C % BLOCK == 0
    t = np.abs(np.where(valid, xf, np.float32(0.0))).reshape(R, C // BLOCK, BLOCK)
    tile_amax = np.max(t, axis=2).astype(np.float32)          # NaN propagates
    scale, scale_inv = tile_scales(tile_amax)
    with np.errstate(invalid="ignore", over="ignore"):
        v = xf * np.repeat(scale_inv, BLOCK, axis=1)           # float32 multiply
    q = np.where(valid, encode_product(xf, v), np.uint8(0)).astype(np.uint8)
    return q, tile_amax, scale


def quantize_1x128(x_bits: np.ndarray, rows_valid: int | None = None):
    """Activation/gradient [R, C]: returns q, q_t and their scale grids.

    * ``q`` [R, C] with ``scale`` [R, C/128] and ``amax`` [R, C/128]: tiles
      along C (the contraction index of forward and dgrad);
    * ``q_t`` [C, R] with ``scale_t`` [C, R/128]: the transposed copy,
      quantized again with tiles along R (the contraction index of wgrad).
    """
    xf = bf16_to_f32(x_bits)
    R, C = xf.shape
    assert R % BLOCK == 0 and C % BLOCK == 0
    valid = _valid_mask(R, C, rows_valid)
    q, amax, scale = _quantize_row_tiles(xf, valid)
    q_t, _, scale_t = _quantize_row_tiles(np.ascontiguousarray(xf.T),
                                          np.ascontiguousarray(valid.T))
    return q, q_t, amax, scale, scale_t


def quantize_128x128(w_bits: np.ndarray):
    """Weight [R, C]: 128x128 tiles; returns q, q_t, amax, scale, scale_t."""
    wf = bf16_to_f32(w_bits)
    R, C = wf.shape
    assert R % BLOCK == 0 and C % BLOCK == 0
    t = np.abs(wf).reshape(R // BLOCK, BLOCK, C // BLOCK, BLOCK)
    tile_amax = np.max(t, axis=(1, 3)).astype(np.float32)
    scale, scale_inv = tile_scales(tile_amax)
    full_inv = np.repeat(np.repeat(scale_inv, BLOCK, axis=0), BLOCK, axis=1)
    with np.errstate(invalid="ignore", over="ignore"):
        q = encode_product(wf, wf * full_inv)
    return q, np.ascontiguousarray(q.T), tile_amax, scale, np.ascontiguousarray(scale.T)


def block_scaled_gemm(qa, qb, sa, sb, b_rows_per_scale: int) -> np.ndarray:
    """``D = sum_kb (sA[:, kb] outer sB[:, kb]) * S_kb`` in float64.

    ``sa`` is [M, K/128] (one scale per row and block); ``sb`` is
    [N / b_rows_per_scale, K/128] (1 for 1x128 tiles, 128 for 128x128 tiles).
    Each ``S_kb`` is exact (see ``oracle.gemm``); the scale products and the
    sum over blocks are float64.
    """
    da = e4m3.decode(qa)
    db = e4m3.decode(qb)
    M, K = da.shape
    N = db.shape[0]
    assert K % BLOCK == 0 and db.shape[1] == K
    sa64 = np.asarray(sa, dtype=np.float32).astype(np.float64)
    sb64 = np.repeat(np.asarray(sb, dtype=np.float32).astype(np.float64),
                     b_rows_per_scale, axis=0)
    assert sa64.shape == (M, K // BLOCK) and sb64.shape == (N, K // BLOCK)
    D = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // BLOCK):
        ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
        D += np.outer(sa64[:, kb], sb64[:, kb]) * (da[:, ks] @ db[:, ks].T)
    return D


def dequant_rows(q, s, rows_per_scale: int) -> np.ndarray:
    """Dequantized float64 operand for block scales (s is [R/rows_per_scale, K/128])."""
    s64 = np.repeat(np.repeat(np.asarray(s, dtype=np.float32).astype(np.float64),
                              rows_per_scale, axis=0), BLOCK, axis=1)
    return e4m3.decode(q) * s64


def block_error_bound(qa, qb, sa, sb, b_rows_per_scale: int, rel: float = 1e-2):
    da = dequant_rows(qa, sa, 1)
    db = dequant_rows(qb, sb, b_rows_per_scale)
    return rel * np.outer(np.sqrt((da * da).sum(1)), np.sqrt((db * db).sum(1)))


def block_fp32_bound(qa, qb, sa, sb, b_rows_per_scale: int):
    """``(D, bound)``: ``block_scaled_gemm`` and a tight bound on ``|D_gpu - D|`` for a
    kernel that forms each block's partial sum in float32 from zero (n_b products, any
    order, partial sums at most ``A_b = sum_{k in b} |a_k b_k|``), multiplies it by the
    float32 product ``w_b`` of its two scales and adds it to a float32 accumulator (one
    rounding each for the scale product and the fused multiply-add), then rounds to bf16.
    With u = 2**-23 (any faithful float32 rounding), ``Q_b`` the exact result through
    block b and ``T_b`` the block's group-truncation term of ``oracle.gemm`` (the matrix
    instruction's aligned groups of 8), the accumulator is within
    ``sum_b |w_b| (u (n_b + 1) A_b + 2**-10 T_b) + u sum_b |Q_b|``, over
    ``1 - u (K + blocks)``, of D; bf16 rounding adds at most 2**-8 of the value."""
    import torch
    from .gemm import BF16_HALF_ULP, F32_U, FLUSH_FLOOR, GROUP_LOSS, MATRIX_GROUP, group_pow2_max
    da = torch.from_numpy(e4m3.decode(qa))
    db = torch.from_numpy(e4m3.decode(qb))
    M, K = da.shape
    N = db.shape[0]
    assert K % BLOCK == 0 and db.shape[1] == K
    nb = K // BLOCK
    sa64 = torch.from_numpy(np.asarray(sa, dtype=np.float32).astype(np.float64))
    sb64 = torch.from_numpy(np.repeat(np.asarray(sb, dtype=np.float32).astype(np.float64),
                                      b_rows_per_scale, axis=0))
    assert tuple(sa64.shape) == (M, nb) and tuple(sb64.shape) == (N, nb)
    ga = torch.from_numpy(group_pow2_max(qa))
    gb = torch.from_numpy(group_pow2_max(qb))
    gpb = BLOCK // MATRIX_GROUP                    # groups per block
    Q = torch.zeros((M, N), dtype=torch.float64)
    E = torch.zeros((M, N), dtype=torch.float64)
    G = torch.zeros((M, N), dtype=torch.float64)
    W = torch.zeros((M, N), dtype=torch.float64)
    for kb in range(nb):
        ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
        gs = slice(kb * gpb, (kb + 1) * gpb)
        a, b = da[:, ks], db[:, ks]
        w = torch.outer(sa64[:, kb], sb64[:, kb])   # exact: two 24-bit significands
        wA = w.abs() * (a.abs() @ b.abs().T)
        Q.add_(w * (a @ b.T))
        E.add_(wA * (BLOCK + 1)).add_(Q.abs())
        G.add_(w.abs() * (ga[:, gs] @ gb[:, gs].T))
        W.add_(wA)
    # float64's own rounding of the products w * S_b and of the running sum
    e_acc = F32_U * E / (1.0 - F32_U * (K + nb)) + GROUP_LOSS * G + 2.0 ** -50 * nb * W
    bound = e_acc + BF16_HALF_ULP * (Q.abs() + e_acc) + FLUSH_FLOOR
    return Q.numpy(), bound.numpy()
