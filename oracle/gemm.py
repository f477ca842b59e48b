"""The scaled FP8 GEMM, exactly, in float64 (test infrastructure only).

Source: AstrAI ``fp8_state.py`` module comment, "D = A_SCALE * B_SCALE * A * B":
the GEMM multiplies the e4m3 operands as they are and folds both per-tensor
(dequant) scales in afterwards.

Convention: both operands are stored with the contraction index last,
``D[m, n] = sA * sB * sum_k A[m, k] * B[n, k]``. The three GEMMs of a linear
layer ``y = x W^T`` are instances of it:

* forward  y  = sx sw  Qx  . Qw^T     (A = Qx  [M,K],  B = Qw   [N,K])
* dgrad    dx = sg sw  Qg  . Qw       (A = Qg  [M,N],  B = Qw^T [K,N])
* wgrad    dW = sg sx  Qg^T. Qx       (A = Qg^T[N,M],  B = Qx^T [K,M])

Exactness: every finite e4m3 value is a multiple of 2**-9 with magnitude at
most 448 < 2**9, so a product is a multiple of 2**-18 below 2**18 and a sum of
K products stays below K * 2**18. For K < 2**17 every partial sum is a
multiple of 2**-18 below 2**35, which float64 (53 bits) holds exactly; so the
float64 matrix product is exact whatever order BLAS adds in.

Hybrid format (E5M2 gradients as the first operand of dgrad and wgrad):
an E5M2 value is a multiple of 2**-16 below 2**16, so a product with an E4M3
value is a multiple of 2**-25 below 2**25 and a sum no longer fits 53 bits in
general. The float64 product is then exact for K <= 8 and otherwise within
K * 2**-52 * sum_k |a_k b_k| of the exact sum, some ten orders of magnitude
inside the tolerance below.

Tolerance (the target the GPU result is judged by): per element,
``|D_gpu - D| <= 1e-2 * ||dqA[m, :]||_2 * ||dqB[n, :]||_2`` with the
dequantized operands ``dq = decode(Q) * s`` in float64.
"""
from __future__ import annotations

import numpy as np

from . import e4m3, e5m2

EXACT_K_LIMIT = 1 << 17
REL_TOL = 1e-2
CODECS = {"e4m3": e4m3, "e5m2": e5m2}


def unscaled_product(qa: np.ndarray, qb: np.ndarray, a_fmt: str = "e4m3") -> np.ndarray:
    """``S[m, n] = sum_k decode(qa)[m, k] * decode(qb)[n, k]`` in float64 (exact for
    E4M3 operands; ``a_fmt`` "e5m2" decodes A as E5M2)."""
    qa = np.asarray(qa, dtype=np.uint8)
    qb = np.asarray(qb, dtype=np.uint8)
    assert qa.shape[1] == qb.shape[1], "contraction dims differ"
    assert qa.shape[1] < EXACT_K_LIMIT, "float64 is exact only for K < 2**17"
    return CODECS[a_fmt].decode(qa) @ e4m3.decode(qb).T


def scaled_gemm(qa: np.ndarray, qb: np.ndarray, sa, sb, a_fmt: str = "e4m3") -> np.ndarray:
    """``D = S * (float64(sA) * float64(sB))`` for per-tensor scales."""
    return unscaled_product(qa, qb, a_fmt) * (np.float64(np.float32(sa)) *
                                              np.float64(np.float32(sb)))


def row_norms(q: np.ndarray, s, fmt: str = "e4m3") -> np.ndarray:
    """||decode(q)[i, :] * s||_2 in float64 for each row i (per-tensor scale)."""
    d = CODECS[fmt].decode(q) * np.float64(np.float32(s))
    return np.sqrt(np.sum(d * d, axis=1))


def error_bound(qa, qb, sa, sb, rel: float = REL_TOL, a_fmt: str = "e4m3") -> np.ndarray:
    """Per-element tolerance ``rel * ||dqA[m,:]|| * ||dqB[n,:]||``."""
    return rel * np.outer(row_norms(qa, sa, a_fmt), row_norms(qb, sb))


def bf16_round(d: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (via float32, both round to nearest even).

    Used only to describe the output type; parity is judged against the
    float64 result within the tolerance above.
    """
    f = np.asarray(d, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), rounded)
