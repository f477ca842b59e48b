"""Token-count padding (test infrastructure only).

* SpecForge PR 2, Conclusion, Constraints bullet: float8 GEMMs need the token
  count of every micro-batch to be a multiple of 16 (the failure it quotes is a
  token count of 3858, which is not).
* NeMo PR 15754, review thread on BSHD padding: the forward appends
  ``pad = (-T) % seq_multiple`` tokens.

Reading: the padding goes at the end of the concatenated (packed THD) batch,
the padded rows are zero, and they are excluded from amax and written as zero
in the outputs of the forward and dgrad GEMMs.

Alignment under tensor / sequence / context parallelism (NeMo PR 15754, the
same review thread): every rank's share of the tokens must be a multiple of
the FP8 multiple, and a sequence split over ranks must split evenly.

* THD (packed): the helper the thread quotes pads the total to
  ``8 * cp_size * tp_size`` (TE's multiple 8); with this library's multiple 16
  that is ``16 * cp * tp``. Reading (not printed on the pages): with cp > 1
  each sequence is cut into 2 * cp chunks for load-balanced context
  parallelism, so each sequence is padded to a multiple of 2 * cp.
* BSHD: sequence parallelism splits T over tp ranks (T % tp == 0) and each
  rank's GEMM sees M = B * T / tp tokens, which must be a multiple of the FP8
  multiple. Padding T to a multiple of ``base * tp`` alone is not enough (the
  thread's case: B = 16, tp = 4 asks only for a multiple of 2); T must be a
  multiple of lcm(tp, base * tp / gcd(B, base * tp)).
"""
from __future__ import annotations

import math

import numpy as np

TOKEN_MULTIPLE = 16


def pad_amount(T: int, multiple: int = TOKEN_MULTIPLE) -> int:
    """``(-T) % multiple`` with Python's non-negative modulo."""
    if multiple <= 0:
        raise ValueError("multiple must be positive")
    return (-int(T)) % int(multiple)


def padded_count(T: int, multiple: int = TOKEN_MULTIPLE) -> int:
    return int(T) + pad_amount(T, multiple)


def pad_rows(x: np.ndarray, multiple: int = TOKEN_MULTIPLE) -> np.ndarray:
    """Append zero rows to a [T, cols] array so its row count is a multiple."""
    T = x.shape[0]
    out = np.zeros((padded_count(T, multiple),) + x.shape[1:], dtype=x.dtype)
    out[:T] = x
    return out


THD, BSHD = 0, 1


def align_multiples(layout: int, batch: int = 1, tp: int = 1, cp: int = 1,
                    base: int = TOKEN_MULTIPLE) -> tuple[int, int]:
    """(per-sequence multiple, total multiple) of a layout.

    THD: (2 * cp if cp > 1 else 1, base * cp * tp). BSHD (every sequence padded
    to the same length T; no context parallelism): (lcm(tp, base * tp / gcd(B,
    base * tp)), 1) -- the total B * T is then a multiple of base * tp.
    """
    if tp < 1 or cp < 1 or base < 1 or batch < 1:
        raise ValueError("batch, tp, cp and base must be positive")
    if layout == THD:
        return (2 * cp if cp > 1 else 1), base * cp * tp
    if layout == BSHD:
        if cp != 1:
            raise ValueError("BSHD alignment is defined for tensor/sequence parallelism only")
        need = base * tp // math.gcd(batch, base * tp)
        return tp * need // math.gcd(tp, need), 1
    raise ValueError(f"unknown layout {layout}")


def pad_varlen(x: np.ndarray, seqlens, seq_multiple: int = 1, total_multiple: int = 1):
    """Pack sequences with per-sequence padding: sequence i (``seqlens[i]`` rows of the
    packed [sum(seqlens), cols] array ``x``, in order) is copied to row ``cu_pad[i]`` of the
    output and followed by zero rows up to a multiple of ``seq_multiple``; the total is then
    zero-padded to a multiple of ``total_multiple``. Returns ``(x_pad, cu_pad)`` with
    ``cu_pad`` of length len(seqlens) + 1 (its last entry the padded sequences' end, before
    the total padding)."""
    lens = [int(v) for v in seqlens]
    cu_pad = [0]
    for L in lens:
        cu_pad.append(cu_pad[-1] + padded_count(L, seq_multiple))
    T_pad = padded_count(cu_pad[-1], total_multiple)
    out = np.zeros((T_pad,) + x.shape[1:], dtype=x.dtype)
    src = 0
    for i, L in enumerate(lens):
        for r in range(L):
            out[cu_pad[i] + r] = x[src + r]
        src += L
    return out, np.array(cu_pad, dtype=np.int64)


def unpad_varlen(x_pad: np.ndarray, seqlens, cu_pad) -> np.ndarray:
    """The inverse gather: the rows of every sequence, without its padding, packed."""
    lens = [int(v) for v in seqlens]
    out = np.zeros((sum(lens),) + x_pad.shape[1:], dtype=x_pad.dtype)
    dst = 0
    for i, L in enumerate(lens):
        for r in range(L):
            out[dst + r] = x_pad[int(cu_pad[i]) + r]
        dst += L
    return out
