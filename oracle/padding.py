"""Token-count padding (test infrastructure only).

* SpecForge PR 2, Conclusion, Constraints bullet: float8 GEMMs need the token
  count of every micro-batch to be a multiple of 16 (the failure it quotes is a
  token count of 3858, which is not).
* NeMo PR 15754, review thread on BSHD padding: the forward appends
  ``pad = (-T) % seq_multiple`` tokens.

Reading: the padding goes at the end of the concatenated (packed THD) batch,
the padded rows are zero, and they are excluded from amax and written as zero
in the outputs of the forward and dgrad GEMMs.
"""
from __future__ import annotations

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
