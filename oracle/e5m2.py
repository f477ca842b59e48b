"""OCP E5M2 codec (test infrastructure: only tests, smoke and the CPU baseline use it).

The gradient half of the hybrid FP8 format. The pages name E4M3 only; E5M2 is
the other OCP 8-bit format, taken here for gradients (wider range, one
mantissa bit less). Its definition, from the OCP 8-bit floating point
specification:

* code = sign(1) | exponent(5) | mantissa(2), exponent bias 15;
* exponent 0: subnormal, value m * 2**-16 (m = 0..3);
* exponent 1..30: normal, value (1 + m/4) * 2**(e - 15);
* exponent 31: mantissa 0 is infinity (0x7C, 0xFC), mantissa 1..3 NaN;
* so the largest finite magnitude is 0x7B = 1.75 * 2**15 = 57344.

Encoding from float32 (the same readings as for E4M3):

* NaN            -> 0x7F with the input's sign bit;
* |v| >= 57344   -> 0x7B with the sign bit (saturate; this also covers
                    +-inf, so no code of the encoder is ever an infinity);
* otherwise      -> the nearest of the 124 non-negative finite magnitudes,
                    ties to the code whose last bit is 0, with the sign bit
                    applied even when the magnitude rounds to zero.

As in ``oracle.e4m3`` there are two encoders: ``encode_bruteforce`` (argmin of
distances, the definition written out) and ``encode`` (a vectorized search).
"""
from __future__ import annotations

import math

import numpy as np

E5M2_MAX = 57344.0        # OCP E5M2: S.11110.11
NAN_CODE = 0x7F           # the NaN code this encoder emits (S.11111.11)
INF_CODE = 0x7C           # S.11111.00 (decoded, never produced by the encoder)
MAX_CODE = 0x7B
SIGN_BIT = 0x80


def decode_code(code: int) -> float:
    """Value of one E5M2 code, from the OCP closed form (float64, exact)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & SIGN_BIT else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return sign * math.inf if m == 0 else math.copysign(float("nan"), sign)
    if e == 0:
        return sign * m * 2.0 ** -16
    return sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)


def decode_table() -> np.ndarray:
    """All 256 codes decoded to float64."""
    return np.array([decode_code(c) for c in range(256)], dtype=np.float64)


TABLE = decode_table()
# Non-negative finite magnitudes in code order (codes 0x00..0x7B increase).
MAGS = TABLE[:MAX_CODE + 1].copy()


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 codes to float64."""
    return TABLE[np.asarray(codes, dtype=np.uint8)]


def _sign_bits(v: np.ndarray) -> np.ndarray:
    return np.where(np.signbit(v), SIGN_BIT, 0).astype(np.uint8)


def encode_bruteforce(v: np.ndarray, chunk: int = 1 << 15) -> np.ndarray:
    """Definition of the encoder: argmin over all finite magnitudes, ties to the
    even code. Distances in float64 are exact for the two bracketing magnitudes
    (see ``oracle.e4m3.encode_bruteforce``; the E5M2 grid is coarser still)."""
    v = np.asarray(v, dtype=np.float32).ravel()
    out = np.empty(v.shape, dtype=np.uint8)
    even = (np.arange(MAGS.size) % 2 == 0)[None, :]
    for s in range(0, v.size, chunk):
        x = v[s:s + chunk]
        with np.errstate(invalid="ignore"):
            a = np.abs(x.astype(np.float64))
        a_f = np.where(np.isfinite(a), a, 0.0)
        dist = np.abs(a_f[:, None] - MAGS[None, :])
        best = dist.min(axis=1, keepdims=True)
        is_best = dist == best
        pick_even = (is_best & even).any(axis=1)
        code = np.where(pick_even, (is_best & even).argmax(axis=1), is_best.argmax(axis=1))
        code = np.where(a >= E5M2_MAX, MAX_CODE, code)          # includes +-inf
        code = np.where(np.isnan(x), NAN_CODE, code).astype(np.uint8)
        out[s:s + chunk] = code | _sign_bits(x)
    return out


def encode(v: np.ndarray) -> np.ndarray:
    """Vectorized round-to-nearest-even encoder with saturation at 57344."""
    v = np.asarray(v, dtype=np.float32)
    shape = v.shape
    x = v.ravel()
    with np.errstate(invalid="ignore"):
        a = np.abs(x.astype(np.float64))
    small = a < E5M2_MAX                              # False for NaN and inf
    a_c = np.where(small, a, 0.0)
    hi = np.clip(np.searchsorted(MAGS, a_c, side="left"), 0, MAX_CODE)
    lo = np.clip(hi - 1, 0, MAX_CODE)
    d_hi = MAGS[hi] - a_c
    d_lo = a_c - MAGS[lo]
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    code = np.where(a_c == MAGS[hi], hi, code)
    code = np.where(small, code, MAX_CODE)
    code = np.where(np.isnan(x), NAN_CODE, code).astype(np.uint8)
    return (code | _sign_bits(x)).reshape(shape)
