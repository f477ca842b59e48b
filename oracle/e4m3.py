"""OCP E4M3 codec (test infrastructure: only tests, smoke and the CPU baseline use it).

The pages name the format only as "e4m3" with the largest finite value 448
(AstrAI ``fp8_state.py``: ``E4M3_MAX = 448.0``). 448 identifies the OCP OFP8
"E4M3" variant (no infinities, one NaN mantissa pattern per sign), not the
FNUZ variant whose maximum is 240. Its definition, from the OCP 8-bit floating
point specification:

* code = sign(1) | exponent(4) | mantissa(3), exponent bias 7;
* exponent 0: subnormal, value m * 2**-9 (m = 0..7);
* exponent 1..15: normal, value (1 + m/8) * 2**(e - 7);
* exponent 15 with mantissa 7 (0x7F, 0xFF) is NaN; there is no infinity;
* so the largest finite magnitude is 0x7E = 1.75 * 2**8 = 448.

Encoding from float32 (the readings used here for what the pages leave open):

* NaN            -> 0x7F with the input's sign bit;
* |v| >= 448     -> 0x7E with the sign bit (saturate; this also covers +-inf);
* otherwise      -> the nearest of the 127 non-negative finite magnitudes,
                    ties to the code whose last bit is 0 (round to nearest
                    even), with the sign bit applied even when the magnitude
                    rounds to zero (so -0.0 and tiny negatives give 0x80).

Two encoders are kept on purpose: ``encode_bruteforce`` is the definition
written out (argmin of distances), ``encode`` is a vectorized search used by the
rest of the oracle. The tests require them to agree on every bf16 input pattern
times a set of scales.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0          # AstrAI fp8_state.py, E4M3_MAX
NAN_CODE = 0x7F           # OCP E4M3: S.1111.111
MAX_CODE = 0x7E           # OCP E4M3: S.1111.110 = 448
SIGN_BIT = 0x80


def decode_code(code: int) -> float:
    """Value of one E4M3 code, from the OCP closed form (float64, exact)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & SIGN_BIT else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.copysign(float("nan"), sign)
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def decode_table() -> np.ndarray:
    """All 256 codes decoded to float64 (NaN for 0x7F and 0xFF)."""
    return np.array([decode_code(c) for c in range(256)], dtype=np.float64)


TABLE = decode_table()
# Non-negative finite magnitudes in code order. Codes 0x00..0x7E increase
# monotonically in value, so the index of a magnitude IS its code.
MAGS = TABLE[:MAX_CODE + 1].copy()


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 codes to float64."""
    return TABLE[np.asarray(codes, dtype=np.uint8)]


def _sign_bits(v: np.ndarray) -> np.ndarray:
    return np.where(np.signbit(v), SIGN_BIT, 0).astype(np.uint8)


def encode_bruteforce(v: np.ndarray, chunk: int = 1 << 16) -> np.ndarray:
    """Definition of the encoder: argmin over all finite magnitudes.

    Distances are taken in float64. For the two magnitudes that bracket |v|
    the difference is exact (|v| is a float32 and the bracket lies within a
    few binades of it, so the difference needs at most ~30 significant bits).
    Any other magnitude is at least one E4M3 step farther away, which a
    relative rounding error of 2**-53 cannot hide. Ties occur only at exact
    midpoints, which are short dyadic numbers and are therefore also exact.
    """
    v = np.asarray(v, dtype=np.float32).ravel()
    out = np.empty(v.shape, dtype=np.uint8)
    for s in range(0, v.size, chunk):
        x = v[s:s + chunk]
        with np.errstate(invalid="ignore"):
            a = np.abs(x.astype(np.float64))
        dist = np.abs(a[:, None] - MAGS[None, :])          # [n, 127]
        best = dist.min(axis=1, keepdims=True)
        is_best = dist == best
        # among the (at most two) nearest codes prefer the even one
        even = (np.arange(MAGS.size) % 2 == 0)[None, :]
        pick_even = (is_best & even).any(axis=1)
        first_best = is_best.argmax(axis=1)
        first_even_best = (is_best & even).argmax(axis=1)
        code = np.where(pick_even, first_even_best, first_best).astype(np.uint8)
        code = np.where(a >= E4M3_MAX, MAX_CODE, code).astype(np.uint8)
        code = np.where(np.isnan(x), NAN_CODE, code).astype(np.uint8)
        out[s:s + chunk] = code | _sign_bits(x)
    return out


def encode(v: np.ndarray) -> np.ndarray:
    """Vectorized round-to-nearest-even encoder with saturation.

    For |v| < 448: ``hi`` is the first magnitude >= |v| and ``hi - 1`` the one
    below; pick the closer one, and on a tie the even code.
    """
    v = np.asarray(v, dtype=np.float32)
    shape = v.shape
    x = v.ravel()
    with np.errstate(invalid="ignore"):
        a = np.abs(x.astype(np.float64))
    finite_small = a < E4M3_MAX                      # False for NaN and inf
    a_c = np.where(finite_small, a, 0.0)
    hi = np.searchsorted(MAGS, a_c, side="left")     # MAGS[hi] >= a
    hi = np.clip(hi, 0, MAX_CODE)
    lo = np.clip(hi - 1, 0, MAX_CODE)
    d_hi = MAGS[hi] - a_c
    d_lo = a_c - MAGS[lo]
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(a_c == MAGS[hi], hi, code)       # exact hit (incl. 0)
    code = np.where(finite_small, code, MAX_CODE)
    code = np.where(np.isnan(x), NAN_CODE, code).astype(np.uint8)
    return (code | _sign_bits(x)).reshape(shape)
