"""Pins for the oracle's E5M2 codec, the gradient format of the hybrid recipe (CPU only).

What pins it, apart from the oracle itself:
* the OCP E5M2 table's named values (tests/golden/ocp_e5m2_facts.txt);
* IEEE binary16: an E5M2 code is the top byte of the binary16 pattern of the
  same value (same sign, exponent bias 15 and special values, two mantissa bits
  instead of ten), so numpy's float16 decodes every code independently, and
  rounding a binary16 pattern to its top byte with integer arithmetic (round
  half to even on the dropped byte) encodes every binary16 value;
* the brute-force definition (argmin, ties to even) over every bf16 pattern
  times a set of scales, against the vectorized encoder;
* saturation, signed zero and NaN special cases.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import e5m2, quantize, scaling


def _facts(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "ocp_e5m2_facts.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, value = line.split()[:2]
            rows.append((int(code, 16), value))
    return rows


def test_named_values_from_ocp_table(golden_dir):
    facts = _facts(golden_dir)
    assert len(facts) >= 12
    for code, value in facts:
        got = e5m2.decode_code(code)
        if value == "nan":
            assert np.isnan(got), hex(code)
        elif value in ("inf", "-inf"):
            assert np.isinf(got) and (got < 0) == value.startswith("-"), hex(code)
        elif value == "-0":
            assert got == 0.0 and np.signbit(got), hex(code)
        else:
            assert Fraction(got) == Fraction(value), (hex(code), got, value)


def test_decode_equals_binary16_top_byte():
    codes = np.arange(256, dtype=np.uint16)
    half = (codes << 8).view(np.float16).astype(np.float64)
    t = e5m2.TABLE
    assert np.array_equal(np.isnan(t), np.isnan(half))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], half[ok])
    assert np.array_equal(np.signbit(t[ok]), np.signbit(half[ok]))


def _round_half_bits_to_e5m2(h: np.ndarray) -> np.ndarray:
    """Expected code for binary16 patterns h (finite or infinite): drop the low
    byte with round half to even on the magnitude, then saturate at 0x7B."""
    h = h.astype(np.uint32)
    sign = (h >> 8) & 0x80
    mag = h & 0x7FFF
    top, low = mag >> 8, mag & 0xFF
    up = (low > 0x80) | ((low == 0x80) & ((top & 1) == 1))
    top = top + up.astype(np.uint32)
    top = np.minimum(top, e5m2.MAX_CODE)        # 0x7C and above: beyond 57344 (or inf)
    return (top | sign).astype(np.uint8)


def test_encoder_matches_binary16_rounding_everywhere():
    h = np.arange(65536, dtype=np.uint16)
    f = h.view(np.float16)
    keep = ~np.isnan(f)
    v = f[keep].astype(np.float32)
    want = _round_half_bits_to_e5m2(h[keep])
    assert np.array_equal(e5m2.encode(v), want)
    assert np.array_equal(e5m2.encode_bruteforce(v), want)


@pytest.mark.parametrize("scale_inv", [1.0, 57344.0, 57344.0 / 3.7, 2.0 ** -20, 2.0 ** 20,
                                       57344.0 / 1e-3])
def test_vectorized_equals_bruteforce_all_bf16(scale_inv):
    bits = np.arange(65536, dtype=np.uint16)
    x = quantize.bf16_to_f32(bits)
    with np.errstate(invalid="ignore", over="ignore"):
        v = x * np.float32(scale_inv)
    assert np.array_equal(e5m2.encode(v), e5m2.encode_bruteforce(v))


def test_round_trip_all_codes():
    for c in range(256):
        val = e5m2.decode_code(c)
        got = int(e5m2.encode(np.array([val], dtype=np.float32))[0])
        if np.isnan(val):
            assert got == (0x7F | (c & 0x80)), hex(c)
        elif np.isinf(val):
            assert got == (0x7B | (c & 0x80)), hex(c)       # saturation, not infinity
        else:
            assert got == c, hex(c)


@pytest.mark.parametrize("value, code", [
    (57344.0, 0x7B), (61439.0, 0x7B), (61440.0, 0x7B), (1e30, 0x7B), (np.inf, 0x7B),
    (-np.inf, 0xFB), (2.0 ** -17, 0x00), (3 * 2.0 ** -17, 0x02), (2.0 ** -17 * 1.0001, 0x01),
    (0.0, 0x00), (-0.0, 0x80), (-(2.0 ** -20), 0x80), (1.125, 0x3C), (1.375, 0x3E),
    (np.nan, 0x7F)])
def test_special_values(value, code):
    assert int(e5m2.encode(np.array([value], dtype=np.float32))[0]) == code


def test_nan_product_takes_input_sign():
    x = np.array([-1.0, 1.0], dtype=np.float32)
    v = np.array([np.nan, np.nan], dtype=np.float32)
    assert list(quantize.encode_product(x, v, "e5m2")) == [0xFF, 0x7F]


def test_scale_with_e5m2_max_is_the_correctly_rounded_quotient():
    rng = np.random.default_rng(5)
    for a in np.concatenate([rng.lognormal(-6, 4, 500), [1e-12, 1e-3, 1.0, 57344.0]]):
        a32 = np.float32(a)
        s, si = scaling.scale_from_amax(a32, scaling.E5M2_MAX)
        for got, num, den in ((s, Fraction(float(max(a32, scaling.AMAX_FLOOR))), 57344),
                              (si, Fraction(57344), Fraction(float(max(a32, scaling.AMAX_FLOOR))))):
            exact = Fraction(num) / Fraction(den)
            g = Fraction(float(got))
            up = Fraction(float(np.nextafter(got, np.float32(np.inf))))
            dn = Fraction(float(np.nextafter(got, np.float32(0))))
            assert abs(g - exact) <= abs(up - exact) and abs(g - exact) <= abs(dn - exact)


def test_current_scale_maps_amax_to_max_code():
    rng = np.random.default_rng(6)
    for _ in range(200):
        a = np.float32(rng.lognormal(0, 5))
        _, si = scaling.scale_from_amax(a, scaling.E5M2_MAX)
        code = int(e5m2.encode(np.array([a * si], dtype=np.float32))[0])
        assert code == 0x7B
