"""Pins for the oracle's E4M3 codec (CPU only).

What pins it, apart from the oracle itself:
* the OCP E4M3 table's named values (tests/golden/ocp_e4m3_facts.txt) and the
  page constant 448;
* structural facts of the format (253 distinct finite values, monotone codes,
  spacing 32 next to 448, 2**-9 at the bottom);
* the brute-force definition (argmin, ties to even) over every bf16 bit
  pattern times a set of scales;
* hand-picked special values (saturation, subnormal ties, signed zero, NaN).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import e4m3


def _facts(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "ocp_e4m3_facts.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, value = line.split()[:2]
            rows.append((int(code, 16), value))
    return rows


def test_named_values_from_ocp_table(golden_dir):
    facts = _facts(golden_dir)
    assert len(facts) >= 10
    for code, value in facts:
        got = e4m3.decode_code(code)
        if value == "nan":
            assert np.isnan(got), hex(code)
        elif value == "-0":
            assert got == 0.0 and np.signbit(got), hex(code)
        else:
            assert Fraction(got) == Fraction(value), (hex(code), got, value)


def test_max_is_page_constant():
    assert e4m3.E4M3_MAX == 448.0
    assert np.nanmax(e4m3.TABLE) == 448.0
    assert e4m3.TABLE[e4m3.MAX_CODE] == 448.0


def test_table_structure():
    t = e4m3.TABLE
    assert np.isnan(t).sum() == 2 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    finite = t[~np.isnan(t)]
    assert finite.size == 254
    assert np.unique(finite).size == 253            # +0 and -0 compare equal
    # codes 0x00..0x7E are strictly increasing; negative half mirrors them
    assert np.all(np.diff(e4m3.MAGS) > 0)
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])
    # spacing: 2**-9 among subnormals and in the first normal binade, 32 at the top
    assert e4m3.MAGS[1] - e4m3.MAGS[0] == 2.0 ** -9
    assert e4m3.MAGS[0x7E] - e4m3.MAGS[0x7D] == 32.0
    # every finite value is a multiple of 2**-9 (the GEMM exactness argument uses this)
    assert np.all(np.mod(finite * 512.0, 1.0) == 0.0)


def test_round_trip_all_256_codes():
    vals = e4m3.TABLE.astype(np.float32)
    for enc in (e4m3.encode, e4m3.encode_bruteforce):
        codes = enc(vals)
        assert np.array_equal(codes, np.arange(256, dtype=np.uint8)), enc.__name__


SPECIAL = [
    (448.0, 0x7E), (-448.0, 0xFE), (464.0, 0x7E), (479.0, 0x7E), (1e30, 0x7E),
    (np.inf, 0x7E), (-np.inf, 0xFE), (3.4e38, 0x7E),
    (2.0 ** -10, 0x00),                 # half of the smallest subnormal: tie -> even (0)
    (-(2.0 ** -10), 0x80),
    (3 * 2.0 ** -10, 0x02),             # midway between 0x01 and 0x02: tie -> even
    (3 * 2.0 ** -11, 0x01),             # 0.75 * 2**-9 -> nearest is 2**-9
    (5 * 2.0 ** -10, 0x02),             # midway between 0x02 and 0x03 -> even 0x02
    (2.0 ** -11, 0x00), (1e-30, 0x00), (-1e-30, 0x80),
    (0.0, 0x00), (-0.0, 0x80),
    (1.0625, 0x38),                     # midway 1 (0x38) / 1.125 (0x39) -> even 0x38
    (1.1875, 0x3A),                     # midway 1.125 / 1.25 -> even 0x3A
    (1.0625 + 2.0 ** -20, 0x39),        # just above the midpoint
    (432.0, 0x7E),                      # midway 416 (0x7D) / 448 (0x7E) -> even 0x7E
    (431.0, 0x7D),
    (7.5 * 2.0 ** -9, 0x08),            # midway max subnormal 0x07 / min normal 0x08 -> even 0x08
    (np.nan, 0x7F), (-np.nan, 0xFF),
]


@pytest.mark.parametrize("value,code", SPECIAL)
def test_special_values(value, code):
    v = np.array([value], dtype=np.float32)
    assert e4m3.encode(v)[0] == code, (value, hex(e4m3.encode(v)[0]))
    assert e4m3.encode_bruteforce(v)[0] == code


def _all_bf16_as_f32():
    return (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)


SCALES = [1.0, 448.0, 0.5, 2.0 ** -20, 2.0 ** 20, 448.0 / 3.0, 448.0 / 0.11, 1.0 / 448.0,
          448.0 / 1e-12]


@pytest.mark.parametrize("scale_inv", SCALES)
def test_vectorized_equals_bruteforce_all_bf16(scale_inv):
    x = _all_bf16_as_f32()
    with np.errstate(over="ignore", invalid="ignore"):
        v = x * np.float32(scale_inv)
    assert np.array_equal(e4m3.encode(v), e4m3.encode_bruteforce(v))


def test_vectorized_equals_bruteforce_random_f32_patterns():
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    assert np.array_equal(e4m3.encode(v), e4m3.encode_bruteforce(v))


def test_every_midpoint_ties_to_even():
    m = e4m3.MAGS
    mids = ((m[:-1] + m[1:]) / 2).astype(np.float32)      # midpoints are exact in float32
    assert np.all(mids.astype(np.float64) == (m[:-1] + m[1:]) / 2)
    codes = e4m3.encode(mids)
    lo = np.arange(m.size - 1)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect.astype(np.uint8))
    assert np.array_equal(e4m3.encode(-mids), (expect | 0x80).astype(np.uint8))


def test_decode_of_encode_is_nearest():
    """|decode(encode(v)) - v| <= half the gap of the bracketing codes (RNE bound)."""
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(100_000) * 50).astype(np.float32)
    v = v[np.abs(v) < 448]
    d = e4m3.decode(e4m3.encode(v))
    a = np.abs(v.astype(np.float64))
    hi = np.searchsorted(e4m3.MAGS, a)
    gap = e4m3.MAGS[np.minimum(hi, 126)] - e4m3.MAGS[np.maximum(hi - 1, 0)]
    assert np.all(np.abs(d - v) <= gap / 2 + 0.0)
