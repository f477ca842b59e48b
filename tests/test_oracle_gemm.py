"""Pins for the oracle's scaled GEMM, quantize/amax and padding (CPU only).

* GEMM: brute force with Python integers (every e4m3 value times 2**9 is an
  integer) on the small-shape configuration, index by index, so a transposed
  operand, a wrong contraction index or a dropped scale fails;
* quantize: Q^T is the transpose, padded rows are zero, amax is the brute-force
  maximum over valid rows and equals |x| of some element;
* padding: the pages' worked numbers (3858 tokens) and the closed form.
"""
import os

import numpy as np
import pytest

import workloads
from oracle import e4m3, gemm, padding
from oracle.quantize import amax, bf16_to_f32, quantize_tensorwise
from oracle.scaling import scale_from_amax


def _int_codes(q):
    """Each code as an exact integer multiple of 2**-9."""
    return [[int(e4m3.decode_code(c) * 512) for c in row] for row in q]


def test_gemm_exact_against_python_integers():
    d = workloads.linear_inputs(1)
    x, w = d["x"], d["w"]
    assert x.shape == (64, 128) and w.shape == (128, 128)
    sx, sx_inv = scale_from_amax(amax(x))
    sw, sw_inv = scale_from_amax(amax(w))
    qx, _, _ = quantize_tensorwise(x, sx_inv)
    qw, _, _ = quantize_tensorwise(w, sw_inv)
    A = _int_codes(qx)
    B = _int_codes(qw)
    S = gemm.unscaled_product(qx, qw)
    D = gemm.scaled_gemm(qx, qw, sx, sw)
    for m in range(64):
        for n in range(128):
            acc = 0
            for k in range(128):
                acc += A[m][k] * B[n][k]
            exact = acc / float(1 << 18)          # exact: |acc| < 2**53
            assert S[m, n] == exact
            assert D[m, n] == exact * (float(sx) * float(sw))


def test_gemm_nonsquare_indices():
    rng = np.random.default_rng(0)
    qa = rng.integers(0, 0x7F, size=(3, 5)).astype(np.uint8)   # finite codes only
    qb = rng.integers(0, 0x7F, size=(2, 5)).astype(np.uint8) | 0x80
    D = gemm.scaled_gemm(qa, qb, 2.0, 0.5)
    assert D.shape == (3, 2)
    for m in range(3):
        for n in range(2):
            ref = sum(e4m3.decode_code(qa[m, k]) * e4m3.decode_code(qb[n, k]) for k in range(5))
            assert D[m, n] == ref


def test_gemm_exact_at_large_k():
    """All-448 operands at K = 2**17 - 16: the float64 sum is still exact."""
    K = (1 << 17) - 16
    qa = np.full((1, K), 0x7E, np.uint8)
    qb = np.full((2, K), 0x7E, np.uint8)
    qb[1, ::2] = 0x01
    S = gemm.unscaled_product(qa, qb)
    assert S[0, 0] == 448 * 448 * K
    assert S[0, 1] == 448 * 448 * (K // 2) + 448 * 2.0 ** -9 * (K // 2)


def test_error_bound_definition():
    qa = np.array([[0x38, 0x40]], np.uint8)         # [1, 2]
    qb = np.array([[0x40, 0x38], [0x00, 0x38]], np.uint8)  # [2, 1], [0, 1]
    b = gemm.error_bound(qa, qb, 1.0, 3.0)
    assert np.allclose(b, 1e-2 * np.array([[np.sqrt(5) * 3 * np.sqrt(5), np.sqrt(5) * 3]]))


def test_quantize_transpose_and_padding():
    x = workloads.bf16_tensor("normal", (48, 40), 99, 1, 0, std=3.0)
    x[40:] = 0x7FC0                                  # NaN sentinels in the padded rows
    q, qt, a = quantize_tensorwise(x, np.float32(10.0), rows_valid=40)
    assert np.array_equal(qt, q.T)
    assert np.all(q[40:] == 0)
    assert not np.isnan(a)
    vals = [abs(float(v)) for v in bf16_to_f32(x[:40]).ravel()]
    assert a == np.float32(max(vals))
    assert a in set(np.abs(bf16_to_f32(x[:40])).ravel())


def test_amax_edge_cases():
    assert amax(np.zeros((4, 4), np.uint16)) == 0.0
    assert amax(np.full((4, 4), 0x8000, np.uint16)) == 0.0          # -0.0
    x = np.zeros((4, 4), np.uint16)
    x[2, 3] = 0xC2F6                                                # -123.0
    assert amax(x) == 123.0
    x[1, 1] = 0x7FC0
    assert np.isnan(amax(x))
    assert amax(x, rows_valid=1) == 0.0
    assert amax(np.zeros((0, 8), np.uint16)) == 0.0


def test_quantize_uses_float32_product_then_rne():
    # 1.0625 is the midpoint of 1 and 1.125: ties to even -> 0x38
    x = np.array([[0x3F88]], np.uint16)                            # bf16 1.0625
    q, _, _ = quantize_tensorwise(x, np.float32(1.0))
    assert q[0, 0] == 0x38
    # bf16 1.0 times the float32 just above 1.0625 -> rounds up to 0x39
    q, _, _ = quantize_tensorwise(np.array([[0x3F80]], np.uint16),
                                  np.nextafter(np.float32(1.0625), np.float32(2)))
    assert q[0, 0] == 0x39


def _golden_constants(golden_dir):
    out = {}
    with open(os.path.join(golden_dir, "pages_constants.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, value = line.split()[:2]
            out[name] = value
    return out


def test_padding_worked_numbers(golden_dir):
    c = _golden_constants(golden_dir)
    mult = int(c["token_multiple"])
    bad = int(c["bad_token_count"])
    assert mult == padding.TOKEN_MULTIPLE == 16
    assert bad % mult != 0
    assert padding.pad_amount(bad) == 14 and padding.padded_count(bad) == 3872
    assert int(c["fp8_weight_bytes"]) == 4096 * 4096 * 1
    assert int(c["short_storage_bytes"]) == 4092 * 4096


@pytest.mark.parametrize("T,mult,pad", [(0, 16, 0), (1, 16, 15), (15, 16, 1), (16, 16, 0),
                                        (17, 16, 15), (67827, 16, 13), (5, 8, 3), (64, 24, 8)])
def test_pad_amount(T, mult, pad):
    assert padding.pad_amount(T, mult) == pad
    assert padding.padded_count(T, mult) % mult == 0
    assert 0 <= padding.padded_count(T, mult) - T < mult


def test_pad_rows():
    x = np.arange(3 * 5, dtype=np.uint16).reshape(3, 5) + 1
    p = padding.pad_rows(x)
    assert p.shape == (16, 5)
    assert np.array_equal(p[:3], x) and np.all(p[3:] == 0)
    with pytest.raises(ValueError):
        padding.pad_amount(3, 0)


def test_nan_products_take_the_input_sign():
    from oracle.quantize import quantize_values
    x = np.array([0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x3F80, 0xBF80, 0x0000, 0x8000], np.uint16)
    assert list(quantize_values(x, np.float32(2.0))) == [0x7F, 0xFF, 0x7F, 0xFF, 0x40, 0xC0, 0, 0x80]
    # an invalid multiplier makes every product NaN: the sign still comes from x
    assert list(quantize_values(x, np.float32(np.nan))) == [0x7F, 0xFF, 0x7F, 0xFF, 0x7F, 0xFF, 0x7F, 0xFF]
    # inf * 0 is NaN as well
    z = np.array([0x7F80, 0xFF80], np.uint16)
    assert list(quantize_values(z, np.float32(0.0))) == [0x7F, 0xFF]


def test_mixed_format_gemm_against_python_integers():
    """E5M2 first operand: every E5M2 value times 2**16 and every E4M3 value times
    2**9 is an integer, so the exact sum is an integer over 2**25. At K = 8 the
    float64 product is exact; at K = 96 it is within K * 2**-52 * sum |a b|."""
    from oracle import e5m2
    rng = np.random.default_rng(3)
    for K, exact_fp64 in ((8, True), (96, False)):
        qa = rng.integers(0, 0x7C, size=(6, K)).astype(np.uint8)     # finite E5M2 codes
        qa[rng.random(qa.shape) < 0.5] |= 0x80
        qb = rng.integers(0, 0x7F, size=(5, K)).astype(np.uint8)     # finite E4M3 codes
        qb[rng.random(qb.shape) < 0.5] |= 0x80
        S = gemm.unscaled_product(qa, qb, a_fmt="e5m2")
        D = gemm.scaled_gemm(qa, qb, 0.25, 3.0, a_fmt="e5m2")
        for m in range(6):
            for n in range(5):
                terms = [int(e5m2.decode_code(qa[m, k]) * 65536) *
                         int(e4m3.decode_code(qb[n, k]) * 512) for k in range(K)]
                acc = sum(terms)
                mag = sum(abs(t) for t in terms) / float(1 << 25)
                if exact_fp64:
                    assert S[m, n] == acc / float(1 << 25)
                else:
                    assert abs(S[m, n] - acc / float(1 << 25)) <= K * 2.0 ** -52 * mag
                assert D[m, n] == S[m, n] * 0.75
        # the E5M2 operand is really decoded as E5M2: 0x3C is 1.0 there, 1.5 in E4M3
        one = gemm.unscaled_product(np.full((1, 1), 0x3C, np.uint8),
                                    np.full((1, 1), 0x38, np.uint8), a_fmt="e5m2")
        assert one[0, 0] == 1.0


def test_mixed_format_error_bound_uses_e5m2_norms():
    qa = np.array([[0x3C, 0x40]], np.uint8)        # E5M2: 1, 2
    qb = np.array([[0x38, 0x38]], np.uint8)        # E4M3: 1, 1
    b = gemm.error_bound(qa, qb, 1.0, 1.0, a_fmt="e5m2")
    assert b[0, 0] == pytest.approx(1e-2 * np.sqrt(5.0) * np.sqrt(2.0), rel=1e-15)


def test_bshd_alignment_worked_case(golden_dir):
    """The review thread's case: B = 16, tp = 4 with TE's multiple 8. Padding T to
    8 * tp / gcd(B, 8 * tp) gives a multiple of 2, which tp = 4 does not divide; the lcm
    rule asks for 4."""
    c = _golden_constants(golden_dir)
    B, tp, base = int(c["bshd_example_batch"]), int(c["bshd_example_tp"]), int(c["bshd_te_base"])
    naive = base * tp // np.gcd(B, base * tp)
    assert naive == int(c["bshd_example_naive"]) == 2 and naive % tp != 0
    assert padding.align_multiples(padding.BSHD, B, tp, base=base) == (4, 1)


@pytest.mark.parametrize("B,tp,base", [(16, 4, 8), (16, 4, 16), (3, 2, 16), (1, 8, 16),
                                       (6, 4, 16), (5, 3, 8), (32, 1, 16)])
def test_bshd_alignment_is_the_least_valid_multiple(B, tp, base):
    """Brute force: T is valid iff T % tp == 0 and B * T % (base * tp) == 0; the valid T
    are exactly the multiples of the returned multiple."""
    m, total = padding.align_multiples(padding.BSHD, B, tp, base=base)
    assert total == 1
    for T in range(1, 4 * m * base + 1):
        valid = T % tp == 0 and (B * T) % (base * tp) == 0
        assert valid == (T % m == 0), (B, tp, base, T)


def test_thd_alignment(golden_dir):
    c = _golden_constants(golden_dir)
    assert c["thd_multiple_te"] == "8*cp*tp"
    assert padding.align_multiples(padding.THD, tp=2, cp=1, base=8) == (1, 16)
    assert padding.align_multiples(padding.THD, tp=2, cp=4) == (8, 128)
    assert padding.align_multiples(padding.THD) == (1, 16)
    with pytest.raises(ValueError):
        padding.align_multiples(padding.BSHD, 4, 2, cp=2)


def test_pad_and_unpad_varlen_by_hand():
    x = (np.arange(7 * 2, dtype=np.uint16).reshape(7, 2) + 1)       # lengths 3, 1, 3
    p, cu = padding.pad_varlen(x, [3, 1, 3], seq_multiple=4, total_multiple=16)
    assert list(cu) == [0, 4, 8, 12] and p.shape == (16, 2)
    assert np.array_equal(p[0:3], x[0:3]) and np.all(p[3] == 0)
    assert np.array_equal(p[4], x[3]) and np.all(p[5:8] == 0)
    assert np.array_equal(p[8:11], x[4:7]) and np.all(p[11:] == 0)
    assert np.array_equal(padding.unpad_varlen(p, [3, 1, 3], cu), x)
    # every sequence length a multiple already, no total padding: the identity
    q, cu2 = padding.pad_varlen(x[:4], [2, 2], 2, 1)
    assert np.array_equal(q, x[:4]) and list(cu2) == [0, 2, 4]
    # empty sequences take no rows
    r, cu3 = padding.pad_varlen(x[:3], [0, 3, 0], 4, 1)
    assert list(cu3) == [0, 0, 4, 4] and r.shape == (4, 2)
