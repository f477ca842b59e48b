"""Pins of oracle.bias: the column sum against plain Python arithmetic on small exact
inputs, padding rows ignored, and the bias add against its definition."""
import itertools

import numpy as np

from oracle.bias import add_bias, bf16_to_f64, bias_bound, bias_grad, bias_grad_bound


def _bits(values):
    """float values exactly representable in bf16 -> bit patterns."""
    f = np.asarray(values, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_bf16_decode_known_patterns():
    assert bf16_to_f64(np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4040, 0x7F7F],
                                np.uint16)).tolist() == [1.0, -1.0, 0.0, -0.0, 3.0,
                                                         float(np.float32(3.3895314e38))]


def test_column_sums_brute_force():
    rng = np.random.default_rng(1)
    vals = rng.integers(-64, 65, size=(7, 5)).astype(np.float64) / 4   # exact in bf16
    g = _bits(vals)
    for rv in range(0, 8):
        want = [sum(vals[r][c] for r in range(rv)) for c in range(5)]
        assert bias_grad(g, rv).tolist() == want


def test_padding_rows_ignored_even_if_nan():
    g = _bits(np.ones((6, 16)))
    g[4:] = 0x7FC0                         # NaN in the padding rows
    db = bias_grad(g, 4)
    assert np.all(db == 4.0)
    assert np.all(np.isfinite(bias_grad_bound(g, 4)))


def test_add_bias_definition():
    D = np.arange(12, dtype=np.float64).reshape(3, 4)
    b = _bits([0.5, -1.0, 2.0, 0.0])
    y = add_bias(D, b, rows_valid=2)
    for m, n in itertools.product(range(3), range(4)):
        want = D[m, n] + [0.5, -1.0, 2.0, 0.0][n] if m < 2 else 0.0
        assert y[m, n] == want
    assert add_bias(D, _bits(np.zeros(4))).tolist() == D.tolist()
    assert bias_bound(b).tolist() == [2.0 ** -9, 2.0 ** -8, 2.0 ** -7, 0.0]


def test_grad_bound_covers_float32_summation():
    """The bound holds for a float32 left-to-right sum of many terms (the worst order)."""
    rng = np.random.default_rng(2)
    vals = rng.standard_normal((3000, 16)).astype(np.float32)
    g = (vals.view(np.uint32) >> 16).astype(np.uint16)
    exact = bias_grad(g)
    f32 = np.zeros(16, np.float32)
    for r in range(3000):
        f32 += bf16_to_f64(g[r]).astype(np.float32)
    assert np.all(np.abs(f32.astype(np.float64) - exact) <= bias_grad_bound(g))
