"""Pins for the oracle's block-scaled recipe (CPU only).

* special case: when every tile holds the same largest magnitude, every tile
  scale equals the tensorwise current scale, so block codes and the block GEMM
  reduce to the tensorwise ones (checked against oracle.quantize / oracle.gemm,
  which are pinned independently);
* tile invariant: the largest element of each tile encodes to +-448;
* the tile grids are checked entry by entry against a brute-force tile amax,
  including the transposed copy's tiles along the token index;
* the GEMM is checked element by element against an exact rational sum.
"""
from fractions import Fraction

import numpy as np

import workloads
from oracle import block, e4m3, gemm
from oracle.quantize import bf16_to_f32, quantize_tensorwise
from oracle.scaling import scale_from_amax


def _tiles_with_equal_max(R, C, seed):
    x = workloads.bf16_tensor("normal", (R, C), 77, seed, 0, std=1.0)
    f = bf16_to_f32(x)
    x = np.where(np.abs(f) >= 4.0, np.uint16(0x3F80), x)     # keep |x| < 4
    x[:, ::128] = 0x4080          # a 4.0 in every 1x128 row tile (and every 128x128 tile)
    x[::128, :] = 0x4080          # a 4.0 in every 128x1 column tile (the transposed copy's tiles)
    return x


def test_block_reduces_to_tensorwise_when_tile_maxima_agree():
    x = _tiles_with_equal_max(256, 256, 1)
    w = _tiles_with_equal_max(256, 256, 2)
    s, si = scale_from_amax(np.float32(4.0))
    qx, qx_t, ax, sx, sx_t = block.quantize_1x128(x)
    qw, qw_t, aw, sw, sw_t = block.quantize_128x128(w)
    assert np.all(ax == 4.0) and np.all(aw == 4.0)
    assert np.all(sx == s) and np.all(sx_t == s) and np.all(sw == s)
    tq, tq_t, _ = quantize_tensorwise(x, si)
    assert np.array_equal(qx, tq) and np.array_equal(qx_t, tq_t)
    D = block.block_scaled_gemm(qx, qw, sx, sw, 128)
    Dt = gemm.scaled_gemm(qx, qw, s, s)
    # two float64 roundings per element at most: relative to the largest entry
    assert np.allclose(D, Dt, rtol=1e-12, atol=1e-12 * np.abs(Dt).max())


def test_tile_grids_brute_force():
    x = workloads.bf16_tensor("outlier_normal", (256, 384), 5, 1, 0, rate=0.01, mult=100.0)
    q, q_t, amax, sc, sc_t = block.quantize_1x128(x, rows_valid=200)
    f = bf16_to_f32(x)
    rng = np.random.default_rng(0)
    for _ in range(40):
        r, kb = int(rng.integers(0, 256)), int(rng.integers(0, 3))
        tile = f[r, kb * 128:(kb + 1) * 128] if r < 200 else np.zeros(128, np.float32)
        a = max(abs(float(v)) for v in tile)
        assert amax[r, kb] == np.float32(a)
        assert sc[r, kb] == scale_from_amax(np.float32(a))[0]
        if r < 200:
            i = int(np.argmax(np.abs(tile)))
            assert q[r, kb * 128 + i] & 0x7F == 0x7E
        else:
            assert np.all(q[r] == 0)
    for _ in range(40):
        c, rb = int(rng.integers(0, 384)), int(rng.integers(0, 2))
        col = [abs(float(f[r, c])) if r < 200 else 0.0 for r in range(rb * 128, (rb + 1) * 128)]
        s, si = scale_from_amax(np.float32(max(col)))
        assert sc_t[c, rb] == s
        expect = e4m3.encode(f[rb * 128:(rb + 1) * 128, c] * si)
        expect[np.arange(rb * 128, (rb + 1) * 128) >= 200] = 0
        assert np.array_equal(q_t[c, rb * 128:(rb + 1) * 128], expect)


def test_weight_tiles_transpose():
    w = workloads.bf16_tensor("outlier_normal", (256, 384), 5, 2, 0, rate=0.01, mult=100.0)
    q, q_t, amax, sc, sc_t = block.quantize_128x128(w)
    assert np.array_equal(q_t, q.T) and np.array_equal(sc_t, sc.T)
    f = np.abs(bf16_to_f32(w))
    for i in range(2):
        for j in range(3):
            assert amax[i, j] == f[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128].max()


def test_block_gemm_exact_rational():
    rng = np.random.default_rng(9)
    qa = rng.integers(0, 0xFF, size=(2, 256)).astype(np.uint8)
    qb = rng.integers(0, 0xFF, size=(128, 256)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0
    qb[(qb & 0x7F) == 0x7F] = 0
    sa = np.array([[0.5, 3.0], [0.25, 1e-3]], np.float32)
    sb = np.array([[2.0, 0.125]], np.float32)
    D = block.block_scaled_gemm(qa, qb, sa, sb, 128)
    for m in range(2):
        for n in (0, 5, 127):
            exact = Fraction(0)
            for k in range(256):
                exact += (Fraction(float(sa[m, k // 128])) * Fraction(float(sb[0, k // 128]))
                          * Fraction(e4m3.decode_code(qa[m, k])) * Fraction(e4m3.decode_code(qb[n, k])))
            assert abs(Fraction(D[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)
