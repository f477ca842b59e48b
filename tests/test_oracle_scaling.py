"""Pins for the oracle's scale arithmetic and the delayed-scaling schedule (CPU only).

* scale / scale_inv are checked against the exact rational quotient with
  correct float32 rounding (Fractions), not against a re-typed formula;
* the 1e-12 floor is checked against its float32 bit pattern;
* the weight ring is checked against the hand-worked schedule in
  tests/golden/weight_ring_schedule.txt (AstrAI fp8_state.py semantics);
* the one-step delay of x/g scales is checked step by step.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import scaling
from oracle.linear import DelayedLinear


def nearest_f32(fr: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational (ties to even)."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def test_floor_bits():
    assert np.array(scaling.AMAX_FLOOR, np.float32).view(np.uint32) == 0x2B8CBCCC
    assert scaling.E4M3_MAX == 448


@pytest.mark.parametrize("amax", [1.0, 0.11, 3.0, 300.0, 1e-3, 7.0, 0.0172, 2.0 ** -30,
                                  1e-12, 448.0, 65504.0, 3.3895314e38])
def test_scale_is_correctly_rounded_quotient(amax):
    a = np.float32(amax)
    scale, scale_inv = scaling.scale_from_amax(a)
    a = max(a, scaling.AMAX_FLOOR)
    assert scale == nearest_f32(Fraction(float(a)) / 448)
    assert scale_inv == nearest_f32(Fraction(448) / Fraction(float(a)))
    assert scale.dtype == np.float32 and scale_inv.dtype == np.float32


def test_scale_many_random_amax():
    rng = np.random.default_rng(3)
    for a in (rng.lognormal(0, 4, 400)).astype(np.float32):
        s, si = scaling.scale_from_amax(a)
        assert s == nearest_f32(Fraction(float(a)) / 448)
        assert si == nearest_f32(Fraction(448) / Fraction(float(a)))


def test_zero_and_tiny_amax_clamp():
    for a in (0.0, -0.0, 1e-20, 9.99e-13):
        s, si = scaling.scale_from_amax(a)
        fl = Fraction(float(scaling.AMAX_FLOOR))
        assert s == nearest_f32(fl / 448) and si == nearest_f32(448 / fl)


def test_nan_amax_propagates():
    s, si = scaling.scale_from_amax(np.float32(np.nan))
    assert np.isnan(s) and np.isnan(si)


def test_current_scale_maps_amax_to_448():
    """With scale_inv = 448/amax, |x| = amax lands in (432, 464) and encodes to 0x7E."""
    from oracle.quantize import quantize_values
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 0x7F80, size=5000).astype(np.uint16)        # positive finite bf16
    for b in bits:
        a = (np.uint32(b) << 16).view(np.float32)
        if a < 1e-12:
            continue
        _, si = scaling.scale_from_amax(a)
        assert quantize_values(np.array([b], np.uint16), si)[0] == 0x7E
        assert quantize_values(np.array([b | 0x8000], np.uint16), si)[0] == 0xFE


def _golden_ring(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "weight_ring_schedule.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, lo, hi, s, si = line.split()
            rows.append((name, int(lo), int(hi), Fraction(s), Fraction(si)))
    return rows


SEQ = {
    "inc": lambda t: Fraction(t, 64),
    "dec": lambda t: Fraction(64 - t, 64),
    "const": lambda t: Fraction(1, 4),
    "spike": lambda t: Fraction(2) if t == 20 else Fraction(1, 64),
    "zero": lambda t: Fraction(0),
}


def test_weight_ring_matches_hand_schedule(golden_dir):
    rows = _golden_ring(golden_dir)
    assert {r[0] for r in rows} == set(SEQ)
    for name, amax_of in SEQ.items():
        lin = DelayedLinear()
        expect = {}
        for (n, lo, hi, s, si) in rows:
            if n == name:
                for t in range(lo, hi + 1):
                    expect[t] = (nearest_f32(s), nearest_f32(si))
        for t in range(1, 51):
            lin.begin_step()
            assert (lin.w.scale, lin.w.scale_inv) == expect[t], (name, t)
            lin.w.record(np.float32(float(amax_of(t))))
            assert lin.w.pos == t % 16


def test_ring_nan_window_keeps_scale():
    m = scaling.WeightScales()
    m.scale, m.scale_inv = np.float32(0.5), np.float32(2.0)
    m.record(np.float32(np.nan))
    m.refresh()
    assert m.scale == np.float32(0.5) and m.scale_inv == np.float32(2.0)


def test_window_and_refresh_predicate():
    """The window as a function of what was recorded: ones at first, entry i mod 16 for the
    i-th amax (17 records wrap to entry 0); refreshes fall on steps 16, 32, ..."""
    w = scaling.window_after([])
    assert w.dtype == np.float32 and np.all(w == 1.0) and w.size == 16
    w = scaling.window_after([np.float32(v) for v in range(2, 19)])   # 17 amaxes: 2 .. 18
    assert w[0] == 18 and w[1] == 3 and w[15] == 17
    assert [t for t in range(1, 50) if scaling.refresh_due(t)] == [16, 32, 48]
    assert scaling.window_scale(np.zeros(16, np.float32)) is None
    assert scaling.window_scale(np.full(16, np.nan, np.float32)) is None
    s, si = scaling.window_scale(np.float32([0.5] * 15 + [448.0]))
    assert s == np.float32(1.0) and si == np.float32(1.0)


def test_activation_and_grad_scales_are_one_step_late():
    """x at step t is quantized with the scale computed from amax_x of step t-1."""
    rng = np.random.default_rng(5)
    lin = DelayedLinear()
    prev = None
    for t in range(1, 5):
        lin.begin_step()
        x = (rng.standard_normal((32, 32)) * (t + 1)).astype(np.float32)
        w = (rng.standard_normal((16, 32)) * 0.02).astype(np.float32)
        g = (rng.standard_normal((32, 16)) * 1e-3).astype(np.float32)
        xb = (x.view(np.uint32) >> 16).astype(np.uint16)
        wb = (w.view(np.uint32) >> 16).astype(np.uint16)
        gb = (g.view(np.uint32) >> 16).astype(np.uint16)
        f = lin.forward(xb, wb)
        b = lin.backward(gb)
        if prev is None:
            assert f["sx_inv"] == 1.0 and b["sg_inv"] == 1.0
        else:
            assert (f["sx"], f["sx_inv"]) == scaling.scale_from_amax(prev[0])
            assert (b["sg"], b["sg_inv"]) == scaling.scale_from_amax(prev[1])
        prev = (f["amax_x"], b["amax_g"])


def test_scales_only_step_follows_the_full_step():
    """The GEMM-free bookkeeping used for long full-size runs tracks forward/backward exactly."""
    import workloads
    full, lite = DelayedLinear(), DelayedLinear()
    w = workloads.linear_inputs(2, 0, M=32, K=32, N=16)["w"]
    for t in range(1, 35):
        d = workloads.linear_inputs(2, t, M=32, K=32, N=16)
        full.begin_step()
        lite.begin_step()
        f = full.forward(d["x"], w, rows_valid=30)
        b = full.backward(d["g"])
        u = lite.scales_only_step(d["x"], w, d["g"], rows_valid=30)
        assert (u["sx"], u["sw"], u["sg"]) == (f["sx"], f["sw"], b["sg"])
        assert (u["sx_inv"], u["sw_inv"], u["sg_inv"]) == (f["sx_inv"], f["sw_inv"], b["sg_inv"])
        s1, s2 = full.state(), lite.state()
        assert np.array_equal(s1.pop("hist"), s2.pop("hist")) and s1 == s2
        w = workloads.drift(w, 2, t, 1e-4)
