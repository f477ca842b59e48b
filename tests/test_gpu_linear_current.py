"""The one-launch current-scaling forward of a small linear (fp8_linear_fwd_current)
against the oracle: amaxes, scales and multipliers bit for bit, the codes byte for byte,
y within both GEMM bounds. Config 1 (x [64, 128], W [128, 128], N(0, 1)), other shapes up
to the 64 KiB code limit (one 16x16 tile per workgroup: up to 256 tiles, up to 16 K steps;
amax loads all at once or in batches; a tile's own rows held from the start or read again),
the codes not asked for or only one of them, an all-zero input (the 1e-12 amax clamp), and a
NaN in x or in W (NaN amax, NaN scale: every code of that operand is the NaN code)."""
import numpy as np
import pytest

import workloads
from oracle import gemm
from oracle.linear import current_scaled_forward
from tests.gpu_util import (assert_same_bytes, assert_within, dev_bf16, f32_bits, host_bf16_bits,
                            host_bf16_f64, host_u8, note)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_fp8_linear_amd as m
    m.load()
    return m


def _run(lib, x, w):
    note(f"fp8_linear_fwd_current x {x.shape} w {w.shape}")
    y, sc, qx, qw = lib.fp8_linear_fwd_current(dev_bf16(x), dev_bf16(w), want_codes=True)
    torch.cuda.synchronize()
    return host_bf16_f64(y), sc.cpu().numpy(), host_u8(qx), host_u8(qw)


def _check(lib, x, w):
    y, sc, qx, qw = _run(lib, x, w)
    ref = current_scaled_forward(x, w)
    want = [ref["sx"], ref["sw"], ref["sx_inv"], ref["sw_inv"]]
    assert [f32_bits(v) for v in sc] == [f32_bits(v) for v in want], (sc, want)
    assert_same_bytes(qx, ref["qx"], "qx")
    assert_same_bytes(qw, ref["qw"], "qw")
    D, tight = gemm.fp32_bound(ref["qx"], ref["qw"], ref["sx"], ref["sw"])
    assert_within(y, D, gemm.error_bound(ref["qx"], ref["qw"], ref["sx"], ref["sw"]), "y")
    assert_within(y, D, tight, "y (float32 accumulation)")


def test_config1(lib):
    d = workloads.linear_inputs(1)
    assert d["x"].shape == (64, 128) and d["w"].shape == (128, 128)
    _check(lib, d["x"], d["w"])


@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (32, 96, 256), (256, 256, 128),
                                   (128, 128, 256), (48, 208, 128), (16, 496, 128),
                                   (112, 16, 128), (32, 16, 512), (16, 16, 2048)])
def test_shapes(lib, M, N, K):
    d = workloads.linear_inputs(2, 1, M=M, K=K, N=N)
    _check(lib, d["x"], d["w"])
    o = workloads.bf16_tensor("outlier_normal", (M, K), 5, 3 + M, 0, rate=0.01, mult=100.0)
    _check(lib, o, d["w"])


def test_codes_not_wanted(lib):
    d = workloads.linear_inputs(2, 1, M=48, K=384, N=80)
    _check(lib, d["x"], d["w"])
    note("fp8_linear_fwd_current x (48, 384) w (80, 384), with and without qx, qw")
    y1, sc1, _, _ = lib.fp8_linear_fwd_current(dev_bf16(d["x"]), dev_bf16(d["w"]),
                                               want_codes=True)
    y2, sc2, qx2, qw2 = lib.fp8_linear_fwd_current(dev_bf16(d["x"]), dev_bf16(d["w"]))
    torch.cuda.synchronize()
    assert qx2 is None and qw2 is None
    assert_same_bytes(host_bf16_bits(y2), host_bf16_bits(y1), "y")
    assert_same_bytes(host_u8(sc2), host_u8(sc1), "scales")


def test_zero_input(lib):
    d = workloads.linear_inputs(1)
    x = np.zeros_like(d["x"])
    _check(lib, x, d["w"])


def test_nan_in_x(lib):
    d = workloads.linear_inputs(1)
    x = d["x"].copy()
    x[5, 17] = 0x7FC0                      # a quiet NaN
    y, sc, qx, qw = _run(lib, x, d["w"])
    ref = current_scaled_forward(x, d["w"])
    assert np.isnan(sc[0]) and np.isnan(sc[2]) and np.isnan(ref["sx"])
    assert f32_bits(sc[1]) == f32_bits(ref["sw"]) and f32_bits(sc[3]) == f32_bits(ref["sw_inv"])
    assert_same_bytes(qx, ref["qx"], "qx (NaN multiplier)")
    assert_same_bytes(qw, ref["qw"], "qw")
    assert np.all(np.isnan(y))


def test_one_code_tensor(lib):
    """qx asked for without qw, then qw without qx: each is written whole by its own tiles."""
    d = workloads.linear_inputs(2, 1, M=48, K=256, N=64)
    ref = current_scaled_forward(d["x"], d["w"])
    note("fp8_linear_fwd_current x (48, 256) w (64, 256), qx only then qw only")
    qx = torch.full((48, 256), 0xAB, dtype=torch.uint8, device="cuda")
    lib.fp8_linear_fwd_current(dev_bf16(d["x"]), dev_bf16(d["w"]), qx=qx)
    qw = torch.full((64, 256), 0xAB, dtype=torch.uint8, device="cuda")
    lib.fp8_linear_fwd_current(dev_bf16(d["x"]), dev_bf16(d["w"]), qw=qw)
    torch.cuda.synchronize()
    assert_same_bytes(host_u8(qx), ref["qx"], "qx")
    assert_same_bytes(host_u8(qw), ref["qw"], "qw")


def test_nan_in_w(lib):
    d = workloads.linear_inputs(2, 1, M=32, K=128, N=48)
    w = d["w"].copy()
    w[40, 3] = 0xFFC0                      # a negative quiet NaN, in the last tile row of W
    y, sc, qx, qw = _run(lib, d["x"], w)
    ref = current_scaled_forward(d["x"], w)
    assert np.isnan(sc[1]) and np.isnan(sc[3]) and np.isnan(ref["sw"])
    assert f32_bits(sc[0]) == f32_bits(ref["sx"]) and f32_bits(sc[2]) == f32_bits(ref["sx_inv"])
    assert_same_bytes(qx, ref["qx"], "qx")
    assert_same_bytes(qw, ref["qw"], "qw (NaN multiplier)")
    assert np.all(np.isnan(y))
