"""Pins for the oracle's layer wiring: which operands and scales each GEMM takes (CPU only).

The library routine here is PyTorch's CPU autograd in float64: for y = x W^T,
dx = g W and dW = g^T x. Fed the dequantized operands (codes times their
scales), autograd must reproduce the oracle's forward, dgrad and wgrad, which
the oracle computes from the transposed copies instead. A swapped transposed
copy, a wrong scale pair or a missing padding mask fails here.
"""
import numpy as np
import torch

import workloads
from oracle import block, e4m3
from oracle.linear import DelayedLinear, block_linear_step, current_scaled_forward


def _autograd(xdq, wdq, gdq):
    x = torch.tensor(xdq, dtype=torch.float64, requires_grad=True)
    w = torch.tensor(wdq, dtype=torch.float64, requires_grad=True)
    y = torch.nn.functional.linear(x, w)
    y.backward(torch.tensor(gdq, dtype=torch.float64))
    return y.detach().numpy(), x.grad.numpy(), w.grad.numpy()


def _close(a, b):
    scale = max(1.0, float(np.abs(b).max()))
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12 * scale)


def test_delayed_linear_matches_autograd():
    lin = DelayedLinear()
    for step in range(3):
        d = workloads.linear_inputs(2, step, M=48, K=64, N=32)
        d["g"] = (workloads.bf16_to_f32(d["g"]) * 1000).astype(np.float32)   # O(1) grads
        d["g"] = workloads.f32_to_bf16(d["g"])
        lin.begin_step()
        f = lin.forward(d["x"], d["w"], rows_valid=40)
        b = lin.backward(d["g"])
        xdq = e4m3.decode(f["qx"]) * np.float64(f["sx"])
        wdq = e4m3.decode(f["qw"]) * np.float64(f["sw"])
        gdq = e4m3.decode(b["qg"]) * np.float64(b["sg"])
        y, dx, dw = _autograd(xdq, wdq, gdq)
        y[40:] = 0.0
        dx[40:] = 0.0
        _close(f["y"], y)
        _close(b["dx"], dx)
        _close(b["dw"], dw)
        assert np.all(f["qx"][40:] == 0) and np.all(b["qg"][40:] == 0)


def test_current_forward_matches_autograd():
    d = workloads.linear_inputs(1)
    f = current_scaled_forward(d["x"], d["w"])
    xdq = e4m3.decode(f["qx"]) * np.float64(f["sx"])
    wdq = e4m3.decode(f["qw"]) * np.float64(f["sw"])
    y, _, _ = _autograd(xdq, wdq, np.zeros((64, 128)))
    _close(f["y"], y)
    assert (f["qx"] & 0x7F).max() == 0x7E     # current scaling: amax maps to 448


def test_block_linear_matches_autograd():
    M, K, N = 256, 256, 384
    d = workloads.linear_inputs(5, 0, M=M, K=K, N=N)
    r = block_linear_step(d["x"], d["w"], d["g"], rows_valid=200)
    xdq = block.dequant_rows(r["qx"], r["sx"], 1)
    wdq = block.dequant_rows(r["qw"], r["sw"], 128)
    gdq = block.dequant_rows(r["qg"], r["sg"], 1)
    y, dx, _ = _autograd(xdq, wdq, gdq)
    y[200:] = 0.0
    dx[200:] = 0.0
    _close(r["y"], y)
    _close(r["dx"], dx)
    # wgrad contracts over tokens with the transposed copies' own tile scales
    gdq_t = block.dequant_rows(r["qg_t"], r["sg_t"], 1)      # [N, M]
    xdq_t = block.dequant_rows(r["qx_t"], r["sx_t"], 1)      # [K, M]
    _close(r["dw"], gdq_t @ xdq_t.T)
    _, _, dw_ref = _autograd(xdq_t.T, wdq, gdq_t.T)
    _close(r["dw"], dw_ref)


def test_hybrid_format_linear_matches_autograd():
    """E5M2 gradients: the gradient scale comes from 57344 and dgrad/wgrad decode
    Qg and Qg^T as E5M2."""
    from oracle import e5m2, scaling
    lin = DelayedLinear(grad_format="e5m2")
    for step in range(3):
        d = workloads.linear_inputs(2, step, M=48, K=64, N=32)
        lin.begin_step()
        f = lin.forward(d["x"], d["w"], rows_valid=40)
        b = lin.backward(d["g"])
        xdq = e4m3.decode(f["qx"]) * np.float64(f["sx"])
        wdq = e4m3.decode(f["qw"]) * np.float64(f["sw"])
        gdq = e5m2.decode(b["qg"]) * np.float64(b["sg"])
        y, dx, dw = _autograd(xdq, wdq, gdq)
        y[40:] = 0.0
        dx[40:] = 0.0
        _close(f["y"], y)
        _close(b["dx"], dx)
        _close(b["dw"], dw)
        # the next gradient scale is amax/57344 (one step late)
        assert lin.g_scale == scaling.scale_from_amax(b["amax_g"], 57344.0)[0]
        assert np.all(b["qg"][40:] == 0)
