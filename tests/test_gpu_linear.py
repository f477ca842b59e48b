"""GPU parity for whole steps of the layer: the delayed-scaling schedule, padding, varlen batches.

* small shapes: every quantized byte, amax and scale bit-exact, every GEMM output within the
  tolerance, for 20 consecutive steps (crossing the first ring refresh at step 16);
* config 2 at full size (M = K = N = 4096, 32 steps, drifting W) is in test_gpu_fullsize.py;
* config 4 (packed varlen batch padded to a multiple of 16): padding rows excluded from amax
  and zero in y/dx, with NaN sentinels in the padding.
"""
import numpy as np
import pytest

import workloads
from oracle import gemm
from oracle.linear import DelayedLinear
from oracle.padding import padded_count
from oracle.quantize import quantize_values
from tests.gpu_util import (assert_same_bytes, assert_within, dev_bf16, f32_bits, host_bf16_f64,
                            host_u8, note)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_fp8_linear_amd as m
    m.load()
    return m


def _scales_equal(gpu: dict, ref: dict, what: str) -> None:
    for k in ("w_scale", "w_scale_inv", "x_scale", "x_scale_inv", "g_scale", "g_scale_inv"):
        assert f32_bits(gpu[k]) == f32_bits(ref[k]), (what, k, gpu[k], ref[k])
    assert np.array_equal(gpu["hist"].view(np.uint32), ref["hist"].view(np.uint32)), what
    assert gpu["idx"] == ref["idx"] and gpu["step"] == ref["step"], what


def test_small_shape_every_byte_20_steps(lib):
    """Every code, amax and scale of 20 delayed-scaling steps against the oracle. The layer
    under test keeps its amaxes for inspection; a second layer in the default mode (amax
    folded into a buffer that the scale update clears) must produce the same bytes."""
    M, K, N, rv = 272, 384, 400, 250
    lin = lib.DelayedScalingLinear("cuda", keep_amax=True)
    lin2 = lib.DelayedScalingLinear("cuda")
    ref = DelayedLinear()
    w = workloads.linear_inputs(2, 0, M=M, K=K, N=N)["w"]
    for t in range(1, 21):
        d = workloads.linear_inputs(2, t, M=M, K=K, N=N)
        x, g = d["x"].copy(), d["g"].copy()
        x[rv:] = 0x7FC0                       # sentinels in padding rows
        g[rv:] = 0xFFC0
        note(f"small-shape step {t}")
        lin.begin_step()
        bufs = {}
        y = lin.forward(dev_bf16(x), dev_bf16(w), rows_valid=rv, bufs=bufs)
        dx, dw = lin.backward(dev_bf16(g))
        qx_t, qw_t, _ = lin._saved
        lin2.begin_step()
        y2 = lin2.forward(dev_bf16(x), dev_bf16(w), rows_valid=rv)
        dx2, dw2 = lin2.backward(dev_bf16(g))
        qx_t2, qw_t2, _ = lin2._saved
        torch.cuda.synchronize()
        assert torch.equal(qx_t, qx_t2) and torch.equal(qw_t, qw_t2), f"codes step {t}"
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"y step {t}"
        assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16)), f"dx step {t}"
        assert torch.equal(dw.view(torch.int16), dw2.view(torch.int16)), f"dw step {t}"
        assert f32_bits(lin2.amax_x.item()) == f32_bits(lin2.amax_g.item()) == 0
        assert f32_bits(lin2.amax_w.item()) == 0
        ref.begin_step()
        f = ref.forward(x, w, rows_valid=rv)
        b = ref.backward(g)
        assert f32_bits(lin.amax_x.item()) == f32_bits(f["amax_x"])
        assert f32_bits(lin.amax_w.item()) == f32_bits(f["amax_w"])
        assert f32_bits(lin.amax_g.item()) == f32_bits(b["amax_g"])
        assert_same_bytes(host_u8(qx_t), f["qx_t"], f"qx_t step {t}")
        assert_same_bytes(host_u8(qw_t), f["qw_t"], f"qw_t step {t}")
        assert_within(host_bf16_f64(y), f["y"],
                      gemm.error_bound(f["qx"], f["qw"], f["sx"], f["sw"]), f"y step {t}")
        assert_within(host_bf16_f64(dx), b["dx"],
                      gemm.error_bound(b["qg"], f["qw_t"], b["sg"], f["sw"]), f"dx step {t}")
        assert_within(host_bf16_f64(dw), b["dw"],
                      gemm.error_bound(b["qg_t"], f["qx_t"], b["sg"], f["sx"]), f"dw step {t}")
        lin.end_step()
        lin2.end_step()
        _scales_equal(lin.state(), ref.state(), f"step {t}")
        _scales_equal(lin2.state(), ref.state(), f"default mode, step {t}")
        w = workloads.drift(w, 2, t, 1e-4)


@pytest.mark.parametrize("count,len_hi", [(12, 300), (64, 2048)])
def test_config4_packed_varlen(lib, count, len_hi):
    """Packed THD batch: T = sum of lengths, padded (fp8_pad_tokens) to T_pad % 16 == 0;
    K = N = 4096 at full size. Padding rows: excluded from amax, zero in y and dx."""
    d = workloads.varlen_batch(4, count=count, len_hi=len_hi)
    T = d["T"]
    T_pad = padded_count(T)
    x, w, g = d["x"], d["w"], d["g"]
    note(f"config 4 varlen: {count} seqs, T={T}, T_pad={T_pad}")
    xd, gd = dev_bf16(x), dev_bf16(g)
    xp, tp = lib.fp8_pad_tokens(xd)
    assert tp == T_pad
    # g: pad in place inside a buffer whose tail holds NaN sentinels
    gbuf = torch.full((T_pad, g.shape[1]), float("nan"), dtype=torch.bfloat16, device="cuda")
    gbuf[:T] = gd
    lib.fp8_pad_tokens(gbuf, T=T, x_pad=gbuf)
    torch.cuda.synchronize()
    assert torch.all(xp[T:] == 0).item() and torch.all(gbuf[T:] == 0).item()
    assert torch.equal(xp[:T].view(torch.int16), xd.view(torch.int16))
    # rows_valid = T on top: the sentinel-free padded rows must still be excluded
    lin = lib.DelayedScalingLinear("cuda", keep_amax=True)
    lin.begin_step()
    y = lin.forward(xp, dev_bf16(w), rows_valid=T)
    dx, dw = lin.backward(gbuf)
    torch.cuda.synchronize()
    ref = DelayedLinear()
    ref.begin_step()
    used = ref.scales_only_step(np.concatenate([x, np.zeros((T_pad - T, x.shape[1]), np.uint16)]),
                                w, np.concatenate([g, np.zeros((T_pad - T, g.shape[1]), np.uint16)]),
                                rows_valid=T)
    assert f32_bits(lin.amax_x.item()) == f32_bits(used["amax_x"])
    assert f32_bits(lin.amax_g.item()) == f32_bits(used["amax_g"])
    yh, dxh = host_bf16_f64(y), host_bf16_f64(dx)
    assert np.all(yh[T:] == 0) and np.all(dxh[T:] == 0)
    rng = np.random.default_rng(4)
    dwh = host_bf16_f64(dw)
    for _ in range(16):
        m = int(rng.integers(0, T))
        n, k = (int(v) for v in rng.integers(0, 4096, 2))
        qa = quantize_values(x[m:m + 1], used["sx_inv"])
        qb = quantize_values(w[n:n + 1], used["sw_inv"])
        ex = gemm.scaled_gemm(qa, qb, used["sx"], used["sw"])[0, 0]
        assert abs(yh[m, n] - ex) <= gemm.error_bound(qa, qb, used["sx"], used["sw"])[0, 0]
        qg_col = np.ascontiguousarray(quantize_values(g[:, n], used["sg_inv"])[None, :])
        qx_col = np.ascontiguousarray(quantize_values(x[:, k], used["sx_inv"])[None, :])
        ex = gemm.scaled_gemm(qg_col, qx_col, used["sg"], used["sx"])[0, 0]
        assert abs(dwh[n, k] - ex) <= gemm.error_bound(qg_col, qx_col, used["sg"], used["sx"])[0, 0]
