"""GPU parity for the autograd wrapper (Fp8Linear inside fp8_autocast) against the oracle's
delayed-scaling layer: outputs, input and weight gradients within the GEMM tolerance, the
whole scale schedule bit-exact, for aligned and ragged token counts; state saved and
restored mid-run continues byte for byte; a step without backward keeps the gradient
scale."""
import numpy as np
import pytest

import workloads
from oracle import gemm
from oracle.bias import add_bias, bias_bound, bias_grad, bias_grad_bound
from oracle.linear import DelayedLinear
from tests.gpu_util import assert_within, dev_bf16, f32_bits, host_bf16_f64, note

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


def _pad(bits, rows):
    out = np.zeros((rows, bits.shape[1]), np.uint16)
    out[:bits.shape[0]] = bits
    return out


@pytest.mark.parametrize("M", [272, 250])
def test_module_matches_oracle_20_steps(lib, M):
    K, N = 384, 400
    lib.fp8_state().reset()
    layer = lib.Fp8Linear(K, N, device="cuda")
    ref = DelayedLinear()
    Mp = M + (-M) % 16
    w = workloads.linear_inputs(2, 0, M=Mp, K=K, N=N)["w"]
    for t in range(1, 21):
        d = workloads.linear_inputs(2, t, M=Mp, K=K, N=N)
        x, g = d["x"][:M], d["g"][:M]
        note(f"Fp8Linear step {t} M={M}")
        layer.weight.data.copy_(dev_bf16(w))
        layer.weight.grad = None
        xd = dev_bf16(x).requires_grad_(True)
        with lib.fp8_autocast():
            y = layer(xd)
        y.backward(dev_bf16(g))
        torch.cuda.synchronize()
        ref.begin_step()
        f = ref.forward(_pad(x, Mp), w, rows_valid=M)
        b = ref.backward(_pad(g, Mp))
        assert tuple(y.shape) == (M, N) and tuple(xd.grad.shape) == (M, K)
        assert_within(host_bf16_f64(y), f["y"][:M],
                      gemm.error_bound(f["qx"], f["qw"], f["sx"], f["sw"])[:M], f"y step {t}")
        assert_within(host_bf16_f64(xd.grad), b["dx"][:M],
                      gemm.error_bound(b["qg"], f["qw_t"], b["sg"], f["sw"])[:M],
                      f"dx step {t}")
        assert_within(host_bf16_f64(layer.weight.grad), b["dw"],
                      gemm.error_bound(b["qg_t"], f["qx_t"], b["sg"], f["sx"]), f"dw step {t}")
        _scales_equal(layer._lin.state(), ref.state(), f"step {t}")
        w = workloads.drift(w, 2, t, 1e-4)
    lib.fp8_state().reset()


def _run(lib, layer, steps, first, M=256, K=256, N=384):
    """Steps first .. first + steps - 1 of a fixed input schedule; the raw bytes of y,
    x.grad and W.grad of each step."""
    outs = []
    for t in range(first, first + steps):
        d = workloads.linear_inputs(2, t, M=M, K=K, N=N)
        layer.weight.data.copy_(dev_bf16(d["w"]))
        layer.weight.grad = None
        xd = dev_bf16(d["x"]).requires_grad_(True)
        with lib.fp8_autocast():
            y = layer(xd)
        y.backward(dev_bf16(d["g"]))
        torch.cuda.synchronize()
        outs.append([y.view(torch.int16).cpu(), xd.grad.view(torch.int16).cpu(),
                     layer.weight.grad.view(torch.int16).cpu()])
    return outs


def test_state_save_and_restore(lib):
    """18 steps in one go against 13 steps, save, restore into a fresh layer, 5 more: the
    last 5 steps (crossing the refresh at step 16) agree byte for byte."""
    lib.fp8_state().reset()
    note("save/restore: uninterrupted run")
    a = lib.Fp8Linear(256, 384, device="cuda")
    full = _run(lib, a, 18, 1)
    lib.fp8_state().reset()
    note("save/restore: 13 steps, save, restore, 5 steps")
    b = lib.Fp8Linear(256, 384, device="cuda")
    _run(lib, b, 13, 1)
    sd = {k: v.clone() if torch.is_tensor(v) else v for k, v in b.state_dict().items()}
    gsd = lib.fp8_state().state_dict()
    del b
    lib.fp8_state().reset()
    c = lib.Fp8Linear(256, 384, device="cuda")
    c.load_state_dict(sd)
    lib.fp8_state().load_state_dict(gsd)
    tail = _run(lib, c, 5, 14)
    for i, (u, v) in enumerate(zip(full[13:], tail)):
        for name, p, q in zip(("y", "dx", "dw"), u, v):
            assert torch.equal(p, q), (i + 14, name)
    lib.fp8_state().reset()


def test_step_without_backward(lib):
    """Step 2 runs the forward under no_grad: the activation scale still advances, the
    gradient scale is carried over, and step 3 matches the oracle that skipped a backward."""
    M, K, N = 256, 256, 384
    lib.fp8_state().reset()
    layer = lib.Fp8Linear(K, N, device="cuda")
    ref = DelayedLinear()
    for t in (1, 2, 3):
        d = workloads.linear_inputs(2, t, M=M, K=K, N=N)
        note(f"no-backward schedule, step {t}")
        layer.weight.data.copy_(dev_bf16(d["w"]))
        layer.weight.grad = None
        ref.begin_step()
        if t == 2:
            with lib.fp8_autocast(), torch.no_grad():
                y = layer(dev_bf16(d["x"]))
            f = ref.forward(d["x"], d["w"])
            torch.cuda.synchronize()
            assert_within(host_bf16_f64(y), f["y"],
                          gemm.error_bound(f["qx"], f["qw"], f["sx"], f["sw"]), "y no_grad")
            continue
        xd = dev_bf16(d["x"]).requires_grad_(True)
        with lib.fp8_autocast():
            y = layer(xd)
        y.backward(dev_bf16(d["g"]))
        torch.cuda.synchronize()
        f = ref.forward(d["x"], d["w"])
        b = ref.backward(d["g"])
        assert_within(host_bf16_f64(xd.grad), b["dx"],
                      gemm.error_bound(b["qg"], f["qw_t"], b["sg"], f["sw"]), f"dx step {t}")
        _scales_equal(layer._lin.state(), ref.state(), f"step {t}")
    lib.fp8_state().reset()


@pytest.mark.parametrize("M", [256, 250])
def test_module_with_bias(lib, M):
    """Fp8Linear(bias=True): y = x W^T + b through the bias epilogue, db the column sum of
    the output gradient over the valid tokens; 3 steps against the oracle."""
    K, N = 256, 384
    lib.fp8_state().reset()
    layer = lib.Fp8Linear(K, N, bias=True, device="cuda")
    ref = DelayedLinear()
    Mp = M + (-M) % 16
    for t in (1, 2, 3):
        d = workloads.linear_inputs(2, t, M=Mp, K=K, N=N)
        x, g, w = d["x"][:M], d["g"][:M], d["w"]
        bias = workloads.bf16_tensor("normal", (N,), 2, 99, t, std=0.1)
        note(f"Fp8Linear with bias, step {t}, M={M}")
        layer.weight.data.copy_(dev_bf16(w))
        layer.bias.data.copy_(dev_bf16(bias))
        layer.weight.grad = None
        layer.bias.grad = None
        xd = dev_bf16(x).requires_grad_(True)
        with lib.fp8_autocast():
            y = layer(xd)
        y.backward(dev_bf16(g))
        torch.cuda.synchronize()
        ref.begin_step()
        f = ref.forward(_pad(x, Mp), w, rows_valid=M)
        b = ref.backward(_pad(g, Mp))
        want = add_bias(f["y"][:M], bias)
        bound = gemm.error_bound(f["qx"], f["qw"], f["sx"], f["sw"])[:M] + bias_bound(bias)[None, :]
        assert_within(host_bf16_f64(y), want, bound, f"y step {t}")
        assert_within(host_bf16_f64(layer.bias.grad), bias_grad(_pad(g, Mp), M),
                      bias_grad_bound(_pad(g, Mp), M), f"db step {t}")
        assert_within(host_bf16_f64(xd.grad), b["dx"][:M],
                      gemm.error_bound(b["qg"], f["qw_t"], b["sg"], f["sw"])[:M], f"dx step {t}")
        _scales_equal(layer._lin.state(), ref.state(), f"step {t}")
    lib.fp8_state().reset()


def test_module_with_e5m2_gradients(lib):
    """Fp8Linear(grad_format="e5m2") through torch autograd, 18 steps (across the step-16
    refresh) at a ragged token count, against the oracle's hybrid-format layer."""
    M, K, N = 250, 384, 400
    lib.fp8_state().reset()
    layer = lib.Fp8Linear(K, N, device="cuda", grad_format="e5m2")
    ref = DelayedLinear(grad_format="e5m2")
    Mp = M + (-M) % 16
    w = workloads.linear_inputs(2, 0, M=Mp, K=K, N=N)["w"]
    for t in range(1, 19):
        d = workloads.linear_inputs(2, t, M=Mp, K=K, N=N)
        x, g = d["x"][:M], d["g"][:M]
        note(f"Fp8Linear e5m2 step {t}")
        layer.weight.data.copy_(dev_bf16(w))
        layer.weight.grad = None
        xd = dev_bf16(x).requires_grad_(True)
        with lib.fp8_autocast():
            y = layer(xd)
        y.backward(dev_bf16(g))
        torch.cuda.synchronize()
        ref.begin_step()
        f = ref.forward(_pad(x, Mp), w, rows_valid=M)
        b = ref.backward(_pad(g, Mp))
        assert_within(host_bf16_f64(y), f["y"][:M],
                      gemm.error_bound(f["qx"], f["qw"], f["sx"], f["sw"])[:M], f"y step {t}")
        assert_within(host_bf16_f64(xd.grad), b["dx"][:M],
                      gemm.error_bound(b["qg"], f["qw_t"], b["sg"], f["sw"], a_fmt="e5m2")[:M],
                      f"dx step {t}")
        assert_within(host_bf16_f64(layer.weight.grad), b["dw"],
                      gemm.error_bound(b["qg_t"], f["qx_t"], b["sg"], f["sx"], a_fmt="e5m2"),
                      f"dw step {t}")
        _scales_equal(layer._lin.state(), ref.state(), f"step {t}")
        w = workloads.drift(w, 2, t, 1e-4)
    sd = layer.state_dict()
    same = lib.Fp8Linear(K, N, device="cuda", grad_format="e5m2")
    same.load_state_dict(sd)
    assert same._lin.grad_format == "e5m2"
    _scales_equal(same._lin.state(), ref.state(), "restored")
    fresh = lib.Fp8Linear(K, N, device="cuda")            # E4M3 gradients: a mismatch
    with pytest.raises(ValueError):
        fresh.load_state_dict(sd)
    lib.fp8_state().reset()
