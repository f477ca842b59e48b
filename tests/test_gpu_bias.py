"""GPU parity for the bias: the forward epilogue (every GEMM kernel path, ragged shapes,
padded rows, an empty contraction) and the bias gradient (column sums over the valid rows)
against the float64 oracle, within the stated tolerances."""
import numpy as np
import pytest

import workloads
from oracle import gemm
from oracle.bias import add_bias, bias_bound, bias_grad, bias_grad_bound
from oracle.quantize import amax as o_amax
from oracle.quantize import quantize_tensorwise
from oracle.scaling import scale_from_amax
from tests.gpu_util import dev_bf16, dev_f32, host_bf16_bits, host_bf16_f64, note

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_fp8_linear_amd as m
    m.load()
    return m


def _codes(shape, seed, kind="normal", **p):
    bits = workloads.bf16_tensor(kind, shape, 71, seed, 0, **p)
    s, si = scale_from_amax(o_amax(bits))
    q, _, _ = quantize_tensorwise(bits, si)
    return q, s


def _dev(q):
    return torch.from_numpy(np.ascontiguousarray(q)).cuda()


# (M, N, K, M_valid): the 32x32x64 kernels (small outputs, odd K-step counts), the
# 16x16x128 kernel with 256x256 tiles (and its K-tail variant), 224x256 and 256x224 tiles
FWD = [(64, 128, 128, 64), (528, 784, 656, 500), (2064, 2320, 512, 2000),
       (2304, 2048, 528, 2300), (4352, 4096, 512, 4352), (4096, 7152, 512, 1200)]


@pytest.mark.parametrize("M,N,K,mv", FWD)
def test_forward_bias(lib, M, N, K, mv):
    qa, sa = _codes((M, K), 81 + M, "student_t", nu=3)
    qb, sb = _codes((N, K), 82 + N, "normal", std=0.02)
    bias = workloads.bf16_tensor("normal", (N,), 71, 83 + N, 0, std=0.5)
    note(f"fp8_linear_fwd_bias M={M} N={N} K={K} M_valid={mv}")
    y = lib.fp8_linear_fwd(_dev(qa), _dev(qb), dev_f32(sa), dev_f32(sb), M_valid=mv,
                           bias=dev_bf16(bias))
    torch.cuda.synchronize()
    yh = host_bf16_f64(y)
    assert np.all(yh[mv:] == 0)
    D = gemm.scaled_gemm(qa[:mv], qb, sa, sb)
    want = add_bias(D, bias)
    bound = gemm.error_bound(qa[:mv], qb, sa, sb) + bias_bound(bias)[None, :]
    err = np.abs(yh[:mv] - want)
    assert np.all(err <= bound), (np.argmax(err - bound), float(np.max(err - bound)))


def test_forward_bias_empty_contraction_and_unsupported(lib):
    M, N = 64, 256
    bias = workloads.bf16_tensor("normal", (N,), 71, 90, 0, std=1.0)
    note("fp8_linear_fwd_bias with K = 0")
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    lib.fp8_linear_fwd(torch.empty((M, 0), dtype=torch.uint8, device="cuda"),
                       torch.empty((N, 0), dtype=torch.uint8, device="cuda"), dev_f32(1.0),
                       dev_f32(1.0), y=y, M_valid=40, bias=dev_bf16(bias))
    torch.cuda.synchronize()
    yb = host_bf16_bits(y)
    assert np.all(yb[:40] == bias[None, :]) and np.all(yb[40:] == 0)
    note("bias with the block recipe is refused")
    with pytest.raises(lib.Fp8Error):
        lib.fp8_linear_fwd(torch.zeros((128, 128), dtype=torch.uint8, device="cuda"),
                           torch.zeros((128, 128), dtype=torch.uint8, device="cuda"),
                           torch.ones((128, 1), device="cuda"), torch.ones((1, 1), device="cuda"),
                           gran=lib.FP8_BLOCK_1x128, bias=dev_bf16(bias[:128]))


@pytest.mark.parametrize("rows,cols,rv", [(272, 400, 250), (64, 16, 64), (1040, 4096, 1000),
                                          (8192, 4096, 8192), (96, 32, 0)])
def test_bias_grad(lib, rows, cols, rv):
    g = workloads.bf16_tensor("normal", (rows, cols), 71, 91 + rows, 0, std=1e-3)
    g[rv:] = 0x7FC0                        # NaN in the padding rows: never read
    note(f"fp8_bias_grad rows={rows} cols={cols} rows_valid={rv}")
    gd = dev_bf16(g)
    db = lib.fp8_bias_grad(gd, rows_valid=rv)
    db2 = lib.fp8_bias_grad(gd, rows_valid=rv)
    torch.cuda.synchronize()
    assert torch.equal(db.view(torch.int16), db2.view(torch.int16)), "not deterministic"
    got = host_bf16_f64(db)
    err = np.abs(got - bias_grad(g, rv))
    assert np.all(err <= bias_grad_bound(g, rv)), float(np.max(err))
