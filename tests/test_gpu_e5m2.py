"""GPU parity for the hybrid format: gradients coded in OCP E5M2, x and W in E4M3.

* quantize: every bf16 pattern times a set of multipliers, the codes and their transpose
  bit-exact with the oracle's E5M2 encoder; ragged shapes with padding sentinels; amax;
* scale update with 57344 as the format maximum, bit-exact;
* the GEMM with an E5M2 first operand (dgrad, wgrad), within the tolerance against the
  float64 oracle, on both kernel families (16x16x128 for large outputs, 32x32x64 otherwise);
* whole layer steps with E5M2 gradients: codes, amaxes and the scale trajectory bit-exact
  with the oracle's hybrid layer, the GEMM outputs within the tolerance.
"""
import numpy as np
import pytest

import workloads
from oracle import gemm
from oracle.linear import DelayedLinear
from oracle.quantize import amax as o_amax
from oracle.quantize import quantize_tensorwise, quantize_values
from oracle.scaling import E5M2_MAX, scale_from_amax
from tests.gpu_util import (assert_same_bytes, assert_within, dev_bf16, dev_f32, f32_bits,
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


ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
SCALES = [1.0, 57344.0, 0.5, 2.0 ** -20, 2.0 ** 20, 57344.0 / 3.0, 57344.0 / 1e-3,
          57344.0 / 1e-12, 3.14159, 1e-30, 448.0]


@pytest.mark.parametrize("scale_inv", SCALES)
def test_every_bf16_pattern_e5m2(lib, scale_inv):
    note(f"e5m2 quantize all bf16 patterns, scale_inv={scale_inv}")
    x = dev_bf16(ALL_BF16)
    q, qt, a, _, _ = lib.fp8_quantize_amax(x, scale_inv=dev_f32(scale_inv), e5m2=True)
    torch.cuda.synchronize()
    oq = quantize_values(ALL_BF16, np.float32(scale_inv), "e5m2")
    assert_same_bytes(host_u8(q), oq, f"e5m2 all-bf16 q scale_inv={scale_inv}")
    assert_same_bytes(host_u8(qt), np.ascontiguousarray(oq.T), "e5m2 all-bf16 q_t")
    assert np.isnan(a.item())


@pytest.mark.parametrize("rows,cols,rv", [(144, 272, 144), (272, 528, 200), (1040, 784, 1033)])
def test_ragged_shapes_and_padding_e5m2(lib, rows, cols, rv):
    g = workloads.bf16_tensor("normal", (rows, cols), 95, rows, cols, std=1e-3)
    g[rv:] = 0xFFC0
    _, si = scale_from_amax(o_amax(g, rv), E5M2_MAX)
    note(f"e5m2 quantize [{rows},{cols}] rows_valid={rv}")
    q, qt, a, _, _ = lib.fp8_quantize_amax(dev_bf16(g), rows_valid=rv, scale_inv=dev_f32(si),
                                           e5m2=True)
    torch.cuda.synchronize()
    oq, oqt, oa = quantize_tensorwise(g, si, rv, "e5m2")
    assert_same_bytes(host_u8(q), oq, "e5m2 q")
    assert_same_bytes(host_u8(qt), oqt, "e5m2 q_t")
    assert f32_bits(a.item()) == f32_bits(oa)


def test_scale_update_e5m2(lib):
    rng = np.random.default_rng(7)
    amaxes = np.concatenate([rng.lognormal(-5, 5, 64), [0.0, 1e-13, 1e-12, 57344.0, 3e5]])
    for a in amaxes.astype(np.float32):
        am = dev_f32(a)
        s, si = dev_f32(0.0), dev_f32(0.0)
        note(f"e5m2 scale from amax {a}")
        lib.fp8_scale_update(lib.FP8_SCALE_FROM_AMAX, amax=am, scale=s, scale_inv=si, e5m2=True)
        torch.cuda.synchronize()
        os_, osi = scale_from_amax(a, E5M2_MAX)
        assert f32_bits(s.item()) == f32_bits(os_) and f32_bits(si.item()) == f32_bits(osi), a
    hist = dev_f32(rng.lognormal(-4, 2, 16).astype(np.float32))
    s, si = dev_f32(1.0), dev_f32(1.0)
    lib.fp8_scale_update(lib.FP8_SCALE_REFRESH, hist=hist, scale=s, scale_inv=si, e5m2=True)
    torch.cuda.synchronize()
    m = np.float32(hist.cpu().numpy().max())
    assert f32_bits(s.item()) == f32_bits(np.float32(m / np.float32(57344.0)))
    assert f32_bits(si.item()) == f32_bits(np.float32(np.float32(57344.0) / m))


def _e5m2_codes(shape, seed):
    """Gradient-like E5M2 codes: N(0, 1e-3) quantized with its current scale."""
    g = workloads.bf16_tensor("normal", shape, seed, *shape, std=1e-3)
    s, si = scale_from_amax(o_amax(g), E5M2_MAX)
    return quantize_values(g, si, "e5m2"), s


def _e4m3_codes(shape, seed):
    w = workloads.bf16_tensor("normal", shape, seed, *shape, std=0.02)
    s, si = scale_from_amax(o_amax(w))
    return quantize_values(w, si), s


def _dev_u8(q):
    return torch.from_numpy(np.ascontiguousarray(q)).cuda()


@pytest.mark.parametrize("M,N,K,mv", [(2048, 2304, 2048, 2000), (2064, 2080, 2112, 2050),
                                       (272, 400, 384, 250), (96, 160, 48, 96)])
def test_dgrad_wgrad_with_e5m2_gradients(lib, M, N, K, mv):
    """dgrad: A = Qg [M, N] (E5M2), B = Qw^T [K, N]; wgrad: A = Qg^T [N, M], B = Qx^T [K, M]."""
    qg, sg = _e5m2_codes((M, N), 96)
    qg[mv:] = 0
    qw_t, sw = _e4m3_codes((K, N), 97)
    qx_t, sx = _e4m3_codes((K, M), 98)
    qx_t[:, mv:] = 0
    qg_t = np.ascontiguousarray(qg.T)
    note(f"e5m2 dgrad M={M} N={N} K={K} mv={mv}")
    dx = lib.fp8_linear_dgrad(_dev_u8(qg), _dev_u8(qw_t), dev_f32(sg), dev_f32(sw), M_valid=mv,
                              a_e5m2=True)
    note(f"e5m2 wgrad M={M} N={N} K={K}")
    dw = lib.fp8_linear_wgrad(_dev_u8(qg_t), _dev_u8(qx_t), dev_f32(sg), dev_f32(sx),
                              a_e5m2=True)
    torch.cuda.synchronize()
    ex = gemm.scaled_gemm(qg, qw_t, sg, sw, "e5m2")
    ex[mv:] = 0.0
    assert_within(host_bf16_f64(dx), ex, gemm.error_bound(qg, qw_t, sg, sw, a_fmt="e5m2"), "dx")
    ew = gemm.scaled_gemm(qg_t, qx_t, sg, sx, "e5m2")
    assert_within(host_bf16_f64(dw), ew, gemm.error_bound(qg_t, qx_t, sg, sx, a_fmt="e5m2"), "dw")
    # the codes are really read as E5M2: the same bytes read as E4M3 give another result
    dx4 = lib.fp8_linear_dgrad(_dev_u8(qg), _dev_u8(qw_t), dev_f32(sg), dev_f32(sw), M_valid=mv)
    torch.cuda.synchronize()
    assert not torch.equal(dx4.view(torch.int16), dx.view(torch.int16))


def test_layer_steps_with_e5m2_gradients(lib):
    """18 steps (across the step-16 refresh) of the hybrid layer against the oracle's."""
    M, K, N, rv = 272, 384, 400, 250
    lin = lib.DelayedScalingLinear("cuda", keep_amax=True, grad_format="e5m2")
    ref = DelayedLinear(grad_format="e5m2")
    w = workloads.linear_inputs(2, 0, M=M, K=K, N=N)["w"]
    for t in range(1, 19):
        d = workloads.linear_inputs(2, t, M=M, K=K, N=N)
        x, g = d["x"].copy(), d["g"].copy()
        x[rv:] = 0x7FC0
        g[rv:] = 0xFFC0
        note(f"hybrid-format step {t}")
        lin.begin_step()
        y = lin.forward(dev_bf16(x), dev_bf16(w), rows_valid=rv)
        dx, dw = lin.backward(dev_bf16(g))
        qx_t, qw_t, _ = lin._saved
        torch.cuda.synchronize()
        ref.begin_step()
        f = ref.forward(x, w, rows_valid=rv)
        b = ref.backward(g)
        assert f32_bits(lin.amax_g.item()) == f32_bits(b["amax_g"]), t
        assert_same_bytes(host_u8(qx_t), f["qx_t"], f"qx_t step {t}")
        assert_within(host_bf16_f64(y), f["y"],
                      gemm.error_bound(f["qx"], f["qw"], f["sx"], f["sw"]), f"y step {t}")
        assert_within(host_bf16_f64(dx), b["dx"],
                      gemm.error_bound(b["qg"], f["qw_t"], b["sg"], f["sw"], a_fmt="e5m2"),
                      f"dx step {t}")
        assert_within(host_bf16_f64(dw), b["dw"],
                      gemm.error_bound(b["qg_t"], f["qx_t"], b["sg"], f["sx"], a_fmt="e5m2"),
                      f"dw step {t}")
        lin.end_step()
        st, rs = lin.state(), ref.state()
        for k in ("w_scale", "w_scale_inv", "x_scale", "x_scale_inv", "g_scale", "g_scale_inv"):
            assert f32_bits(st[k]) == f32_bits(rs[k]), (t, k, st[k], rs[k])
        w = workloads.drift(w, 2, t, 1e-4)


@pytest.mark.parametrize("M,N,K,what", [(8192, 4096, 14336, "dgrad of gate/up"),
                                        (14336, 4096, 8192, "wgrad of gate/up"),
                                        (4096, 14336, 8192, "wgrad of the down projection"),
                                        (8192, 14336, 4096, "dgrad of the down projection")])
def test_full_size_backward_e5m2_sampled(lib, M, N, K, what):
    """The MLP block's backward launch shapes with E5M2 gradients, in the launch configuration
    the benchmark times: the gradient quantized to E5M2 on the GPU (bit-exact with the oracle
    above), the E4M3 operand likewise, 1024 sampled outputs computed one by one by the oracle
    from the sampled rows."""
    a = workloads.bf16_tensor("normal", (M, K), 3, 61 + K, 0, std=1e-3)
    b = workloads.bf16_tensor("student_t", (N, K), 3, 62 + K, 0, nu=3)
    sa, sai = scale_from_amax(o_amax(a), E5M2_MAX)
    sb, sbi = scale_from_amax(o_amax(b))
    note(f"full size e5m2 {what}: quantize operands on the GPU")
    qa, _, _, _, _ = lib.fp8_quantize_amax(dev_bf16(a), scale_inv=dev_f32(sai), want_q_t=False,
                                           e5m2=True)
    qb, _, _, _, _ = lib.fp8_quantize_amax(dev_bf16(b), scale_inv=dev_f32(sbi), want_q_t=False)
    note(f"full size e5m2 {what}: GEMM {M}x{N}x{K}")
    y = lib.fp8_linear_dgrad(qa, qb, dev_f32(sa), dev_f32(sb), a_e5m2=True)
    torch.cuda.synchronize()
    yh = host_bf16_f64(y)
    rng = np.random.default_rng(K + 1)
    for m, n in zip(rng.integers(0, M, 1024), rng.integers(0, N, 1024)):
        ra = quantize_values(a[m:m + 1], sai, "e5m2")
        rb = quantize_values(b[n:n + 1], sbi)
        D = gemm.scaled_gemm(ra, rb, sa, sb, "e5m2")[0, 0]
        bound = gemm.error_bound(ra, rb, sa, sb, a_fmt="e5m2")[0, 0]
        assert abs(yh[m, n] - D) <= bound, (what, m, n, yh[m, n], D, bound)


def test_full_size_gradient_e5m2(lib):
    """g [8192, 14336] N(0, 1e-3) at the MLP block's size, coded in E5M2 with a stale
    multiplier (both tails saturate): amax exact over the whole tensor, codes and transposed
    codes bit-exact on sampled rows and columns."""
    g = workloads.bf16_tensor("normal", (8192, 14336), 3, workloads.T_G, 0, std=1e-3)
    oa = o_amax(g)
    _, si = scale_from_amax(np.float32(oa / 4), E5M2_MAX)
    note("e5m2 quantize full size [8192,14336]")
    q, qt, a, _, _ = lib.fp8_quantize_amax(dev_bf16(g), scale_inv=dev_f32(si), e5m2=True)
    torch.cuda.synchronize()
    assert f32_bits(a.item()) == f32_bits(oa)
    rng = np.random.default_rng(9)
    for r in rng.choice(8192, 16, replace=False):
        want = quantize_values(g[r], si, "e5m2")
        assert_same_bytes(host_u8(q[int(r)]), want, f"row {r}")
    for c in rng.choice(14336, 16, replace=False):
        want = quantize_values(g[:, c], si, "e5m2")
        assert_same_bytes(host_u8(qt[int(c)]), want, f"q_t row {c}")
    qh = host_u8(q)
    assert (qh == 0x7B).any() and (qh == 0xFB).any()
