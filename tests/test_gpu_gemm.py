"""GPU parity: the scaled FP8 GEMMs (forward, dgrad, wgrad) against the exact float64 oracle.

Tolerance (per element): |D_gpu - D| <= 1e-2 * ||dqA[m,:]||_2 * ||dqB[n,:]||_2, the target
stated for the method, with D the exact result and dq the dequantized operands. The GPU result
is float32-accumulated and rounded to bf16, which keeps it orders of magnitude inside that
bound; the tests also report the worst ratio.
"""
import numpy as np
import pytest

import workloads
from oracle import e4m3, gemm
from oracle.quantize import quantize_tensorwise
from oracle.scaling import scale_from_amax
from oracle.quantize import amax as o_amax
from tests.gpu_util import assert_within, dev_f32, host_bf16_f64, note

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
    """Random e4m3 operands: quantize seeded bf16 data with its current scale (oracle)."""
    bits = workloads.bf16_tensor(kind, shape, 70, seed, 0, **p)
    s, si = scale_from_amax(o_amax(bits))
    q, _, _ = quantize_tensorwise(bits, si)
    return q, s


def _dev(q):
    return torch.from_numpy(np.ascontiguousarray(q)).cuda()


def _exact_and_bound(qa, qb, sa, sb):
    return gemm.scaled_gemm(qa, qb, sa, sb), gemm.error_bound(qa, qb, sa, sb)


def _within_both(got, qa, qb, sa, sb, what):
    """The tolerance of record and the tight float32-accumulation bound (oracle.gemm)."""
    D, tight = gemm.fp32_bound(qa, qb, sa, sb)
    worst = assert_within(got, D, gemm.error_bound(qa, qb, sa, sb), what)
    assert_within(got, D, tight, f"{what} (float32 accumulation)")
    return worst


SHAPES = [(64, 128, 128), (16, 16, 16), (528, 784, 656), (256, 256, 4096), (1040, 272, 1008),
          (4096 + 16, 512, 144)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_forward(lib, M, N, K):
    qa, sa = _codes((M, K), 1 + M, "student_t", nu=3)
    qb, sb = _codes((N, K), 2 + N, "normal", std=0.02)
    note(f"fp8_linear_fwd M={M} N={N} K={K}")
    y = lib.fp8_linear_fwd(_dev(qa), _dev(qb), dev_f32(sa), dev_f32(sb))
    torch.cuda.synchronize()
    D, bound = _exact_and_bound(qa, qb, sa, sb)
    worst = assert_within(host_bf16_f64(y), D, bound, f"fwd {M}x{N}x{K}")
    # the bf16 output rounding alone can use 2**-9 / 1e-2 ~ 0.2 of the bound (|D| <= ||a|| ||b||)
    assert worst < 0.25


@pytest.mark.parametrize("M,N,K", [(528, 784, 656), (64, 128, 128)])
def test_dgrad_and_wgrad(lib, M, N, K):
    """dgrad = Qg . Qw (via Qw^T), wgrad = Qg^T . Qx (via both transposed copies)."""
    qg, sg = _codes((M, N), 3 + M, "normal", std=1e-3)
    qw, sw = _codes((N, K), 4 + N, "normal", std=0.02)
    qx, sx = _codes((M, K), 5 + K, "student_t", nu=3)
    qw_t, qg_t, qx_t = (np.ascontiguousarray(a.T) for a in (qw, qg, qx))
    note(f"fp8_linear_dgrad M={M} N={N} K={K}")
    dx = lib.fp8_linear_dgrad(_dev(qg), _dev(qw_t), dev_f32(sg), dev_f32(sw))
    note(f"fp8_linear_wgrad M={M} N={N} K={K}")
    dw = lib.fp8_linear_wgrad(_dev(qg_t), _dev(qx_t), dev_f32(sg), dev_f32(sx))
    torch.cuda.synchronize()
    assert tuple(dx.shape) == (M, K) and tuple(dw.shape) == (N, K)
    D, b = _exact_and_bound(qg, qw_t, sg, sw)
    assert_within(host_bf16_f64(dx), D, b, "dgrad")
    D, b = _exact_and_bound(qg_t, qx_t, sg, sx)
    assert_within(host_bf16_f64(dw), D, b, "wgrad")


def test_m_valid_rows_are_zero(lib):
    M, N, K = 272, 256, 128
    qa, sa = _codes((M, K), 11, std=1.0)
    qb, sb = _codes((N, K), 12, std=1.0)
    note("fp8_linear_fwd with M_valid=200")
    y = lib.fp8_linear_fwd(_dev(qa), _dev(qb), dev_f32(sa), dev_f32(sb), M_valid=200)
    note("fp8_linear_dgrad with M_valid=200")
    dx = lib.fp8_linear_dgrad(_dev(qa), _dev(qb), dev_f32(sa), dev_f32(sb), M_valid=200)
    torch.cuda.synchronize()
    yh, dxh = host_bf16_f64(y), host_bf16_f64(dx)
    assert np.all(yh[200:] == 0) and np.all(dxh[200:] == 0)
    D, b = _exact_and_bound(qa[:200], qb, sa, sb)
    assert_within(yh[:200], D, b, "fwd valid rows")


def test_special_operands(lib):
    """All-448 operands at K=4096 (largest partial sums), zeros, and signed zeros."""
    M = N = 128
    K = 4096
    qa = np.full((M, K), 0x7E, np.uint8)
    qa[1::2] = 0xFE
    qb = np.full((N, K), 0x7E, np.uint8)
    qb[:, ::3] = 0x80
    qb[5] = 0
    note("fp8_linear_fwd saturated operands")
    y = lib.fp8_linear_fwd(_dev(qa), _dev(qb), dev_f32(1 / 448), dev_f32(1 / 448))
    torch.cuda.synchronize()
    D, b = _exact_and_bound(qa, qb, np.float32(1 / 448), np.float32(1 / 448))
    assert_within(host_bf16_f64(y), D, b, "saturated")
    assert np.all(host_bf16_f64(y)[:, 5] == 0)


def test_degenerate_shapes(lib):
    """No tokens, an empty contraction (every sum is +0, operands and scales unread), and no
    valid rows, on the small-output kernel and on the 16x16x128 kernel."""
    u8 = dict(dtype=torch.uint8, device="cuda")
    one = dev_f32(1.0)
    note("fp8_linear_fwd with M = 0")
    qb, sb = _codes((128, 128), 61, std=1.0)
    y = lib.fp8_linear_fwd(torch.empty((0, 128), **u8), _dev(qb), one, dev_f32(sb))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 128)
    for N, K in [(128, 64), (2048, 2048)]:
        for gran in (lib.FP8_TENSORWISE, lib.FP8_BLOCK_1x128):
            note(f"fp8_linear_wgrad over 0 tokens N={N} K={K} gran={gran}")
            dw = torch.full((N, K), 3.0, dtype=torch.bfloat16, device="cuda")
            if gran == lib.FP8_TENSORWISE:
                sg, sx = one, one
            else:
                sg = torch.empty((N, 0), dtype=torch.float32, device="cuda")
                sx = torch.empty((K, 0), dtype=torch.float32, device="cuda")
            lib.fp8_linear_wgrad(torch.empty((N, 0), **u8), torch.empty((K, 0), **u8), sg, sx,
                                 dw=dw, gran=gran)
            torch.cuda.synchronize()
            assert torch.all(dw.view(torch.int16) == 0), (N, K, gran)
    for M, N, K in [(64, 128, 128), (2048, 2048, 512)]:
        note(f"fp8_linear_fwd with M_valid = 0, M={M} N={N} K={K}")
        qa = np.full((M, K), 0x7F, np.uint8)          # NaN codes: still zeros
        qb, sb = _codes((N, K), 62 + N, std=1.0)
        y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        lib.fp8_linear_fwd(_dev(qa), _dev(qb), one, dev_f32(sb), y=y, M_valid=0)
        torch.cuda.synchronize()
        assert torch.all(y.view(torch.int16) == 0), (M, N, K)
    note("block recipe fwd with M_valid = 0")
    M, N, K = 256, 384, 512
    qa = np.full((M, K), 0x7F, np.uint8)
    qb, _ = _codes((N, K), 63, std=1.0)
    sa = torch.ones((M, K // 128), dtype=torch.float32, device="cuda")
    sw = torch.ones((N // 128, K // 128), dtype=torch.float32, device="cuda")
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    lib.fp8_linear_fwd(_dev(qa), _dev(qb), sa, sw, y=y, M_valid=0, gran=lib.FP8_BLOCK_1x128)
    torch.cuda.synchronize()
    assert torch.all(y.view(torch.int16) == 0)


def test_full_size_headline_sampled(lib):
    """The MLP block's gate/up forward at M=8192, K=4096, N=14336 (the launch configuration the
    benchmark times): 2048 sampled outputs computed one by one by the oracle."""
    M, K, N = 8192, 4096, 14336
    x = workloads.bf16_tensor("student_t", (M, K), 3, workloads.T_X, 0, nu=3)
    w = workloads.bf16_tensor("normal", (N, K), 3, workloads.T_WGATE, 0, std=0.02)
    sx, sxi = scale_from_amax(o_amax(x))
    sw, swi = scale_from_amax(o_amax(w))
    note("full size: quantize x, w on the GPU")
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    wd = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
    qx, _, _, _, _ = lib.fp8_quantize_amax(xd, scale_inv=dev_f32(sxi), want_q_t=False)
    qw, _, _, _, _ = lib.fp8_quantize_amax(wd, scale_inv=dev_f32(swi), want_q_t=False)
    note("full size: fp8_linear_fwd 8192x14336x4096")
    y = lib.fp8_linear_fwd(qx, qw, dev_f32(sx), dev_f32(sw))
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    ms = rng.integers(0, M, 2048)
    ns = rng.integers(0, N, 2048)
    yh = host_bf16_f64(y)
    from oracle.quantize import quantize_values
    for m, n in zip(ms, ns):
        a = quantize_values(x[m:m + 1], sxi)
        bq = quantize_values(w[n:n + 1], swi)
        D = gemm.scaled_gemm(a, bq, sx, sw)[0, 0]
        bound = gemm.error_bound(a, bq, sx, sb=sw)[0, 0]
        assert abs(yh[m, n] - D) <= bound, (m, n, yh[m, n], D, bound)


# Shapes the 16x16x128 kernel takes (output of at least 2048 x 2048, K of at least 512),
# with ragged M and N (partial 256-row / 256-column tiles), padded rows (M_valid < M), and
# K that is not a multiple of its 256-byte stage pair (a tail chunk and a padding stage).
@pytest.mark.parametrize("M,N,K,mv", [(2064, 2320, 512, 2064), (2320, 2064, 768, 2301),
                                      (4096, 1040, 1024, 4000),
                                      # K tails: 528 = 4 stages + 16 bytes, 1040 = 8 + 16
                                      (2304, 2048, 528, 2300), (2048, 2176, 1040, 2048)])
def test_wide_kernel_ragged(lib, M, N, K, mv):
    qa, sa = _codes((M, K), 31 + M, "student_t", nu=3)
    qb, sb = _codes((N, K), 32 + N, "normal", std=0.02)
    note(f"fp8_linear_fwd M={M} N={N} K={K} M_valid={mv}")
    y = lib.fp8_linear_fwd(_dev(qa), _dev(qb), dev_f32(sa), dev_f32(sb), M_valid=mv)
    torch.cuda.synchronize()
    yh = host_bf16_f64(y)
    assert np.all(yh[mv:] == 0)
    worst = _within_both(yh[:mv], qa[:mv], qb, sa, sb, f"fwd {M}x{N}x{K}")
    assert worst < 0.25


# Outputs of at least 2048 x 2048 with a contraction shorter than 512 take the 32x32x64
# kernel with 256x256 tiles: four-stage ring (K/64 a multiple of 4), two-stage ring (even),
# and one tile per workgroup (odd K/64); ragged rows and padded rows included.
@pytest.mark.parametrize("M,N,K,mv", [(2048, 2048, 256, 2048), (2064, 2048, 384, 2000),
                                      (2048, 2304, 128, 2048), (2064, 2048, 144, 2050)])
def test_wide_output_short_contraction(lib, M, N, K, mv):
    test_wide_kernel_ragged(lib, M, N, K, mv)


@pytest.mark.parametrize("M,N,K,mv", [
    # more than one round of 256x256 tiles: 224-row tiles (ragged last tile row), then
    # 224-column tiles (ragged last tile column), with a ragged contraction on each
    (4352, 4096, 512, 4352), (4352, 4096, 528, 4301), (4096, 7152, 512, 1200),
    (4096, 7152, 784, 900)])
def test_narrow_tile_kernels_ragged(lib, M, N, K, mv):
    """Output grids that the 16x16x128 kernel covers with 224x256 or 256x224 tiles (fewer
    idle workgroups in the last round): every computed row checked against the oracle,
    padded rows zero."""
    test_wide_kernel_ragged(lib, M, N, K, mv)


@pytest.mark.parametrize("M,N,K,what", [(8192, 4096, 14336, "dgrad"), (14336, 4096, 8192, "wgrad"),
                                        (4096, 14336, 8192, "wgrad of the down projection")])
def test_full_size_backward_shapes_sampled(lib, M, N, K, what):
    """The MLP block's dgrad (contraction over 14336) and wgrad (contraction over the 8192
    tokens) launch shapes: operands quantized on the GPU (bit-exact with the oracle, see
    test_gpu_quantize), 1024 sampled outputs computed one by one by the oracle from the
    sampled rows."""
    from oracle.quantize import quantize_values
    a = workloads.bf16_tensor("normal", (M, K), 3, 41 + K, 0, std=1e-3)
    b = workloads.bf16_tensor("student_t", (N, K), 3, 42 + K, 0, nu=3)
    sa, sai = scale_from_amax(o_amax(a))
    sb, sbi = scale_from_amax(o_amax(b))
    note(f"full size {what}: quantize operands on the GPU")
    ad = torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    bd = torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
    qa, _, _, _, _ = lib.fp8_quantize_amax(ad, scale_inv=dev_f32(sai), want_q_t=False)
    qb, _, _, _, _ = lib.fp8_quantize_amax(bd, scale_inv=dev_f32(sbi), want_q_t=False)
    note(f"full size {what}: fp8 GEMM {M}x{N}x{K}")
    y = lib.fp8_linear_fwd(qa, qb, dev_f32(sa), dev_f32(sb))
    torch.cuda.synchronize()
    yh = host_bf16_f64(y)
    rng = np.random.default_rng(K)
    for m, n in zip(rng.integers(0, M, 1024), rng.integers(0, N, 1024)):
        ra = quantize_values(a[m:m + 1], sai)
        rb = quantize_values(b[n:n + 1], sbi)
        D = gemm.scaled_gemm(ra, rb, sa, sb)[0, 0]
        bound = gemm.error_bound(ra, rb, sa, sb)[0, 0]
        assert abs(yh[m, n] - D) <= bound, (what, m, n, yh[m, n], D, bound)


@pytest.mark.parametrize("M,N,K,mv", [(2304, 2048, 512, 2200), (2304, 2048, 512, 0),
                                      (272, 256, 128, 200)])
def test_padded_rows_are_zero_even_if_nan(lib, M, N, K, mv):
    """Rows at or past M_valid are written as zeros whatever their codes hold: here NaN
    codes (0x7F), whose sums are NaN (both the 16x16x128 kernel's shape and a small one),
    into an output that held NaN before the call."""
    qa, sa = _codes((M, K), 51 + M, "normal", std=1.0)
    qb, sb = _codes((N, K), 52 + N, "normal", std=1.0)
    qa[mv:] = 0x7F
    note(f"fp8_linear_fwd NaN pad rows M={M} N={N} K={K} M_valid={mv}")
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    lib.fp8_linear_fwd(_dev(qa), _dev(qb), dev_f32(sa), dev_f32(sb), y=y, M_valid=mv)
    torch.cuda.synchronize()
    yh = host_bf16_f64(y)
    assert np.all(yh[mv:] == 0), "padded rows"
    D, b = _exact_and_bound(qa[:mv], qb, sa, sb)
    assert_within(yh[:mv], D, b, "valid rows")
