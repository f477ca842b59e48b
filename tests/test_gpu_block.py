"""GPU parity for the block-scaled recipe: 1x128 / 128x128 tile quantize bit-exact (codes, tile
amaxes, tile scales, and the transposed copy re-quantized along tokens), and the per-block
scaled GEMMs within the tolerance."""
import numpy as np
import pytest

import workloads
from oracle import block
from tests.gpu_util import (assert_same_bytes, assert_within, dev_bf16, host_bf16_f64, host_u8,
                            note)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_fp8_linear_amd as m
    m.load()
    return m


def _bits32(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _f32_equal(got, want, what):
    assert got.shape == want.shape, what
    g, w = _bits32(got), _bits32(want)
    bad = np.flatnonzero(g.ravel() != w.ravel())
    assert bad.size == 0, f"{what}: {bad.size} differ, first {got.ravel()[bad[0]]} vs {want.ravel()[bad[0]]}"


@pytest.mark.parametrize("rows,cols,rv", [(128, 128, 128), (384, 256, 300), (256, 640, 1)])
def test_quantize_1x128(lib, rows, cols, rv):
    x = workloads.bf16_tensor("outlier_normal", (rows, cols), 5, rows + cols, 0, rate=0.01, mult=100.0)
    x[rv:] = 0x7FC0
    note(f"block 1x128 quantize {rows}x{cols} rv={rv}")
    q, qt, a, s, st = lib.fp8_quantize_amax(dev_bf16(x), rows_valid=rv, gran=lib.FP8_BLOCK_1x128)
    torch.cuda.synchronize()
    oq, oqt, oa, os_, ost = block.quantize_1x128(x, rv)
    assert_same_bytes(host_u8(q), oq, "q")
    assert_same_bytes(host_u8(qt), oqt, "q_t")
    _f32_equal(a.cpu().numpy(), oa, "tile amax")
    _f32_equal(s.cpu().numpy(), os_, "row-tile scales")
    _f32_equal(st.cpu().numpy(), ost, "column-tile scales")


@pytest.mark.parametrize("rows,cols", [(128, 128), (384, 256)])
def test_quantize_128x128(lib, rows, cols):
    w = workloads.bf16_tensor("outlier_normal", (rows, cols), 5, 7 + rows, 0, rate=0.01, mult=100.0)
    note(f"block 128x128 quantize {rows}x{cols}")
    q, qt, a, s, st = lib.fp8_quantize_amax(dev_bf16(w), gran=lib.FP8_BLOCK_128x128)
    torch.cuda.synchronize()
    oq, oqt, oa, os_, ost = block.quantize_128x128(w)
    assert_same_bytes(host_u8(q), oq, "q")
    assert_same_bytes(host_u8(qt), oqt, "q_t")
    _f32_equal(a.cpu().numpy(), oa, "tile amax")
    _f32_equal(s.cpu().numpy(), os_, "scales")
    _f32_equal(st.cpu().numpy(), ost, "transposed scales")


@pytest.mark.parametrize("M,K,N,rv", [(256, 256, 384, 256), (384, 512, 256, 300)])
def test_block_linear_step(lib, M, K, N, rv):
    d = workloads.linear_inputs(5, 0, M=M, K=K, N=N)
    x, w, g = d["x"], d["w"], d["g"]
    note(f"block recipe step M={M} K={K} N={N}")
    B = lib.FP8_BLOCK_1x128
    qx, qx_t, _, sx, sx_t = lib.fp8_quantize_amax(dev_bf16(x), rows_valid=rv, gran=B)
    qw, qw_t, _, sw, sw_t = lib.fp8_quantize_amax(dev_bf16(w), gran=lib.FP8_BLOCK_128x128)
    qg, qg_t, _, sg, sg_t = lib.fp8_quantize_amax(dev_bf16(g), rows_valid=rv, gran=B)
    y = lib.fp8_linear_fwd(qx, qw, sx, sw, M_valid=rv, gran=B)
    dx = lib.fp8_linear_dgrad(qg, qw_t, sg, sw_t, M_valid=rv, gran=B)
    dw = lib.fp8_linear_wgrad(qg_t, qx_t, sg_t, sx_t, gran=B)
    torch.cuda.synchronize()
    r = __import__("oracle.linear", fromlist=["x"]).block_linear_step(x, w, g, rv)
    assert_same_bytes(host_u8(qx_t), r["qx_t"], "qx_t")
    assert_same_bytes(host_u8(qg_t), r["qg_t"], "qg_t")
    yb = block.block_error_bound(r["qx"], r["qw"], r["sx"], r["sw"], 128)
    assert_within(host_bf16_f64(y), r["y"], yb, "block fwd")
    db = block.block_error_bound(r["qg"], r["qw_t"], r["sg"], r["sw_t"], 128)
    assert_within(host_bf16_f64(dx), r["dx"], db, "block dgrad")
    wb = block.block_error_bound(r["qg_t"], r["qx_t"], r["sg_t"], r["sx_t"], 1)
    assert_within(host_bf16_f64(dw), r["dw"], wb, "block wgrad")


@pytest.mark.parametrize("M,K,N,rv", [(2176, 768, 1152, 2176), (1408, 1024, 2304, 1350),
                                      (1536, 768, 1280, 1500),
                                      # odd 128-block counts: 640 -> 5, 1152 -> 9 (padding stage)
                                      (1280, 640, 1152, 1280)])
def test_block_linear_step_wide_kernel(lib, M, K, N, rv):
    """Shapes the 16x16x128 block kernel takes (contraction of at least 512): rows ragged
    against its 256-row tiles, padded token rows, odd counts of 128-wide blocks, all three
    GEMMs."""
    test_block_linear_step(lib, M, K, N, rv)


@pytest.mark.parametrize("M,K,N,rv", [(4224, 640, 4096, 4200), (4224, 4096, 640, 4200),
                                      (4224, 512, 4096, 4224), (4224, 4096, 1536, 4100),
                                      (4224, 768, 4096, 4210)])
def test_block_wide_tiles(lib, M, K, N, rv):
    """Outputs of at least 256 tiles of 256x256 take the 256x256-tile kernel (one weight scale
    per 128x128 block: forward, with y [M, N], and input gradient, with dx [M, K]): rows ragged
    against the tiles, padded token rows, an odd count of 128-wide blocks (5) in the
    contraction, an even count not divisible by 4 (6: per-stage scale loads, no padding
    stage), and counts divisible by 4 (4 and 12), whose scales load 4 blocks at a time
    into two alternating regions (one or three groups per tile, so the region of a tile's
    first group alternates between tiles). Every output against both bounds (the tolerance
    and float32 accumulation)."""
    test_block_linear_step(lib, M, K, N, rv)
    d = workloads.linear_inputs(5, 0, M=M, K=K, N=N)
    x, w, g = d["x"], d["w"], d["g"]
    B = lib.FP8_BLOCK_1x128
    qx, _, _, sx, _ = lib.fp8_quantize_amax(dev_bf16(x), rows_valid=rv, gran=B)
    qw, qw_t, _, sw, sw_t = lib.fp8_quantize_amax(dev_bf16(w), gran=lib.FP8_BLOCK_128x128)
    qg, _, _, sg, _ = lib.fp8_quantize_amax(dev_bf16(g), rows_valid=rv, gran=B)
    wide = [("fwd", lib.fp8_linear_fwd(qx, qw, sx, sw, M_valid=rv, gran=B), qx, qw, sx, sw)] \
        if N >= 4096 else \
        [("dgrad", lib.fp8_linear_dgrad(qg, qw_t, sg, sw_t, M_valid=rv, gran=B), qg, qw_t, sg, sw_t)]
    torch.cuda.synchronize()
    for what, out, qa, qb, sa, sb in wide:
        note(f"block wide tiles: {what} {M}x{K}x{N}, tight bound")
        got = host_bf16_f64(out)
        assert np.all(got[rv:] == 0), what
        qah, sah = host_u8(qa)[:rv], sa.cpu().numpy().astype(np.float64)[:rv]
        D, tight = block.block_fp32_bound(qah, host_u8(qb), sah, sb.cpu().numpy().astype(np.float64), 128)
        assert_within(got[:rv], D, tight, f"block {what} (float32 accumulation)")


@pytest.mark.parametrize("M,K,N,rv", [(512, 4096, 4096, 500), (1536, 4096, 4352, 1536)])
def test_block_wide_tiles_wgrad(lib, M, K, N, rv):
    """Weight gradients dW [N, K] of at least 256 tiles of 256x256 take the 256x256-tile
    kernel with one scale per B row (both operands carry per-row scales over 128-token
    blocks), when the token count is a multiple of 512: 4 and 12 token blocks (one and three
    scale groups per tile), padded tokens, ragged tiles. dW against both bounds."""
    test_block_linear_step(lib, M, K, N, rv)
    d = workloads.linear_inputs(5, 0, M=M, K=K, N=N)
    B = lib.FP8_BLOCK_1x128
    _, qx_t, _, _, sx_t = lib.fp8_quantize_amax(dev_bf16(d["x"]), rows_valid=rv, gran=B)
    _, qg_t, _, _, sg_t = lib.fp8_quantize_amax(dev_bf16(d["g"]), rows_valid=rv, gran=B)
    dw = lib.fp8_linear_wgrad(qg_t, qx_t, sg_t, sx_t, gran=B)
    torch.cuda.synchronize()
    note(f"block wide tiles: wgrad {N}x{K} over {M} tokens, tight bound")
    D, tight = block.block_fp32_bound(host_u8(qg_t), host_u8(qx_t),
                                      sg_t.cpu().numpy().astype(np.float64),
                                      sx_t.cpu().numpy().astype(np.float64), 1)
    assert_within(host_bf16_f64(dw), D, tight, "block wgrad (float32 accumulation)")


def test_block_full_size_sampled(lib):
    """The block recipe at its benchmark size (M=16384, K=N=8192, outliers x100 at 1%):
    tile grids bit-exact on sampled tiles, GEMM outputs on sampled elements."""
    M, K, N = 16384, 8192, 8192
    d = workloads.linear_inputs(5, 0)
    x, w, g = d["x"], d["w"], d["g"]
    assert x.shape == (M, K) and w.shape == (N, K) and g.shape == (M, N)
    B = lib.FP8_BLOCK_1x128
    note("block full size: quantize x, w, g")
    qx, qx_t, _, sx, sx_t = lib.fp8_quantize_amax(dev_bf16(x), gran=B)
    qw, qw_t, _, sw, sw_t = lib.fp8_quantize_amax(dev_bf16(w), gran=lib.FP8_BLOCK_128x128)
    qg, qg_t, _, sg, sg_t = lib.fp8_quantize_amax(dev_bf16(g), gran=B)
    note("block full size: fwd, dgrad, wgrad")
    y = lib.fp8_linear_fwd(qx, qw, sx, sw, gran=B)
    dx = lib.fp8_linear_dgrad(qg, qw_t, sg, sw_t, gran=B)
    dw = lib.fp8_linear_wgrad(qg_t, qx_t, sg_t, sx_t, gran=B)
    torch.cuda.synchronize()
    yh, dxh, dwh = host_bf16_f64(y), host_bf16_f64(dx), host_bf16_f64(dw)
    sxh, swh, sgh = sx.cpu().numpy(), sw.cpu().numpy(), sg.cpu().numpy()
    sx_th, sg_th = sx_t.cpu().numpy(), sg_t.cpu().numpy()
    qxh, qwh, qgh = host_u8(qx), host_u8(qw), host_u8(qg)
    rng = np.random.default_rng(12)
    # tile grids: rows of x (1x128 tiles), one 128x128 block row of W, columns of x (the
    # transposed copy's tiles along tokens); the oracle quantizes the 128-row / 128-column
    # slab that holds each sample
    for r in rng.choice(M, 3, replace=False):
        r0 = int(r) - int(r) % 128
        oq, _, _, os_, _ = block.quantize_1x128(np.ascontiguousarray(x[r0:r0 + 128]))
        assert_same_bytes(qxh[r], oq[r % 128], f"qx row {r}")
        _f32_equal(sxh[r], os_[r % 128], f"sx row {r}")
    wq, _, _, wsc, _ = block.quantize_128x128(np.ascontiguousarray(w[:128]))
    assert_same_bytes(qwh[:128], wq, "qw block row 0")
    _f32_equal(swh[:1], wsc, "sw block row 0")
    qx_th = host_u8(qx_t)
    for c in rng.choice(K, 2, replace=False):
        c0 = int(c) - int(c) % 128
        _, oqt, _, _, ost = block.quantize_1x128(np.ascontiguousarray(x[:, c0:c0 + 128]))
        assert_same_bytes(qx_th[c], oqt[c % 128], f"qx_t row {c}")
        _f32_equal(sx_th[c], ost[c % 128], f"sx_t row {c}")
    # GEMM samples: exact per-block sums from the GPU's own codes and scales (checked above)
    for _ in range(24):
        m, n, k = int(rng.integers(0, M)), int(rng.integers(0, N)), int(rng.integers(0, K))
        ex = block.block_scaled_gemm(qxh[m:m + 1], qwh[n:n + 1], sxh[m:m + 1],
                                     swh[n // 128:n // 128 + 1], 1)
        bd = block.block_error_bound(qxh[m:m + 1], qwh[n:n + 1], sxh[m:m + 1],
                                     swh[n // 128:n // 128 + 1], 1)
        assert abs(yh[m, n] - ex[0, 0]) <= bd[0, 0], ("y", m, n)
    qw_th = host_u8(qw_t)
    sw_th = sw_t.cpu().numpy()
    for _ in range(12):
        m, k = int(rng.integers(0, M)), int(rng.integers(0, K))
        ex = block.block_scaled_gemm(qgh[m:m + 1], qw_th[k:k + 1], sgh[m:m + 1],
                                     sw_th[k // 128:k // 128 + 1], 1)
        bd = block.block_error_bound(qgh[m:m + 1], qw_th[k:k + 1], sgh[m:m + 1],
                                     sw_th[k // 128:k // 128 + 1], 1)
        assert abs(dxh[m, k] - ex[0, 0]) <= bd[0, 0], ("dx", m, k)
    qg_th = host_u8(qg_t)
    for _ in range(12):
        n, k = int(rng.integers(0, N)), int(rng.integers(0, K))
        ex = block.block_scaled_gemm(qg_th[n:n + 1], qx_th[k:k + 1], sg_th[n:n + 1],
                                     sx_th[k:k + 1], 1)
        bd = block.block_error_bound(qg_th[n:n + 1], qx_th[k:k + 1], sg_th[n:n + 1],
                                     sx_th[k:k + 1], 1)
        assert abs(dwh[n, k] - ex[0, 0]) <= bd[0, 0], ("dw", n, k)
