"""GPU parity at full size: whole tensors at M = K = N = 4096, and 1024 x 1024 output subsets
of every GEMM launch shape of the MLP block and of the block recipe.

Every GEMM output is judged twice against the exact float64 oracle:

* the tolerance of record, ``1e-2 * ||row(A)|| * ||col(B)||`` of the dequantized operands
  (``oracle.gemm.error_bound``);
* the tight float32-accumulation bound (``oracle.gemm.fp32_bound``,
  ``oracle.block.block_fp32_bound``), which also sees a single 128-wide block of a long
  contraction dropped or counted twice, where the norm tolerance cannot.

The GEMMs read the GPU's own codes and scales; every code (and scale) they read is first
checked byte for byte against the oracle's quantize of the same bf16 inputs.

Config 2 runs the 32 steps of delayed scaling once (a module fixture): the scale and ring
trajectory is compared at every step, and every byte of Qx, Qx^T, Qw, Qw^T, Qg, Qg^T and
every output of y, dx and dW at steps 1 (scales 1.0), 16 (the first ring refresh) and 32
(the first refresh over a full window of real amaxes).
"""
import numpy as np
import pytest

import workloads
from oracle import block, gemm
from oracle.linear import DelayedLinear
from oracle.quantize import amax as o_amax
from oracle.quantize import quantize_tensorwise, quantize_values
from oracle.scaling import scale_from_amax
from tests.gpu_util import (assert_same_bytes, assert_within, dev_bf16, dev_f32, f32_bits,
                            host_bf16_bits, host_bf16_f64, host_u8, note)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

KEEP_STEPS = (1, 16, 32)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_fp8_linear_amd as m
    m.load()
    return m


def _bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _judge(what, got, qa, qb, sa, sb, a_fmt="e4m3"):
    """Both tolerances on one output block; returns the worst ratios (norm, tight)."""
    D, tight = gemm.fp32_bound(qa, qb, sa, sb, a_fmt)
    w_norm = assert_within(got, D, gemm.error_bound(qa, qb, sa, sb, a_fmt=a_fmt),
                           f"{what} (norm tolerance)")
    w_tight = assert_within(got, D, tight, f"{what} (float32-accumulation bound)")
    note(f"{what}: worst err/bound {w_norm:.3g} (norm), {w_tight:.3g} (float32 accumulation)")
    return w_norm, w_tight


# ---------------------------------------------------------------- config 2, whole tensors
@pytest.fixture(scope="module")
def config2(lib):
    c = workloads.CONFIGS[2]
    M, K, N = c["M"], c["K"], c["N"]
    lin = lib.DelayedScalingLinear("cuda", keep_amax=True)
    ref = DelayedLinear()
    u8 = dict(dtype=torch.uint8, device="cuda")
    bufs = dict(qw=torch.empty((N, K), **u8), qw_t=torch.empty((K, N), **u8),
                qx=torch.empty((M, K), **u8), qx_t=torch.empty((K, M), **u8),
                qg=torch.empty((M, N), **u8), qg_t=torch.empty((N, M), **u8))
    w = workloads.linear_inputs(2, 0)["w"]
    run = dict(trajectory=[], kept={}, code_mismatch=[])
    rng = np.random.default_rng(2)
    for t in range(1, c["steps"] + 1):
        d = workloads.linear_inputs(2, t)
        x, g = d["x"], d["g"]
        note(f"config 2 step {t}")
        lin.begin_step()
        y = lin.forward(dev_bf16(x), dev_bf16(w), bufs=bufs)
        dx, dw = lin.backward(dev_bf16(g), bufs=bufs)
        torch.cuda.synchronize()
        ref.begin_step()
        used = ref.scales_only_step(x, w, g)
        amaxes = tuple(f32_bits(a.item()) for a in (lin.amax_x, lin.amax_w, lin.amax_g))
        # every step: two sampled rows of each code tensor (whole tensors at KEEP_STEPS)
        for name, bits, si in (("qx", x, used["sx_inv"]), ("qw", w, used["sw_inv"]),
                               ("qg", g, used["sg_inv"])):
            for r in rng.choice(bits.shape[0], 2, replace=False):
                got = host_u8(bufs[name][int(r)])
                if not np.array_equal(got, quantize_values(bits[r], si)):
                    run["code_mismatch"].append((t, name, int(r)))
        if t in KEEP_STEPS:
            run["kept"][t] = dict(
                x=x, w=w, g=g, used=used,
                codes={k: host_u8(v) for k, v in bufs.items()},
                out={k: host_bf16_bits(v) for k, v in (("y", y), ("dx", dx), ("dw", dw))})
        lin.end_step()
        run["trajectory"].append((t, amaxes, lin.state(), ref.state(), used))
        w = workloads.drift(w, 2, t, c["drift"])
    return run


def test_config2_scale_trajectory(config2):
    """The amaxes and every scale and ring entry, bit-exact at each of the 32 steps (and two
    sampled rows of every code tensor at each step)."""
    assert not config2["code_mismatch"], config2["code_mismatch"][:5]
    for t, amaxes, gpu, ref, used in config2["trajectory"]:
        assert amaxes == tuple(f32_bits(used[k]) for k in ("amax_x", "amax_w", "amax_g")), t
        for k in ("w_scale", "w_scale_inv", "x_scale", "x_scale_inv", "g_scale", "g_scale_inv"):
            assert f32_bits(gpu[k]) == f32_bits(ref[k]), (t, k, gpu[k], ref[k])
        assert np.array_equal(gpu["hist"].view(np.uint32), ref["hist"].view(np.uint32)), t
        assert gpu["idx"] == ref["idx"] and gpu["step"] == ref["step"] == t


@pytest.mark.parametrize("t", KEEP_STEPS)
def test_config2_whole_tensors(config2, t):
    k = config2["kept"][t]
    u, c, o = k["used"], k["codes"], k["out"]
    note(f"config 2 step {t}: whole code tensors")
    for name, bits, si in (("x", k["x"], u["sx_inv"]), ("w", k["w"], u["sw_inv"]),
                           ("g", k["g"], u["sg_inv"])):
        q, q_t, _ = quantize_tensorwise(bits, si)
        assert_same_bytes(c[f"q{name}"], q, f"Q{name} step {t}")
        assert_same_bytes(c[f"q{name}_t"], q_t, f"Q{name}^T step {t}")
    note(f"config 2 step {t}: whole y, dx, dW")
    _judge(f"y step {t}", _bits_to_f64(o["y"]), c["qx"], c["qw"], u["sx"], u["sw"])
    _judge(f"dx step {t}", _bits_to_f64(o["dx"]), c["qg"], c["qw_t"], u["sg"], u["sw"])
    _judge(f"dW step {t}", _bits_to_f64(o["dw"]), c["qg_t"], c["qx_t"], u["sg"], u["sx"])


# ---------------------------------------------------------------- MLP launch shapes
def _pick(n, tile, rng, count=1024):
    """``count`` sorted distinct indices below n: both ends, the edges of the first and
    last tiles of ``tile`` rows (also 224-row tiles), the rest at random."""
    must = {0, 1, n - 1, n - 2, tile - 1, tile, 223, 224, n - tile, n - tile - 1, n // 2}
    idx = set(i for i in must if 0 <= i < n)
    while len(idx) < count:
        idx.update(int(v) for v in rng.choice(n, count - len(idx), replace=False))
    return np.array(sorted(idx)[:count])


def _mlp(tensor_id, kind, shape, **p):
    """One tensor of the MLP block's inputs, drawn exactly as the benchmark draws it."""
    return workloads.bf16_tensor(kind, shape, 3, tensor_id, 0, **p)


def _quantize_dev(lib, bits, q=True, q_t=False, e5m2=False):
    fmax = 57344.0 if e5m2 else 448.0
    s, si = scale_from_amax(o_amax(bits), fmax)
    qd, qtd, _, _, _ = lib.fp8_quantize_amax(dev_bf16(bits), scale_inv=dev_f32(si), want_q=q,
                                             want_q_t=q_t, e5m2=e5m2)
    return qd, qtd, s, si


M_TOK, D_MODEL, D_FF = 8192, 4096, 14336
ST = dict(nu=3)
W02 = dict(std=0.02)
G13 = dict(std=1e-3)


def test_subset_forward_gate(lib):
    """y = x W_gate^T: the 8192 x 14336 x 4096 launch (also dgrad of the down projection)."""
    x = _mlp(workloads.T_X, "student_t", (M_TOK, D_MODEL), **ST)
    w = _mlp(workloads.T_WGATE, "normal", (D_FF, D_MODEL), **W02)
    qx, _, sx, sxi = _quantize_dev(lib, x)
    qw, _, sw, swi = _quantize_dev(lib, w)
    note("subset: fp8_linear_fwd 8192x14336x4096")
    y = lib.fp8_linear_fwd(qx, qw, dev_f32(sx), dev_f32(sw))
    torch.cuda.synchronize()
    rng = np.random.default_rng(101)
    ms, ns = _pick(M_TOK, 256, rng), _pick(D_FF, 256, rng)
    qa, qb = host_u8(qx[ms]), host_u8(qw[ns])
    assert_same_bytes(qa, quantize_values(x[ms], sxi), "Qx rows")
    assert_same_bytes(qb, quantize_values(w[ns], swi), "Qw rows")
    got = host_bf16_f64(y[torch.from_numpy(ms).cuda()][:, torch.from_numpy(ns).cuda()])
    _judge("fwd 8192x14336x4096 subset", got, qa, qb, sx, sw)


@pytest.mark.parametrize("grad_format", ["e4m3", "e5m2"])
def test_subset_dgrad_gate(lib, grad_format):
    """dx = g W_gate: the 8192 x 4096 x 14336 launch (also the down projection's forward),
    with E4M3 gradients and with the hybrid format's E5M2 gradients."""
    e5 = grad_format == "e5m2"
    g = _mlp(workloads.T_GGATE, "normal", (M_TOK, D_FF), **G13)
    w = _mlp(workloads.T_WGATE, "normal", (D_FF, D_MODEL), **W02)
    qg, _, sg, sgi = _quantize_dev(lib, g, e5m2=e5)
    _, qw_t, sw, swi = _quantize_dev(lib, w, q=False, q_t=True)
    note(f"subset: fp8_linear_dgrad 8192x4096x14336 ({grad_format} gradients)")
    dx = lib.fp8_linear_dgrad(qg, qw_t, dev_f32(sg), dev_f32(sw), a_e5m2=e5)
    torch.cuda.synchronize()
    rng = np.random.default_rng(102)
    ms, ks = _pick(M_TOK, 256, rng), _pick(D_MODEL, 256, rng)
    qa, qb = host_u8(qg[ms]), host_u8(qw_t[ks])
    assert_same_bytes(qa, quantize_values(g[ms], sgi, grad_format), "Qg rows")
    assert_same_bytes(qb, quantize_values(np.ascontiguousarray(w[:, ks].T), swi), "Qw^T rows")
    got = host_bf16_f64(dx[torch.from_numpy(ms).cuda()][:, torch.from_numpy(ks).cuda()])
    _judge(f"dgrad 8192x4096x14336 subset ({grad_format})", got, qa, qb, sg, sw, grad_format)


@pytest.mark.parametrize("which", ["gate", "down"])
def test_subset_wgrad(lib, which):
    """dW = g^T x over the 8192 tokens: 14336 x 4096 x 8192 (gate and up; 224-row tiles) and
    4096 x 14336 x 8192 (down; 224-column tiles)."""
    if which == "gate":
        g = _mlp(workloads.T_GGATE, "normal", (M_TOK, D_FF), **G13)
        x = _mlp(workloads.T_X, "student_t", (M_TOK, D_MODEL), **ST)
    else:
        g = _mlp(workloads.T_GDOWN, "normal", (M_TOK, D_MODEL), **G13)
        x = _mlp(workloads.T_H, "student_t", (M_TOK, D_FF), **ST)
    _, qg_t, sg, sgi = _quantize_dev(lib, g, q=False, q_t=True)
    _, qx_t, sx, sxi = _quantize_dev(lib, x, q=False, q_t=True)
    N, K = g.shape[1], x.shape[1]
    note(f"subset: fp8_linear_wgrad {N}x{K}x{M_TOK}")
    dw = lib.fp8_linear_wgrad(qg_t, qx_t, dev_f32(sg), dev_f32(sx))
    torch.cuda.synchronize()
    rng = np.random.default_rng(103)
    ns, ks = _pick(N, 224, rng), _pick(K, 256, rng)
    qa, qb = host_u8(qg_t[ns]), host_u8(qx_t[ks])
    assert_same_bytes(qa, quantize_values(np.ascontiguousarray(g[:, ns].T), sgi), "Qg^T rows")
    assert_same_bytes(qb, quantize_values(np.ascontiguousarray(x[:, ks].T), sxi), "Qx^T rows")
    got = host_bf16_f64(dw[torch.from_numpy(ns).cuda()][:, torch.from_numpy(ks).cuda()])
    _judge(f"wgrad {N}x{K}x{M_TOK} subset", got, qa, qb, sg, sx)


# ---------------------------------------------------------------- block recipe
def test_subset_block_recipe(lib):
    """Block recipe at M = 16384, K = N = 8192 (1% outliers x100): the forward (128x128 weight
    tiles) and wgrad (1x128 tiles along the tokens on both operands) launches, on 1024 rows
    of x by 8 whole 128-row weight tiles, and 1024 x 1024 of dW."""
    M, K, N = 16384, 8192, 8192
    d = workloads.linear_inputs(5, 0)
    x, w, g = d["x"], d["w"], d["g"]
    B = lib.FP8_BLOCK_1x128
    note("block subset: quantize x, W, g at full size")
    qx, qx_t, _, sx, sx_t = lib.fp8_quantize_amax(dev_bf16(x), gran=B)
    qw, _, _, sw, _ = lib.fp8_quantize_amax(dev_bf16(w), gran=lib.FP8_BLOCK_128x128,
                                            want_q_t=False)
    _, qg_t, _, _, sg_t = lib.fp8_quantize_amax(dev_bf16(g), gran=B, want_q=False)
    note("block subset: fwd 16384x8192x8192 and wgrad 8192x8192x16384")
    y = lib.fp8_linear_fwd(qx, qw, sx, sw, gran=B)
    dw = lib.fp8_linear_wgrad(qg_t, qx_t, sg_t, sx_t, gran=B)
    torch.cuda.synchronize()
    rng = np.random.default_rng(105)
    # forward: 1024 rows of x, 8 whole weight tiles (the oracle needs a tile's 128 rows)
    ms = _pick(M, 256, rng)
    tiles = np.sort(np.concatenate([[0, N // 128 - 1], rng.choice(np.arange(1, N // 128 - 1), 6,
                                                                 replace=False)]))
    ns = (tiles[:, None] * 128 + np.arange(128)[None, :]).ravel()
    oq, _, _, os_, _ = block.quantize_1x128(np.ascontiguousarray(x[ms]))
    qa, sa = host_u8(qx[ms]), sx.cpu().numpy()[ms]
    assert_same_bytes(qa, oq, "Qx rows")
    assert np.array_equal(sa.view(np.uint32), os_.view(np.uint32)), "sx rows"
    wq, _, _, wsc, _ = block.quantize_128x128(np.ascontiguousarray(w[ns]))
    qb, sb = host_u8(qw[ns]), sw.cpu().numpy()[tiles]
    assert_same_bytes(qb, wq, "Qw tiles")
    assert np.array_equal(sb.view(np.uint32), wsc.view(np.uint32)), "sw tiles"
    got = host_bf16_f64(y[torch.from_numpy(ms).cuda()][:, torch.from_numpy(ns).cuda()])
    D, tight = block.block_fp32_bound(qa, qb, sa, sb, 128)
    wn = assert_within(got, D, block.block_error_bound(qa, qb, sa, sb, 128), "block fwd (norm)")
    wt = assert_within(got, D, tight, "block fwd (float32 accumulation)")
    note(f"block fwd subset: worst err/bound {wn:.3g} (norm), {wt:.3g} (float32 accumulation)")
    # wgrad: rows of Qg^T (columns of g) and Qx^T (columns of x), tiles along the tokens
    ns, ks = _pick(N, 256, rng), _pick(K, 256, rng)
    _, oqa, _, _, osa = block.quantize_1x128(np.ascontiguousarray(g[:, ns]))
    _, oqb, _, _, osb = block.quantize_1x128(np.ascontiguousarray(x[:, ks]))
    qa, sa = host_u8(qg_t[ns]), sg_t.cpu().numpy()[ns]
    qb, sb = host_u8(qx_t[ks]), sx_t.cpu().numpy()[ks]
    assert_same_bytes(qa, oqa, "Qg^T rows")
    assert_same_bytes(qb, oqb, "Qx^T rows")
    assert np.array_equal(sa.view(np.uint32), osa.view(np.uint32)), "sg^T rows"
    assert np.array_equal(sb.view(np.uint32), osb.view(np.uint32)), "sx^T rows"
    got = host_bf16_f64(dw[torch.from_numpy(ns).cuda()][:, torch.from_numpy(ks).cuda()])
    D, tight = block.block_fp32_bound(qa, qb, sa, sb, 1)
    wn = assert_within(got, D, block.block_error_bound(qa, qb, sa, sb, 1), "block wgrad (norm)")
    wt = assert_within(got, D, tight, "block wgrad (float32 accumulation)")
    note(f"block wgrad subset: worst err/bound {wn:.3g} (norm), {wt:.3g} (float32 accumulation)")
