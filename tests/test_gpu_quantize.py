"""GPU parity: tensorwise quantize + amax + transposed copy, bit-exact with the oracle."""
import numpy as np
import pytest

import workloads
from oracle import e4m3
from oracle.quantize import amax as o_amax
from oracle.quantize import quantize_tensorwise, quantize_values
from oracle.scaling import scale_from_amax
from tests.gpu_util import (assert_same_bytes, dev_bf16, dev_f32, f32_bits, host_u8, note)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_fp8_linear_amd as m
    m.load()
    return m


def _gpu_quantize(m, x_bits, scale_inv, rows_valid=None):
    x = dev_bf16(x_bits)
    si = dev_f32(scale_inv)
    q, qt, a, _, _ = m.fp8_quantize_amax(x, rows_valid=rows_valid, scale_inv=si)
    torch.cuda.synchronize()
    return host_u8(q), host_u8(qt), np.float32(a.item())


def _check(m, x_bits, scale_inv, rows_valid=None, what=""):
    q, qt, a = _gpu_quantize(m, x_bits, scale_inv, rows_valid)
    oq, oqt, oa = quantize_tensorwise(x_bits, np.float32(scale_inv), rows_valid)
    assert_same_bytes(q, oq, f"q {what}")
    assert_same_bytes(qt, oqt, f"q_t {what}")
    if np.isnan(oa):
        assert np.isnan(a), what
    else:
        assert f32_bits(a) == f32_bits(oa), (what, a, oa)


ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
FINITE_BF16 = np.where((ALL_BF16 & 0x7F80) == 0x7F80, np.uint16(0), ALL_BF16)

EXHAUSTIVE_SCALES = [1.0, 448.0, 0.5, 2.0 ** -20, 2.0 ** 20, 448.0 / 3.0, 448.0 / 0.11,
                     1.0 / 448.0, 448.0 / 1e-12, 448.0 / 301.7, 3.14159, 1e-30]


@pytest.mark.parametrize("scale_inv", EXHAUSTIVE_SCALES)
def test_every_bf16_pattern(lib, scale_inv):
    """All 65 536 bf16 patterns (inf/NaN included) times a scale: every code bit-exact."""
    note(f"quantize all bf16 patterns, scale_inv={scale_inv}")
    q, qt, a = _gpu_quantize(lib, ALL_BF16, scale_inv)
    oq = quantize_values(ALL_BF16, np.float32(scale_inv))
    assert_same_bytes(q, oq, f"all-bf16 q scale_inv={scale_inv}")
    assert_same_bytes(qt, np.ascontiguousarray(oq.T), "all-bf16 q_t")
    assert np.isnan(a)                                  # NaN patterns are present
    note("finite patterns only: amax")
    _, _, a2 = _gpu_quantize(lib, FINITE_BF16, scale_inv)
    assert f32_bits(a2) == f32_bits(o_amax(FINITE_BF16))


def test_random_scales_normal_data(lib):
    rng = np.random.default_rng(17)
    x = workloads.bf16_tensor("normal", (256, 512), 90, 1, 0, std=1.0)
    for si in (448.0 / rng.lognormal(0, 3, 8)).astype(np.float32):
        note(f"quantize N(0,1) [256,512] scale_inv={si}")
        _check(lib, x, si, what=f"scale_inv={si}")


@pytest.mark.parametrize("rows,cols,rv", [(16, 16, 16), (144, 272, 144), (272, 528, 200),
                                           (400, 48, 1), (128, 256, 0), (1040, 784, 1033)])
def test_ragged_shapes_and_padding_rows(lib, rows, cols, rv):
    """Tiles are 128x256: these shapes leave ragged row and column tails; rows >= rv hold NaN
    sentinels that must be neither read into amax nor quantized."""
    x = workloads.bf16_tensor("student_t", (rows, cols), 91, rows, cols, nu=3)
    x[rv:] = 0x7FC0
    a = o_amax(x, rv)
    _, si = scale_from_amax(a)
    note(f"quantize ragged {rows}x{cols} rows_valid={rv}")
    _check(lib, x, si, rows_valid=rv, what=f"{rows}x{cols} rv={rv}")


def test_empty(lib):
    note("quantize empty input")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    amax = torch.full((1,), 5.0, device="cuda")
    lib.fp8_quantize_amax(x, scale_inv=dev_f32(1.0), amax=amax)
    torch.cuda.synchronize()
    assert amax.item() == 0.0


def test_amax_only_and_q_only(lib):
    x = workloads.bf16_tensor("normal", (128, 256), 92, 1, 0, std=2.0)
    note("quantize: amax only")
    _, _, a, _, _ = lib.fp8_quantize_amax(dev_bf16(x), want_q=False, want_q_t=False)
    torch.cuda.synchronize()
    assert f32_bits(a.item()) == f32_bits(o_amax(x))
    note("quantize: q only, no amax")
    q, qt, a, _, _ = lib.fp8_quantize_amax(dev_bf16(x), scale_inv=dev_f32(7.0), want_q_t=False,
                                           want_amax=False)
    torch.cuda.synchronize()
    assert qt is None and a is None
    assert_same_bytes(host_u8(q), quantize_values(x, np.float32(7.0)), "q only")


def test_amax_accumulate_and_clear(lib):
    """FP8_AMAX_ACCUMULATE folds max|x| into the amax buffer's value; FP8_SCALE_CLEAR_AMAX
    leaves +0 in it after the update that reads it (FROM_AMAX and RECORD)."""
    x = workloads.bf16_tensor("student_t", (272, 528), 93, 2, 0, nu=3)
    oa = o_amax(x)
    si = np.float32(448.0) / oa
    for prior in (np.float32(0.0), np.float32(oa * 4), np.float32(oa / 4)):
        note(f"quantize with amax accumulate, prior {prior}")
        a = dev_f32(prior)
        q, qt, a2, _, _ = lib.fp8_quantize_amax(dev_bf16(x), scale_inv=dev_f32(si), amax=a,
                                                amax_accumulate=True)
        torch.cuda.synchronize()
        assert a2 is a
        assert f32_bits(a.item()) == f32_bits(max(prior, oa)), (prior, a.item(), oa)
        oq, oqt, _ = quantize_tensorwise(x, si)
        assert_same_bytes(host_u8(q), oq, "q with accumulate")
        assert_same_bytes(host_u8(qt), oqt, "q_t with accumulate")
    note("quantize with amax accumulate, no valid rows")
    a = dev_f32(3.0)
    lib.fp8_quantize_amax(dev_bf16(x), rows_valid=0, scale_inv=dev_f32(si), amax=a,
                          amax_accumulate=True)
    torch.cuda.synchronize()
    assert a.item() == 3.0
    note("scale update FROM_AMAX with clear")
    a = dev_f32(oa)
    s_ = torch.empty(1, device="cuda")
    si_ = torch.empty(1, device="cuda")
    lib.fp8_scale_update(lib.FP8_SCALE_FROM_AMAX, amax=a, scale=s_, scale_inv=si_, clear_amax=True)
    torch.cuda.synchronize()
    os_, osi = scale_from_amax(oa)
    assert f32_bits(s_.item()) == f32_bits(os_) and f32_bits(si_.item()) == f32_bits(osi)
    assert f32_bits(a.item()) == 0
    note("scale update RECORD with clear")
    a = dev_f32(oa)
    hist = torch.ones(16, device="cuda")
    lib.fp8_scale_update(lib.FP8_SCALE_RECORD, amax=a, hist=hist, pos=5, clear_amax=True)
    torch.cuda.synchronize()
    h = hist.cpu().numpy()
    assert f32_bits(h[5]) == f32_bits(oa) and np.all(np.delete(h, 5) == 1.0)
    assert f32_bits(a.item()) == 0


def test_current_scaling_config1(lib):
    """Config 1's forward quantize: amax pass, scale, then the cast (all on the device)."""
    d = workloads.linear_inputs(1)
    for name in ("x", "w"):
        xb = d[name]
        x = dev_bf16(xb)
        note(f"current scaling config 1: {name}")
        _, _, a, _, _ = lib.fp8_quantize_amax(x, want_q=False, want_q_t=False)
        s = torch.empty(1, device="cuda")
        si = torch.empty(1, device="cuda")
        lib.fp8_scale_update(lib.FP8_SCALE_FROM_AMAX, amax=a, scale=s, scale_inv=si)
        q, qt, a2, _, _ = lib.fp8_quantize_amax(x, scale_inv=si)
        torch.cuda.synchronize()
        oa = o_amax(xb)
        os_, osi = scale_from_amax(oa)
        assert f32_bits(a.item()) == f32_bits(oa) == f32_bits(a2.item())
        assert f32_bits(s.item()) == f32_bits(os_) and f32_bits(si.item()) == f32_bits(osi)
        oq, oqt, _ = quantize_tensorwise(xb, osi)
        assert_same_bytes(host_u8(q), oq, f"config1 {name} q")
        assert_same_bytes(host_u8(qt), oqt, f"config1 {name} q_t")
        assert (host_u8(q) & 0x7F).max() == 0x7E


def test_full_size_headline_activation(lib):
    """x [8192, 4096] Student-t(3) at the MLP block's size: amax exact over the whole tensor,
    codes bit-exact on sampled rows and columns (the oracle computes those one by one)."""
    x = workloads.bf16_tensor("student_t", (8192, 4096), 3, workloads.T_X, 0, nu=3)
    oa = o_amax(x)
    _, si = scale_from_amax(np.float32(oa / 8))          # a stale scale: both tails saturate
    note("quantize full size [8192,4096] Student-t")
    q, qt, a = _gpu_quantize(lib, x, si)
    assert f32_bits(a) == f32_bits(oa)
    rng = np.random.default_rng(5)
    rows = rng.choice(8192, 24, replace=False)
    cols = rng.choice(4096, 24, replace=False)
    for r in rows:
        assert_same_bytes(q[r], quantize_values(x[r], si), f"row {r}")
    for c in cols:
        assert_same_bytes(qt[c], quantize_values(x[:, c], si), f"q_t row {c}")
    assert (q == 0x7E).any() and (q == 0xFE).any()


def test_deterministic(lib):
    x = dev_bf16(workloads.bf16_tensor("student_t", (512, 1024), 93, 1, 0, nu=3))
    si = dev_f32(3.0)
    outs = []
    for i in range(3):
        note(f"determinism run {i}")
        q, qt, a, _, _ = lib.fp8_quantize_amax(x, scale_inv=si)
        torch.cuda.synchronize()
        outs.append((host_u8(q), host_u8(qt), a.item()))
    for o in outs[1:]:
        assert np.array_equal(o[0], outs[0][0]) and np.array_equal(o[1], outs[0][1])
        assert o[2] == outs[0][2]


def test_error_status(lib):
    x = torch.zeros((20, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.Fp8Error, match="multiples of 16"):
        lib.fp8_quantize_amax(x, scale_inv=dev_f32(1.0))
