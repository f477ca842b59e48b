"""GPU parity: scale bookkeeping (bit-exact float32 divisions, ring, refresh) and token padding."""
import numpy as np
import pytest

from oracle.padding import pad_rows, padded_count
from oracle.scaling import WeightScales, scale_from_amax
from tests.gpu_util import dev_f32, f32_bits, host_bf16_bits, note

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_fp8_linear_amd as m
    m.load()
    return m


def test_scale_from_amax_bit_exact(lib):
    rng = np.random.default_rng(21)
    amaxes = list(rng.lognormal(0, 6, 300).astype(np.float32))
    amaxes += [0.0, -0.0, 1e-12, 9.99e-13, 1e-30, 448.0, 0.11, 300.0, 3.3895314e38,
               float(np.float32(1e-12)), 2.0 ** -149, np.inf]
    a_dev = dev_f32(amaxes)
    s = torch.empty_like(a_dev)
    si = torch.empty_like(a_dev)
    note(f"FROM_AMAX on {len(amaxes)} values")
    for i in range(len(amaxes)):
        lib.fp8_scale_update(lib.FP8_SCALE_FROM_AMAX, amax=lib.Slot(a_dev, i),
                             scale=lib.Slot(s, i), scale_inv=lib.Slot(si, i))
    torch.cuda.synchronize()
    sh, sih = s.cpu().numpy(), si.cpu().numpy()
    for i, a in enumerate(amaxes):
        rs, rsi = scale_from_amax(np.float32(a))
        assert f32_bits(sh[i]) == f32_bits(rs), (a, sh[i], rs)
        assert f32_bits(sih[i]) == f32_bits(rsi), (a, sih[i], rsi)


def test_scale_from_nan_amax(lib):
    a = dev_f32([np.nan])
    s, si = dev_f32([1.0]), dev_f32([1.0])
    note("FROM_AMAX NaN")
    lib.fp8_scale_update(lib.FP8_SCALE_FROM_AMAX, amax=a, scale=s, scale_inv=si)
    torch.cuda.synchronize()
    assert np.isnan(s.item()) and np.isnan(si.item())


def test_record_and_refresh_ring(lib):
    """The hand-worked 'inc' schedule: a_t = t/64 recorded for 48 steps, refresh every 16."""
    hist = torch.ones(16, device="cuda")
    scale, scale_inv = dev_f32([1.0]), dev_f32([1.0])
    ref = WeightScales()
    for t in range(1, 49):
        if t % 16 == 0:
            note(f"REFRESH at step {t}")
            lib.fp8_scale_update(lib.FP8_SCALE_REFRESH, hist=hist, scale=scale, scale_inv=scale_inv)
            ref.refresh()
        torch.cuda.synchronize()
        assert f32_bits(scale.item()) == f32_bits(ref.scale), t
        assert f32_bits(scale_inv.item()) == f32_bits(ref.scale_inv), t
        a = dev_f32([t / 64])
        lib.fp8_scale_update(lib.FP8_SCALE_RECORD, amax=a, hist=hist, pos=ref.pos)
        ref.record(np.float32(t / 64))
    torch.cuda.synchronize()
    assert np.array_equal(hist.cpu().numpy(), ref.hist)


def test_refresh_skips_zero_and_nan_windows(lib):
    scale, scale_inv = dev_f32([0.5]), dev_f32([2.0])
    for window in (np.zeros(16, np.float32), np.r_[np.ones(15, np.float32), np.nan]):
        note(f"REFRESH over {window[-1]}-terminated window")
        lib.fp8_scale_update(lib.FP8_SCALE_REFRESH, hist=dev_f32(window), scale=scale,
                             scale_inv=scale_inv)
        torch.cuda.synchronize()
        assert scale.item() == 0.5 and scale_inv.item() == 2.0


@pytest.mark.parametrize("T,cols,mult", [(3858, 64, 16), (1, 16, 16), (16, 32, 16), (0, 16, 16),
                                          (67827, 128, 16), (37, 24, 8), (5, 3, 16)])
def test_pad_tokens(lib, T, cols, mult):
    rng = np.random.default_rng(T)
    x = rng.integers(0, 1 << 16, size=(T, cols), dtype=np.uint32).astype(np.uint16)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    note(f"pad_tokens T={T} cols={cols} multiple={mult}")
    xp, tp = lib.fp8_pad_tokens(xd, multiple=mult)
    torch.cuda.synchronize()
    assert tp == padded_count(T, mult)
    assert np.array_equal(host_bf16_bits(xp), pad_rows(x, mult))
    # in place: a buffer of T_pad rows with garbage (0xFFFF) in the tail
    buf = np.full((tp, cols), 0xFFFF, np.uint16)
    buf[:T] = x
    bd = torch.from_numpy(buf.view(np.int16)).cuda().view(torch.bfloat16)
    note(f"pad_tokens in place T={T}")
    lib.fp8_pad_tokens(bd, T=T, multiple=mult, x_pad=bd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(bd), pad_rows(x, mult))
