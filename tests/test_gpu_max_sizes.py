"""GPU parity at the ABI's size limits (where 32-bit offsets would overflow first).

* a GEMM output just under 2^31 bytes (32768 x 32752 bf16; the last tile column ragged);
* a GEMM operand just under 2^31 bytes with the longest contraction the ABI takes
  (16384 x 131056 codes; K = 2^17 - 16, a K tail on the 16x16x128 kernel);
* a quantize pass over 2^31 bf16 elements (32768 x 65536), whose codes and transposed codes
  lie past 2^31 bytes.
Inputs are seeded and synthetic, drawn on the device with a seeded torch generator; every
expected value is computed by the oracle from rows copied back to the host. Sampled outputs
include the first and last rows and columns.
"""
import numpy as np
import pytest

from oracle import gemm
from oracle.quantize import amax as o_amax
from oracle.quantize import quantize_values
from oracle.scaling import scale_from_amax
from tests.gpu_util import dev_f32, note

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_fp8_linear_amd as m
    m.load()
    return m


def _codes_on_device(shape, seed):
    """Finite E4M3 codes, uniformly drawn (0x7F / 0xFF, the NaN codes, mapped to 0x7E / 0xFE)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=g)
    q[(q & 0x7F) == 0x7F] -= 1
    return q


def _samples(rng, M, N, n):
    ms = np.concatenate([[0, M - 1, M - 1, 0], rng.integers(0, M, n)])
    ns = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, n)])
    return ms, ns


def _check_sampled(y, qa, qb, sa, sb, ms, ns, what):
    yd = y[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()]
    got = (yd.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16) \
        .view(np.float32).astype(np.float64)
    rows_a = {int(m): qa[int(m)].cpu().numpy()[None] for m in np.unique(ms)}
    rows_b = {int(n): qb[int(n)].cpu().numpy()[None] for n in np.unique(ns)}
    for k, (m, n) in enumerate(zip(ms, ns)):
        a, b = rows_a[int(m)], rows_b[int(n)]
        D = gemm.scaled_gemm(a, b, sa, sb)[0, 0]
        bound = gemm.error_bound(a, b, sa, sb)[0, 0]
        assert abs(got[k] - D) <= bound, (what, int(m), int(n), got[k], D, bound)


def test_gemm_output_just_under_2_31_bytes(lib):
    M, N, K = 32768, 32752, 512
    assert M * N * 2 < 2 ** 31 and M * (N + 16) * 2 >= 2 ** 31
    qa, qb = _codes_on_device((M, K), 71), _codes_on_device((N, K), 72)
    sa, sb = np.float32(1 / 256), np.float32(1 / 512)
    note(f"max-size GEMM output {M}x{N}x{K}")
    y = lib.fp8_linear_fwd(qa, qb, dev_f32(sa), dev_f32(sb))
    torch.cuda.synchronize()
    ms, ns = _samples(np.random.default_rng(1), M, N, 400)
    # the last tile column (ragged: 32752 = 127 * 256 + 240) and the last rows
    ms = np.concatenate([ms, np.full(32, M - 1), np.arange(M - 32, M)])
    ns = np.concatenate([ns, np.arange(N - 32, N), np.full(32, N - 17)])
    _check_sampled(y, qa, qb, sa, sb, ms, ns, "max output")
    del y, qa, qb
    torch.cuda.empty_cache()


def test_gemm_operand_just_under_2_31_bytes_longest_contraction(lib):
    M, N, K = 16384, 256, (1 << 17) - 16
    assert M * K < 2 ** 31 and K < gemm.EXACT_K_LIMIT
    qa, qb = _codes_on_device((M, K), 73), _codes_on_device((N, K), 74)
    sa, sb = np.float32(1 / 1024), np.float32(1 / 2048)
    note(f"max-size GEMM operand {M}x{N}x{K}")
    y = lib.fp8_linear_fwd(qa, qb, dev_f32(sa), dev_f32(sb))
    torch.cuda.synchronize()
    ms, ns = _samples(np.random.default_rng(2), M, N, 200)
    _check_sampled(y, qa, qb, sa, sb, ms, ns, "max operand")
    del y, qa, qb
    torch.cuda.empty_cache()


def test_quantize_2_31_elements(lib):
    R, C = 32768, 65536
    g = torch.Generator(device="cuda").manual_seed(75)
    x = torch.randn((R, C), device="cuda", generator=g, dtype=torch.float32).to(torch.bfloat16)
    x[R - 1, C - 1] = 37.0              # the maximum sits in the very last element
    x[0, 0] = -36.0
    amax_host = np.float32(37.0)
    _, si = scale_from_amax(amax_host)
    note(f"max-size quantize {R}x{C}")
    q, qt, a, _, _ = lib.fp8_quantize_amax(x, scale_inv=dev_f32(si))
    torch.cuda.synchronize()
    assert np.float32(a.item()) == amax_host
    rng = np.random.default_rng(3)
    rows = np.concatenate([[0, R - 1], rng.integers(0, R, 6)])
    for r in rows:
        xb = x[int(r)].view(torch.int16).cpu().numpy().view(np.uint16)[None]
        want = quantize_values(xb, si)[0]
        assert np.array_equal(q[int(r)].cpu().numpy(), want), int(r)
        assert np.array_equal(qt[:, int(r)].cpu().numpy(), want), int(r)
    cols = np.concatenate([[0, C - 1], rng.integers(0, C, 6)])
    for c in cols:
        assert torch.equal(qt[int(c)], q[:, int(c)]), int(c)
    assert o_amax(np.array([[0x4214]], np.uint16)) == amax_host     # 37.0 as bf16
    del x, q, qt
    torch.cuda.empty_cache()
