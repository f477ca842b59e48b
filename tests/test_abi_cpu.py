"""The C ABI on the CPU: the library loads, exports every declared symbol, and rejects bad
arguments with the documented status before touching the GPU (no kernel is launched).

These calls hand the library small made-up addresses together with sizes or flags that its
host checks reject. They run only where no GPU is visible, so that a check that let one of
them through could never reach a kernel."""
import ctypes
import os
import re

import pytest


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0     # counts devices without initialising one
    except Exception:
        return False


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="passes made-up device addresses; "
                                "host-side checks are tested where no GPU is visible")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8lin.h")
LIB = os.path.join(ROOT, "scaled_fp8_linear_amd", "libfp8lin.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(fp8_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libfp8lin.so not built (python -m scaled_fp8_linear_amd.build)")
    import scaled_fp8_linear_amd as m
    return m.load()


def test_header_declares_the_six_calls():
    names = _declared()
    for n in ("fp8_quantize_amax", "fp8_scale_update", "fp8_linear_fwd", "fp8_linear_dgrad",
              "fp8_linear_wgrad", "fp8_pad_tokens", "fp8_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_version(lib):
    assert lib.fp8_version().decode().startswith("fp8lin")


def _err(lib):
    return lib.fp8_last_error().decode()


def test_token_count_not_multiple_of_16(lib):
    # SpecForge PR 2 quotes a token count of 3858, which float8 GEMMs reject.
    assert lib.fp8_linear_fwd(None, None, None, None, None, 3858, 4096, 4096, 3858, 0, None) == 2
    assert "3858" in _err(lib) and "16" in _err(lib)
    assert lib.fp8_linear_wgrad(None, None, None, None, None, 3858, 4096, 4096, 0, None) == 2


def test_gemm_argument_checks(lib):
    p = ctypes.c_void_p(16)
    assert lib.fp8_linear_fwd(p, p, p, p, None, 16, 16, 16, 16, 0, None) == 1        # NULL y
    assert lib.fp8_linear_fwd(p, p, p, p, ctypes.c_void_p(8), 16, 16, 16, 16, 0, None) == 3
    assert lib.fp8_linear_fwd(p, p, p, p, p, 16, 16, 16, 17, 0, None) == 2           # M_valid > M
    assert lib.fp8_linear_fwd(p, p, p, p, p, 16, 16, 16, 16, 9, None) == 4           # granularity
    assert lib.fp8_linear_fwd(p, p, p, p, p, 16, 16, 1 << 17, 16, 0, None) == 4      # K too long
    assert lib.fp8_linear_dgrad(p, p, p, p, p, 16, 16, -16, 16, 0, None) == 2
    assert lib.fp8_linear_fwd(p, p, p, p, p, 16, 16, 48, 16, 1, None) == 2           # block K%128
    assert lib.fp8_linear_fwd(p, p, None, p, p, 16, 16, 16, 16, 0, None) == 1        # NULL sx
    assert lib.fp8_linear_wgrad(p, p, p, None, p, 16, 16, 16, 0, None) == 1          # NULL sx


def test_current_small_argument_checks(lib):
    p = ctypes.c_void_p(16)
    f = lib.fp8_linear_fwd_current
    assert f(p, p, 24, 128, 128, p, p, None, None, None) == 2           # M % 16
    assert f(p, p, 64, 128, 64, p, p, None, None, None) == 2            # K % 128
    assert f(p, p, 0, 128, 128, p, p, None, None, None) == 2            # empty
    assert f(p, p, 256, 272, 128, p, p, None, None, None) == 4          # codes over 64 KiB
    assert "65536" in _err(lib) and "fp8_linear_fwd" in _err(lib)
    assert f(p, p, 64, 128, 128, None, p, None, None, None) == 1        # NULL y
    assert f(p, p, 64, 128, 128, p, None, None, None, None) == 1        # NULL scales
    assert f(p, p, 64, 128, 128, p, p, ctypes.c_void_p(8), None, None) == 3


def test_quantize_argument_checks(lib):
    p = ctypes.c_void_p(16)
    assert lib.fp8_quantize_amax(None, 16, 16, 16, 0, p, p, p, p, None, None, None) == 1
    assert lib.fp8_quantize_amax(p, 24, 16, 24, 0, p, p, p, p, None, None, None) == 2
    assert lib.fp8_quantize_amax(p, 16, 16, 17, 0, p, p, p, p, None, None, None) == 2
    assert lib.fp8_quantize_amax(p, 16, 16, 16, 0, None, p, None, p, None, None, None) == 1
    assert lib.fp8_quantize_amax(p, 16, 16, 16, 0, p, p, None, p, p, None, None) == 4
    assert lib.fp8_quantize_amax(p, 128, 128, 128, 1, p, p, None, None, p, None, None) == 4
    assert lib.fp8_quantize_amax(p, 128, 128, 128, 1, None, p, None, None, None, None, None) == 1
    assert lib.fp8_quantize_amax(p, 128, 128, 64, 2, None, p, None, None, p, None, None) == 2
    assert lib.fp8_quantize_amax(p, 16, 16, 16, 7, None, None, None, None, None, None, None) == 2


def test_scale_update_argument_checks(lib):
    p = ctypes.c_void_p(16)
    assert lib.fp8_scale_update(0, None, None, 0, 0, p, p, None) == 1
    assert lib.fp8_scale_update(1, p, p, 16, 16, None, None, None) == 2
    assert lib.fp8_scale_update(2, None, p, 0, 0, p, p, None) == 2
    assert lib.fp8_scale_update(5, p, p, 16, 0, p, p, None) == 4


def test_pad_tokens_query(lib):
    out = ctypes.c_int64(-1)
    for T, mult, want in ((3858, 16, 3872), (0, 16, 0), (16, 16, 16), (1, 16, 16), (67827, 16, 67840),
                          (5, 8, 8)):
        assert lib.fp8_pad_tokens(None, T, 4096, mult, None, ctypes.byref(out), None) == 0
        assert out.value == want
    assert lib.fp8_pad_tokens(None, 5, 8, 0, None, ctypes.byref(out), None) == 2
    assert lib.fp8_pad_tokens(None, 5, 8, 16, None, None, None) == 1


def test_amax_flag_checks(lib):
    p = ctypes.c_void_p(16)
    # accumulate is for tensorwise passes only
    assert lib.fp8_quantize_amax(p, 128, 128, 128, 1 | 0x100, None, p, None, p, p, None,
                                 None) == 4
    # clear needs a mode that reads amax
    assert lib.fp8_scale_update(2 | 0x100, p, p, 16, 0, p, p, None) == 4
    assert lib.fp8_scale_update(0 | 0x100, None, None, 0, 0, p, p, None) == 1


def test_e5m2_flag_checks(lib):
    p = ctypes.c_void_p(16)
    # E5M2 codes: tensorwise passes only
    assert lib.fp8_quantize_amax(p, 128, 128, 128, 1 | 0x200, None, p, None, p, p, None,
                                 None) == 4
    # the format maximum matters only to modes that write scales
    assert lib.fp8_scale_update(1 | 0x200, p, p, 16, 0, None, None, None) == 4
    # an E5M2 first operand: tensorwise GEMMs only, and no bias epilogue
    assert lib.fp8_linear_dgrad(p, p, p, p, p, 128, 128, 128, 128, 1 | 0x200, None) == 4
    assert lib.fp8_linear_fwd_bias(p, p, p, p, p, p, 16, 16, 16, 16, 0x200, None) == 4
    # the flag passes the host checks (shape errors are still reported as such)
    assert lib.fp8_linear_wgrad(p, p, p, p, p, 24, 16, 16, 0x200, None) == 2


def test_align_multiple_matches_the_oracle(lib):
    import scaled_fp8_linear_amd as m
    from oracle import padding
    for B in (1, 3, 6, 16, 32):
        for tp in (1, 2, 3, 4, 8):
            for base in (8, 16):
                assert m.fp8_align_multiple(m.FP8_LAYOUT_BSHD, B, tp, 1, base) == \
                    padding.align_multiples(padding.BSHD, B, tp, 1, base), (B, tp, base)
    for tp in (1, 2, 4):
        for cp in (1, 2, 4):
            assert m.fp8_align_multiple(m.FP8_LAYOUT_THD, 1, tp, cp) == \
                padding.align_multiples(padding.THD, 1, tp, cp)
    s, t = ctypes.c_int32(), ctypes.c_int32()
    assert lib.fp8_align_multiple(1, 4, 2, 2, 16, ctypes.byref(s), ctypes.byref(t)) == 4
    assert lib.fp8_align_multiple(7, 4, 2, 1, 16, ctypes.byref(s), ctypes.byref(t)) == 4
    assert lib.fp8_align_multiple(0, 4, 0, 1, 16, ctypes.byref(s), ctypes.byref(t)) == 2


def test_pad_varlen_offsets_match_the_oracle(lib):
    import numpy as np

    import scaled_fp8_linear_amd as m
    import torch
    from oracle import padding
    rng = np.random.default_rng(11)
    lens = [int(v) for v in rng.integers(0, 50, 40)]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = torch.empty((int(cu[-1]), 16), dtype=torch.bfloat16)      # host tensor: offsets only
    for sm, tm in ((1, 16), (4, 16), (8, 128), (3, 5)):
        _, cu_pad, T_pad = m.fp8_pad_varlen(x, cu, sm, tm, query_only=True)
        want, ocu = padding.pad_varlen(np.zeros((int(cu[-1]), 1), np.uint16), lens, sm, tm)
        assert cu_pad == list(ocu) and T_pad == want.shape[0], (sm, tm)
    bad = (ctypes.c_int64 * 3)(0, 5, 3)
    out = ctypes.c_int64()
    assert lib.fp8_pad_varlen(None, bad, 2, 16, 1, 16, None, None, ctypes.byref(out), None) == 2
    good = (ctypes.c_int64 * 3)(0, 5, 9)
    assert lib.fp8_pad_varlen(None, good, 2, 24, 1, 16, None, None, ctypes.byref(out), None) == 2
    assert lib.fp8_pad_varlen(None, good, 2, 16, 0, 16, None, None, ctypes.byref(out), None) == 2
    p = ctypes.c_void_p(16)
    assert lib.fp8_pad_varlen(p, good, 2, 16, 4, 16, p, None, ctypes.byref(out), None) == 1
    # a padded sequence shorter than its sequence
    short = (ctypes.c_int64 * 3)(0, 4, 8)
    assert lib.fp8_unpad_varlen(p, good, short, 2, 16, ctypes.c_void_p(32), None) == 2
