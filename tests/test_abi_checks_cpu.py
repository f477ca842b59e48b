"""The Python binding checks every buffer against the sizes it hands to the C ABI, and raises
ValueError before anything reaches the library: on the CPU, with host tensors, a buffer of
the wrong shape, dtype or layout is named in the error; with every shape right, the call
still stops at the device check (no address is ever passed for a host tensor)."""
import os

import pytest

torch = pytest.importorskip("torch")

import scaled_fp8_linear_amd as m  # noqa: E402

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "scaled_fp8_linear_amd", "libfp8lin.so")
u8, f32, bf = torch.uint8, torch.float32, torch.bfloat16


def _raises(fn, *words):
    with pytest.raises(ValueError) as e:
        fn()
    for w in words:
        assert w in str(e.value), (w, str(e.value))


def test_quantize_buffers():
    x = torch.zeros((32, 48), dtype=bf)
    one = torch.ones(1, dtype=f32)
    _raises(lambda: m.fp8_quantize_amax(x, scale_inv=one, q=torch.empty((32, 32), dtype=u8)), "q ")
    _raises(lambda: m.fp8_quantize_amax(x, scale_inv=one, q_t=torch.empty((32, 48), dtype=u8)),
            "q_t")
    _raises(lambda: m.fp8_quantize_amax(x, scale_inv=one, q=torch.empty((32, 48), dtype=f32)),
            "codes")
    _raises(lambda: m.fp8_quantize_amax(x, scale_inv=torch.ones(0, dtype=f32)), "scale_inv")
    _raises(lambda: m.fp8_quantize_amax(x, scale_inv=one, amax=torch.ones(1, dtype=torch.float64)),
            "amax")
    _raises(lambda: m.fp8_quantize_amax(x, scale_inv=one,
                                        q=torch.empty((48, 32), dtype=u8).t()), "q ")
    xb = torch.zeros((256, 384), dtype=bf)
    _raises(lambda: m.fp8_quantize_amax(xb, gran=m.FP8_BLOCK_1x128,
                                        scale=torch.empty((256, 2), dtype=f32)), "scale")
    _raises(lambda: m.fp8_quantize_amax(xb, gran=m.FP8_BLOCK_1x128,
                                        scale_t=torch.empty((384, 3), dtype=f32)), "scale_t")
    _raises(lambda: m.fp8_quantize_amax(xb, gran=m.FP8_BLOCK_128x128,
                                        amax=torch.empty((256, 3), dtype=f32)), "amax")
    # every shape right: stopped at the device check
    _raises(lambda: m.fp8_quantize_amax(x, scale_inv=one), "device")


def test_gemm_buffers():
    qa = torch.zeros((64, 256), dtype=u8)
    qb = torch.zeros((32, 256), dtype=u8)
    one = torch.ones(1, dtype=f32)
    _raises(lambda: m.fp8_linear_fwd(qa, torch.zeros((32, 128), dtype=u8), one, one),
            "contraction")
    _raises(lambda: m.fp8_linear_fwd(qa, qb, one, one, y=torch.empty((64, 16), dtype=bf)), "y ")
    _raises(lambda: m.fp8_linear_fwd(qa, qb, one, one, y=torch.empty((64, 32), dtype=f32)), "y ")
    _raises(lambda: m.fp8_linear_fwd(qa, qb, torch.ones(0, dtype=f32), one), "sx")
    _raises(lambda: m.fp8_linear_fwd(qa, qb, one, one, M_valid=65), "M_valid")
    _raises(lambda: m.fp8_linear_fwd(qa, qb, one, one, bias=torch.zeros(31, dtype=bf)), "bias")
    B = m.FP8_BLOCK_1x128
    qx, qw = torch.zeros((256, 512), dtype=u8), torch.zeros((384, 512), dtype=u8)
    _raises(lambda: m.fp8_linear_fwd(qx, qw, torch.ones((256, 3), dtype=f32),
                                     torch.ones((3, 4), dtype=f32), gran=B), "sx")
    _raises(lambda: m.fp8_linear_fwd(qx, qw, torch.ones((256, 4), dtype=f32),
                                     torch.ones((384, 4), dtype=f32), gran=B), "sw")
    _raises(lambda: m.fp8_linear_fwd(qx, qw, m.Slot(torch.ones(4, dtype=f32), 1),
                                     torch.ones((3, 4), dtype=f32), gran=B), "grid")
    # dgrad: sg [M, N/128], sw = W's transposed grid [K/128, N/128]
    qg, qw_t = torch.zeros((256, 384), dtype=u8), torch.zeros((512, 384), dtype=u8)
    _raises(lambda: m.fp8_linear_dgrad(qg, qw_t, torch.ones((256, 3), dtype=f32),
                                       torch.ones((3, 4), dtype=f32), gran=B), "sw")
    _raises(lambda: m.fp8_linear_dgrad(qg, qw_t, one, one, dx=torch.empty((256, 384), dtype=bf)),
            "dx")
    # wgrad: sg [N, M/128], sx [K, M/128]
    qg_t, qx_t = torch.zeros((384, 256), dtype=u8), torch.zeros((512, 256), dtype=u8)
    _raises(lambda: m.fp8_linear_wgrad(qg_t, qx_t, torch.ones((384, 1), dtype=f32),
                                       torch.ones((512, 2), dtype=f32), gran=B), "sg")
    _raises(lambda: m.fp8_linear_wgrad(qg_t, qx_t, torch.ones((384, 2), dtype=f32),
                                       torch.ones((512, 1), dtype=f32), gran=B), "sx")
    _raises(lambda: m.fp8_linear_wgrad(qg_t, qx_t, one, one, dw=torch.empty((512, 384), dtype=bf)),
            "dw")
    _raises(lambda: m.fp8_linear_fwd(qa, qb, one, one), "device")


def test_slot_and_scale_update_buffers():
    _raises(lambda: m.Slot(torch.ones(2, dtype=f32), 2), "slot")
    _raises(lambda: m.Slot(torch.ones(2, dtype=f32), -1), "slot")
    _raises(lambda: m.fp8_scale_update(m.FP8_SCALE_REFRESH, hist=torch.ones((4, 4), dtype=f32),
                                       scale=torch.ones(1, dtype=f32),
                                       scale_inv=torch.ones(1, dtype=f32)), "hist")
    _raises(lambda: m.fp8_scale_update(m.FP8_SCALE_FROM_AMAX, amax=torch.ones(0, dtype=f32),
                                       scale=torch.ones(1, dtype=f32),
                                       scale_inv=torch.ones(1, dtype=f32)), "amax")


def test_bias_grad_buffers():
    g = torch.zeros((64, 48), dtype=bf)
    _raises(lambda: m.fp8_bias_grad(g, db=torch.empty(32, dtype=bf)), "db")
    _raises(lambda: m.fp8_bias_grad(g, rows_valid=65), "M_valid")


@pytest.mark.skipif(not os.path.exists(LIB), reason="libfp8lin.so not built")
def test_padding_buffers():
    x = torch.zeros((37, 16), dtype=bf)
    _raises(lambda: m.fp8_pad_tokens(x, x_pad=torch.empty((40, 16), dtype=bf)), "x_pad")
    _raises(lambda: m.fp8_pad_tokens(x, x_pad=torch.empty((48, 32), dtype=bf)), "x_pad")
    _raises(lambda: m.fp8_pad_tokens(x, T=40, x_pad=torch.empty((48, 16), dtype=bf)), "T=40")
    _raises(lambda: m.fp8_pad_tokens(x, T=37, x_pad=x), "in place")
    cu = [0, 10, 30, 37]
    _raises(lambda: m.fp8_pad_varlen(torch.zeros((36, 16), dtype=bf), cu, 4, 16), "offsets")
    _, cu_pad, T_pad = m.fp8_pad_varlen(x, cu, 4, 16, query_only=True)
    _raises(lambda: m.fp8_pad_varlen(x, cu, 4, 16, x_pad=torch.empty((T_pad - 1, 16), dtype=bf)),
            "x_pad")
    _raises(lambda: m.fp8_unpad_varlen(torch.zeros((cu_pad[-1] - 1, 16), dtype=bf), cu, cu_pad),
            "padded offsets")
    _raises(lambda: m.fp8_unpad_varlen(torch.zeros((T_pad, 16), dtype=bf), cu, cu_pad,
                                       x=torch.empty((36, 16), dtype=bf)), "x has shape")
    _raises(lambda: m.fp8_unpad_varlen(torch.zeros((T_pad, 16), dtype=bf), cu, cu_pad[:-1]),
            "length")
    # shapes right: stopped at the device check
    _raises(lambda: m.fp8_pad_varlen(x, cu, 4, 16), "device")


def test_current_small_buffers():
    x, w = torch.zeros((64, 128), dtype=bf), torch.zeros((128, 128), dtype=bf)
    _raises(lambda: m.fp8_linear_fwd_current(x, torch.zeros((128, 64), dtype=bf)), "[M, K]")
    _raises(lambda: m.fp8_linear_fwd_current(x, w, y=torch.empty((64, 64), dtype=bf)), "y ")
    _raises(lambda: m.fp8_linear_fwd_current(x, w, scales=torch.empty(3, dtype=f32)), "scales")
    _raises(lambda: m.fp8_linear_fwd_current(x, w, qx=torch.empty((64, 128), dtype=f32)), "qx")
    _raises(lambda: m.fp8_linear_fwd_current(x, w, qw=torch.empty((128, 64), dtype=u8)), "qw")
    _raises(lambda: m.fp8_linear_fwd_current(x, w), "device")
