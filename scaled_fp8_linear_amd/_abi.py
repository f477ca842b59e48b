"""ctypes binding of ``libfp8lin.so``: argument marshalling only.

Each function here has the name of the C entry point it calls and passes
device pointers, sizes and the current HIP stream through. Every step of the
computation runs in the library's kernels; PyTorch only provides device
memory (outputs the caller did not pass are allocated with ``torch.empty``)
and the stream. If the library is missing this module raises: there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8lin.so")

FP8_OK, FP8_ERR_NULL, FP8_ERR_SHAPE, FP8_ERR_ALIGN, FP8_ERR_UNSUPPORTED, FP8_ERR_HIP = range(6)
FP8_TENSORWISE, FP8_BLOCK_1x128, FP8_BLOCK_128x128 = 0, 1, 2
FP8_SCALE_FROM_AMAX, FP8_SCALE_RECORD, FP8_SCALE_REFRESH = 0, 1, 2
FP8_AMAX_ACCUMULATE = 0x100     # flag for fp8_quantize_amax (tensorwise)
FP8_SCALE_CLEAR_AMAX = 0x100    # flag for fp8_scale_update (FROM_AMAX, RECORD)
FP8_E5M2 = 0x200                # flag: E5M2 codes (quantize), 57344 as format max (scale update)
FP8_A_E5M2 = 0x200              # flag for the GEMMs: the first operand holds E5M2 codes

EXPORTS = ("fp8_quantize_amax", "fp8_scale_update", "fp8_linear_fwd", "fp8_linear_dgrad",
           "fp8_linear_wgrad", "fp8_pad_tokens", "fp8_last_error", "fp8_version",
           "fp8_linear_fwd_bias", "fp8_bias_grad", "fp8_align_multiple", "fp8_pad_varlen",
           "fp8_unpad_varlen", "fp8_linear_fwd_current")
FP8_LAYOUT_THD, FP8_LAYOUT_BSHD = 0, 1


class Fp8Error(RuntimeError):
    """An fp8lin entry point returned an error status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed (status {status}): {msg}")
        self.status = status


_lib = None

_i64, _i32, _int, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_void_p


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once; raise if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m scaled_fp8_linear_amd.build` "
                           "(the HIP library is required; there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    lib.fp8_quantize_amax.argtypes = [_vp, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.fp8_scale_update.argtypes = [_int, _vp, _vp, _i32, _i32, _vp, _vp, _vp]
    lib.fp8_linear_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp]
    lib.fp8_linear_fwd_bias.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                        _int, _vp]
    lib.fp8_bias_grad.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp]
    lib.fp8_linear_fwd_current.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]
    lib.fp8_linear_dgrad.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp]
    lib.fp8_linear_wgrad.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp]
    lib.fp8_pad_tokens.argtypes = [_vp, _i64, _i64, _i32, _vp, ctypes.POINTER(_i64), _vp]
    _p64, _p32 = ctypes.POINTER(_i64), ctypes.POINTER(_i32)
    lib.fp8_align_multiple.argtypes = [_int, _i64, _i32, _i32, _i32, _p32, _p32]
    lib.fp8_pad_varlen.argtypes = [_vp, _p64, _i32, _i64, _i32, _i32, _vp, _p64, _p64, _vp]
    lib.fp8_unpad_varlen.argtypes = [_vp, _p64, _p64, _i32, _i64, _vp, _vp]
    for name in EXPORTS:
        if name not in ("fp8_last_error", "fp8_version"):
            getattr(lib, name).restype = _int
    lib.fp8_last_error.restype = ctypes.c_char_p
    lib.fp8_last_error.argtypes = []
    lib.fp8_version.restype = ctypes.c_char_p
    lib.fp8_version.argtypes = []
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != FP8_OK:
        raise Fp8Error(fn, status, load().fp8_last_error().decode())


def _ptr(t, offset_elems: int = 0):
    """Device address of a tensor (plus an element offset), or None."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("fp8lin takes device tensors")
    if not t.is_contiguous():
        raise ValueError("fp8lin takes contiguous row-major tensors")
    p = t.data_ptr()
    return p + offset_elems * t.element_size() if offset_elems else p


# The current stream's raw handle. torch.cuda.current_stream() builds a Stream object on
# every call, about 3 us of host time, more than this library's own launch; torch's raw
# accessor returns the same handle without it. Where a torch build lacks it, the public
# call serves.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None and _cur_device is not None:
        return _raw_stream(_cur_device())
    return torch.cuda.current_stream().cuda_stream


_CODE_DTYPES = (torch.uint8, torch.float8_e4m3fn, torch.float8_e5m2)
_BF16_DTYPES = (torch.bfloat16, torch.int16, torch.uint16)


def _codes(t):
    """uint8 view of an fp8 code tensor (uint8, float8_e4m3fn or float8_e5m2 storage)."""
    if t is None:
        return None
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise ValueError(f"fp8 codes must be uint8 or float8 storage, got {t.dtype}")
    return t


def _bf16(t):
    if t.dtype not in _BF16_DTYPES:
        raise ValueError(f"expected a bf16 tensor, got {t.dtype}")
    return t


def _f32(t, name):
    if t is not None and t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    return t


class Slot:
    """A float32 element inside a device tensor (a scale slot), passed by address."""

    def __init__(self, tensor, index: int = 0):
        _f32(tensor, "slot")
        if not 0 <= int(index) < tensor.numel():
            raise ValueError(f"slot {index} is outside a tensor of {tensor.numel()} elements")
        self.tensor, self.index = tensor, int(index)

    def ptr(self):
        return _ptr(self.tensor, self.index)


def _fptr(v, name):
    if v is None:
        return None
    if isinstance(v, Slot):
        return v.ptr()
    return _ptr(_f32(v, name))


def _need(t, name, shape, dtypes, dev=None):
    """Check a buffer before its address goes to the library: dtype, exact shape,
    contiguity and device (``dev``: the device of the call's first operand). Raises
    ValueError; nothing has been enqueued at that point."""
    if t is None:
        return
    # one combined test on the common path (every attribute read costs), the reason after
    if (t.dtype in dtypes and t.shape == tuple(shape) and t.is_contiguous()
            and (dev is None or t.device == dev)):
        return
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    raise ValueError(f"{name} is on {t.device}, the operands on {dev}")


def _need_scalar(v, name, dev=None, count=1):
    """A float32 scale or amax: a Slot, or a tensor of at least ``count`` elements."""
    if v is None:
        return
    t = v.tensor if isinstance(v, Slot) else v
    _f32(t, name)
    if not isinstance(v, Slot) and t.numel() < count:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {count}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, the operands on {dev}")


def _need_scales(v, name, gran, grid, dev):
    """Tensorwise: one float32 scale; block recipe: the scale grid of that exact shape."""
    if gran & 0xFF == FP8_TENSORWISE:
        _need_scalar(v, name, dev)
    else:
        if isinstance(v, Slot):
            raise ValueError(f"{name}: the block recipe takes a scale grid, not a slot")
        _need(v, name, grid, (torch.float32,), dev)


def _grids(gran, rows, cols):
    """Shapes of (amax, scale, scale_t) for a block-recipe quantize of [rows, cols]."""
    if gran == FP8_BLOCK_1x128:
        return (rows, cols // 128), (rows, cols // 128), (cols, rows // 128)
    return (rows // 128, cols // 128), (rows // 128, cols // 128), (cols // 128, rows // 128)


def fp8_quantize_amax(x, rows_valid=None, gran=FP8_TENSORWISE, scale_inv=None, q=None, q_t=None,
                      amax=None, scale=None, scale_t=None, want_q=True, want_q_t=True,
                      want_amax=True, amax_accumulate=False, e5m2=False, stream=None):
    """Quantize a bf16 [rows, cols] tensor. Returns (q, q_t, amax, scale, scale_t).

    Outputs that are not passed in are allocated here (``want_*`` False skips them).
    ``amax_accumulate`` (tensorwise): fold max|x| into the given ``amax`` instead of
    overwriting it. ``e5m2`` (tensorwise): E5M2 codes instead of E4M3.
    """
    if amax_accumulate and amax is None:
        raise ValueError("amax_accumulate needs the amax tensor to fold into")
    _bf16(x)
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [rows, cols], got shape {tuple(x.shape)}")
    rows, cols = x.shape
    rv = rows if rows_valid is None else int(rows_valid)
    dev = x.device
    q, q_t = _codes(q), _codes(q_t)
    _need(q, "q", (rows, cols), _CODE_DTYPES, dev)
    _need(q_t, "q_t", (cols, rows), _CODE_DTYPES, dev)
    if gran == FP8_TENSORWISE:
        _need_scalar(scale_inv, "scale_inv", dev)
        _need_scalar(amax, "amax", dev)
        if scale is not None or scale_t is not None:
            raise ValueError("tensorwise quantize takes no scale grids")
    elif gran in (FP8_BLOCK_1x128, FP8_BLOCK_128x128):
        ga, gs, gst = _grids(gran, rows, cols)
        _need(amax, "amax", ga, (torch.float32,), dev)
        _need(scale, "scale", gs, (torch.float32,), dev)
        _need(scale_t, "scale_t", gst, (torch.float32,), dev)
    if want_q and q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if want_q_t and q_t is None:
        q_t = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    if gran == FP8_TENSORWISE:
        if want_amax and amax is None:
            amax = torch.empty(1, dtype=torch.float32, device=dev)
    elif gran in (FP8_BLOCK_1x128, FP8_BLOCK_128x128):
        ga, gs, gst = _grids(gran, rows, cols)
        if want_amax and amax is None:
            amax = torch.empty(ga, dtype=torch.float32, device=dev)
        if q is not None and scale is None:
            scale = torch.empty(gs, dtype=torch.float32, device=dev)
        if q_t is not None and scale_t is None:
            scale_t = torch.empty(gst, dtype=torch.float32, device=dev)
    _check("fp8_quantize_amax", load().fp8_quantize_amax(
        _ptr(x), rows, cols, rv,
        gran | (FP8_AMAX_ACCUMULATE if amax_accumulate else 0) | (FP8_E5M2 if e5m2 else 0),
        _fptr(scale_inv, "scale_inv"), _ptr(q), _ptr(q_t),
        _fptr(amax, "amax"), _fptr(scale, "scale"), _fptr(scale_t, "scale_t"), _stream(stream)))
    return q, q_t, amax, scale, scale_t


def fp8_scale_update(mode, amax=None, hist=None, pos=0, scale=None, scale_inv=None,
                     clear_amax=False, e5m2=False, stream=None):
    """One scale bookkeeping op on the device (see fp8lin.h for the modes).
    ``clear_amax``: set amax to +0 after reading it (FROM_AMAX, RECORD).
    ``e5m2``: scales for E5M2 codes (57344 in place of 448; FROM_AMAX, REFRESH)."""
    if hist is not None:
        _f32(hist, "hist")
        if hist.dim() != 1 or not hist.is_contiguous():
            raise ValueError("hist must be a contiguous 1-D float32 tensor")
    length = 0 if hist is None else hist.numel()
    for v, name in ((amax, "amax"), (scale, "scale"), (scale_inv, "scale_inv")):
        _need_scalar(v, name)
    flags = (FP8_SCALE_CLEAR_AMAX if clear_amax else 0) | (FP8_E5M2 if e5m2 else 0)
    _check("fp8_scale_update", load().fp8_scale_update(
        int(mode) | flags, _fptr(amax, "amax"), _fptr(hist, "hist"), length, int(pos),
        _fptr(scale, "scale"), _fptr(scale_inv, "scale_inv"), _stream(stream)))


def _operands(a, b, an, bn):
    """Two code operands with the contraction index last; returns (a, b) as uint8 views."""
    a, b = _codes(a), _codes(b)
    for t, name in ((a, an), (b, bn)):
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D code tensor")
    if b.device != a.device:
        raise ValueError(f"{bn} is on {b.device}, {an} on {a.device}")
    if a.shape[1] != b.shape[1]:
        raise ValueError(f"{an} {tuple(a.shape)} and {bn} {tuple(b.shape)}: contraction sizes "
                         "differ")
    return a, b


def _m_valid(M_valid, M):
    mv = M if M_valid is None else int(M_valid)
    if not 0 <= mv <= M:
        raise ValueError(f"M_valid={mv} outside [0, {M}]")
    return mv


def fp8_linear_fwd(qx, qw, sx, sw, y=None, M_valid=None, gran=FP8_TENSORWISE, stream=None,
                   bias=None, a_e5m2=False):
    """y [M, N] bf16 = sx * sw * qx [M, K] . qw [N, K]^T (+ bias [N], bf16, in the epilogue).
    ``a_e5m2``: qx holds E5M2 codes."""
    qx, qw = _operands(qx, qw, "qx", "qw")
    M, K = qx.shape
    N = qw.shape[0]
    dev = qx.device
    _need_scales(sx, "sx", gran, (M, K // 128), dev)
    _need_scales(sw, "sw", gran, (N // 128, K // 128), dev)
    _need(y, "y", (M, N), _BF16_DTYPES, dev)
    if bias is not None:
        _need(_bf16(bias), "bias", (N,), _BF16_DTYPES, dev)
    mv = _m_valid(M_valid, M)
    gran = gran | (FP8_A_E5M2 if a_e5m2 else 0)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if bias is not None:
        _check("fp8_linear_fwd_bias", load().fp8_linear_fwd_bias(
            _ptr(qx), _ptr(qw), _fptr(sx, "sx"), _fptr(sw, "sw"), _ptr(bias), _ptr(y), M, N, K,
            mv, gran, _stream(stream)))
        return y
    _check("fp8_linear_fwd", load().fp8_linear_fwd(
        _ptr(qx), _ptr(qw), _fptr(sx, "sx"), _fptr(sw, "sw"), _ptr(y), M, N, K, mv, gran,
        _stream(stream)))
    return y


def fp8_linear_fwd_current(x, w, y=None, scales=None, qx=None, qw=None, want_codes=False,
                           stream=None):
    """One current-scaling forward of a small linear in one launch: amax of x [M, K] and of
    w [N, K] (bf16), their scales, the casts, y [M, N] bf16. Returns (y, scales, qx, qw):
    scales float32 [4] = {sx, sw, sx_inv, sw_inv}; qx, qw the e4m3 codes when passed or
    ``want_codes``, else None."""
    x, w = _bf16(x), _bf16(w)
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"x {tuple(x.shape)} and w {tuple(w.shape)} must be [M, K] and [N, K]")
    M, K = x.shape
    N = w.shape[0]
    dev = x.device
    _need(x, "x", (M, K), _BF16_DTYPES, dev)
    _need(w, "w", (N, K), _BF16_DTYPES, dev)
    _need(y, "y", (M, N), _BF16_DTYPES, dev)
    _need(scales, "scales", (4,), (torch.float32,), dev)
    _need(qx, "qx", (M, K), (torch.uint8,), dev)
    _need(qw, "qw", (N, K), (torch.uint8,), dev)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if scales is None:
        scales = torch.empty(4, dtype=torch.float32, device=dev)
    if want_codes and qx is None:
        qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if want_codes and qw is None:
        qw = torch.empty((N, K), dtype=torch.uint8, device=dev)
    _check("fp8_linear_fwd_current", load().fp8_linear_fwd_current(
        _ptr(x), _ptr(w), M, N, K, _ptr(y), _ptr(scales), _ptr(qx), _ptr(qw), _stream(stream)))
    return y, scales, qx, qw


def fp8_bias_grad(g, rows_valid=None, db=None, stream=None):
    """db [cols] bf16 = column sums of g [rows, cols] over the valid rows (float32 sums)."""
    _bf16(g)
    if g.dim() != 2:
        raise ValueError(f"g must be 2-D [rows, cols], got shape {tuple(g.shape)}")
    rows, cols = g.shape
    rv = _m_valid(rows_valid, rows)
    _need(db, "db", (cols,), _BF16_DTYPES, g.device)
    if db is None:
        db = torch.empty(cols, dtype=torch.bfloat16, device=g.device)
    _check("fp8_bias_grad", load().fp8_bias_grad(_ptr(g), rows, cols, rv, _ptr(db),
                                                 _stream(stream)))
    return db


def fp8_linear_dgrad(qg, qw_t, sg, sw, dx=None, M_valid=None, gran=FP8_TENSORWISE, stream=None,
                     a_e5m2=False):
    """dx [M, K] bf16 = sg * sw * qg [M, N] . qw_t [K, N]^T. ``a_e5m2``: qg holds E5M2 codes.
    Block recipe: sg [M, N/128], sw is W's transposed scale grid [K/128, N/128]."""
    qg, qw_t = _operands(qg, qw_t, "qg", "qw_t")
    M, N = qg.shape
    K = qw_t.shape[0]
    dev = qg.device
    _need_scales(sg, "sg", gran, (M, N // 128), dev)
    _need_scales(sw, "sw", gran, (K // 128, N // 128), dev)
    _need(dx, "dx", (M, K), _BF16_DTYPES, dev)
    mv = _m_valid(M_valid, M)
    gran = gran | (FP8_A_E5M2 if a_e5m2 else 0)
    if dx is None:
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    _check("fp8_linear_dgrad", load().fp8_linear_dgrad(
        _ptr(qg), _ptr(qw_t), _fptr(sg, "sg"), _fptr(sw, "sw"), _ptr(dx), M, N, K, mv, gran,
        _stream(stream)))
    return dx


def fp8_linear_wgrad(qg_t, qx_t, sg, sx, dw=None, gran=FP8_TENSORWISE, stream=None,
                     a_e5m2=False):
    """dw [N, K] bf16 = sg * sx * qg_t [N, M] . qx_t [K, M]^T. ``a_e5m2``: qg_t holds E5M2
    codes. Block recipe: sg [N, M/128], sx [K, M/128] (the transposed copies' grids)."""
    qg_t, qx_t = _operands(qg_t, qx_t, "qg_t", "qx_t")
    N, M = qg_t.shape
    K = qx_t.shape[0]
    dev = qg_t.device
    _need_scales(sg, "sg", gran, (N, M // 128), dev)
    _need_scales(sx, "sx", gran, (K, M // 128), dev)
    _need(dw, "dw", (N, K), _BF16_DTYPES, dev)
    gran = gran | (FP8_A_E5M2 if a_e5m2 else 0)
    if dw is None:
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    _check("fp8_linear_wgrad", load().fp8_linear_wgrad(
        _ptr(qg_t), _ptr(qx_t), _fptr(sg, "sg"), _fptr(sx, "sx"), _ptr(dw), M, N, K, gran,
        _stream(stream)))
    return dw


def fp8_pad_tokens(x, T=None, multiple=16, x_pad=None, query_only=False, stream=None):
    """Pad a bf16 [T, cols] batch to a multiple of ``multiple`` rows.

    Returns ``(x_pad, T_pad)``. With ``query_only`` only T_pad is computed. If
    ``x_pad is x`` the tail of x's own buffer (which must hold T_pad rows) is
    zeroed in place, with T given explicitly.
    """
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [rows, cols], got shape {tuple(x.shape)}")
    cols = x.shape[1]
    T = x.shape[0] if T is None else int(T)
    out = ctypes.c_int64(0)
    lib = load()
    _check("fp8_pad_tokens", lib.fp8_pad_tokens(None, T, cols, int(multiple), None,
                                                ctypes.byref(out), None))
    T_pad = out.value
    if query_only:
        return None, T_pad
    _bf16(x)
    if x_pad is x:
        if x.shape[0] < T_pad:
            raise ValueError(f"in place: the buffer holds {x.shape[0]} rows, needs {T_pad}")
    elif x.shape[0] < T:
        raise ValueError(f"x holds {x.shape[0]} rows, T={T}")
    if x_pad is None:
        x_pad = torch.empty((T_pad, cols), dtype=x.dtype, device=x.device)
    _bf16(x_pad)
    if x_pad.dim() != 2 or x_pad.shape[0] < T_pad or x_pad.shape[1] != cols:
        raise ValueError(f"x_pad has shape {tuple(x_pad.shape)}, needs at least [{T_pad}, {cols}]")
    if x_pad.device != x.device:
        raise ValueError("x_pad and x are on different devices")
    _check("fp8_pad_tokens", lib.fp8_pad_tokens(_ptr(x), T, cols, int(multiple),
                                                _ptr(x_pad), ctypes.byref(out), _stream(stream)))
    return x_pad, T_pad


def fp8_align_multiple(layout, batch=1, tp=1, cp=1, base=16):
    """(per-sequence multiple, total multiple) of a token layout (FP8_LAYOUT_THD or
    FP8_LAYOUT_BSHD) under tensor/sequence (tp) and context (cp) parallelism."""
    seq, tot = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("fp8_align_multiple", load().fp8_align_multiple(
        int(layout), int(batch), int(tp), int(cp), int(base), ctypes.byref(seq),
        ctypes.byref(tot)))
    return seq.value, tot.value


def _offsets(cu):
    arr = (_i64 * len(cu))(*[int(v) for v in cu])
    return arr


def fp8_pad_varlen(x, cu_seqlens, seq_multiple=1, total_multiple=16, x_pad=None,
                   query_only=False, stream=None):
    """Pad every sequence of a packed bf16 [T, cols] batch to a multiple of ``seq_multiple``
    rows and the batch to a multiple of ``total_multiple``. ``cu_seqlens``: host offsets
    [nseq + 1] (a list, or a CPU tensor). Returns ``(x_pad, cu_seqlens_pad, T_pad)``;
    ``query_only`` computes the offsets only (x_pad is None)."""
    cu = _offsets([int(v) for v in cu_seqlens])
    nseq = len(cu) - 1
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [rows, cols], got shape {tuple(x.shape)}")
    cols = x.shape[1]
    cu_pad = (_i64 * (nseq + 1))()
    T_pad = ctypes.c_int64(0)
    lib = load()
    _check("fp8_pad_varlen", lib.fp8_pad_varlen(None, cu, nseq, cols, int(seq_multiple),
                                                int(total_multiple), None, cu_pad,
                                                ctypes.byref(T_pad), None))
    if query_only:
        return None, list(cu_pad), T_pad.value
    _bf16(x)
    if x.shape[0] < cu[nseq]:
        raise ValueError(f"x holds {x.shape[0]} rows, the offsets reach {cu[nseq]}")
    if x_pad is None:
        x_pad = torch.empty((T_pad.value, cols), dtype=x.dtype, device=x.device)
    _bf16(x_pad)
    if x_pad.dim() != 2 or x_pad.shape[0] < T_pad.value or x_pad.shape[1] != cols:
        raise ValueError(f"x_pad has shape {tuple(x_pad.shape)}, needs at least "
                         f"[{T_pad.value}, {cols}]")
    if x_pad.device != x.device:
        raise ValueError("x_pad and x are on different devices")
    _check("fp8_pad_varlen", lib.fp8_pad_varlen(_ptr(x), cu, nseq, cols,
                                                int(seq_multiple), int(total_multiple),
                                                _ptr(x_pad), cu_pad, ctypes.byref(T_pad),
                                                _stream(stream)))
    return x_pad, list(cu_pad), T_pad.value


def fp8_unpad_varlen(x_pad, cu_seqlens, cu_seqlens_pad, x=None, stream=None):
    """The inverse gather of fp8_pad_varlen: the sequences' rows of x_pad, packed."""
    cu = _offsets([int(v) for v in cu_seqlens])
    cu_pad = _offsets([int(v) for v in cu_seqlens_pad])
    nseq = len(cu) - 1
    if len(cu_pad) != nseq + 1:
        raise ValueError("cu_seqlens and cu_seqlens_pad differ in length")
    _bf16(x_pad)
    if x_pad.dim() != 2:
        raise ValueError(f"x_pad must be 2-D [rows, cols], got shape {tuple(x_pad.shape)}")
    cols = x_pad.shape[1]
    if x_pad.shape[0] < cu_pad[nseq]:
        raise ValueError(f"x_pad holds {x_pad.shape[0]} rows, the padded offsets reach "
                         f"{cu_pad[nseq]}")
    if x is None:
        x = torch.empty((int(cu[nseq]), cols), dtype=x_pad.dtype, device=x_pad.device)
    _bf16(x)
    if x.dim() != 2 or x.shape[0] < cu[nseq] or x.shape[1] != cols:
        raise ValueError(f"x has shape {tuple(x.shape)}, needs at least [{cu[nseq]}, {cols}]")
    if x.device != x_pad.device:
        raise ValueError("x and x_pad are on different devices")
    _check("fp8_unpad_varlen", load().fp8_unpad_varlen(_ptr(x_pad), cu, cu_pad, nseq,
                                                      cols, _ptr(x), _stream(stream)))
    return x


def fp8_last_error() -> str:
    return load().fp8_last_error().decode()


def fp8_version() -> str:
    return load().fp8_version().decode()
