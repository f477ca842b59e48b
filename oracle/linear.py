"""One FP8 linear layer, step by step, as the pages schedule it (test infrastructure only).

Source: AstrAI ``fp8_state.py``: ``fp8_autocast`` / ``FP8State.step`` (one
advance per step, refresh every 16), ``fp8_linear_forward`` (quantize x with
the meta's delayed ``x_scale_inv`` and w with ``scale_inv``, scaled GEMM, then
``record(amax_w)`` and the delayed update of ``x_scale``) and
``fp8_linear_backward`` (quantize g with ``g_scale_inv``, dgrad and wgrad, then
the delayed update of ``g_scale``).

Reading for backward: dgrad and wgrad use the forward's transposed copies
(``Qw^T``, ``Qx^T``) together with the scales that produced them. The printed
code passes bf16 ``x`` and the already-updated ``x_scale`` to its backward
kernel; reusing the forward's bytes keeps one scale per quantized tensor and
is what the transposed copies are for.

Shapes: x [M, K], W [N, K], g = dL/dy [M, N]; y [M, N], dx [M, K], dW [N, K].
Rows ``m >= rows_valid`` are token padding: excluded from amax, zero in y/dx.
"""
from __future__ import annotations

import numpy as np

from . import block as blk
from .gemm import scaled_gemm
from .quantize import amax as amax_of
from .quantize import quantize_tensorwise
from .scaling import E4M3_MAX, E5M2_MAX, WeightScales, refresh_due, scale_from_amax


class DelayedLinear:
    """``FP8TensorMeta`` of one weight plus its activation/gradient scales.

    ``grad_format`` "e5m2" is the hybrid format: g is coded in E5M2 with scales
    from 57344 instead of 448, and dgrad/wgrad take it as their first operand;
    x and W stay E4M3."""

    def __init__(self, update_interval: int = 16, grad_format: str = "e4m3"):
        assert grad_format in ("e4m3", "e5m2")
        self.grad_format = grad_format
        self.update_interval = update_interval
        self.step = 0
        self.w = WeightScales(update_interval)
        self.x_scale = np.float32(1.0)
        self.x_scale_inv = np.float32(1.0)
        self.g_scale = np.float32(1.0)
        self.g_scale_inv = np.float32(1.0)
        self._saved = None

    def begin_step(self) -> bool:
        """``fp8_autocast`` entry: returns True if the weight scale refreshed."""
        self.step += 1
        refreshed = refresh_due(self.step, self.update_interval)
        if refreshed:
            self.w.refresh()
        return refreshed

    def forward(self, x_bits, w_bits, rows_valid=None):
        M = x_bits.shape[0]
        rv = M if rows_valid is None else int(rows_valid)
        sw, sw_inv = self.w.scale, self.w.scale_inv
        sx, sx_inv = self.x_scale, self.x_scale_inv
        qw, qw_t, amax_w = quantize_tensorwise(w_bits, sw_inv)
        qx, qx_t, amax_x = quantize_tensorwise(x_bits, sx_inv, rv)
        y = scaled_gemm(qx, qw, sx, sw)
        y[rv:] = 0.0
        self._finish_forward(amax_w, amax_x)
        self._saved = dict(qw_t=qw_t, qx_t=qx_t, sx=sx, sw=sw, rv=rv)
        return dict(y=y, qx=qx, qx_t=qx_t, qw=qw, qw_t=qw_t, amax_x=amax_x,
                    amax_w=amax_w, sx=sx, sx_inv=sx_inv, sw=sw, sw_inv=sw_inv)

    def backward(self, g_bits):
        s = self._saved
        rv = s["rv"]
        sg, sg_inv = self.g_scale, self.g_scale_inv
        gf = self.grad_format
        qg, qg_t, amax_g = quantize_tensorwise(g_bits, sg_inv, rv, gf)
        dx = scaled_gemm(qg, s["qw_t"], sg, s["sw"], gf)
        dx[rv:] = 0.0
        dw = scaled_gemm(qg_t, s["qx_t"], sg, s["sx"], gf)
        self._finish_backward(amax_g)
        return dict(dx=dx, dw=dw, qg=qg, qg_t=qg_t, amax_g=amax_g, sg=sg, sg_inv=sg_inv)

    def _finish_forward(self, amax_w, amax_x) -> None:
        """After the forward: record the weight amax, delay the activation scale."""
        self.w.record(amax_w)
        self.x_scale, self.x_scale_inv = scale_from_amax(amax_x)

    def _finish_backward(self, amax_g) -> None:
        """After the backward: delay the gradient scale."""
        fmax = E5M2_MAX if self.grad_format == "e5m2" else E4M3_MAX
        self.g_scale, self.g_scale_inv = scale_from_amax(amax_g, fmax)

    def scales_only_step(self, x_bits, w_bits, g_bits, rows_valid=None) -> dict:
        """The same bookkeeping as forward + backward without the GEMMs (for long runs at
        full size). Returns the scales in force during this step and the three amaxes."""
        rv = x_bits.shape[0] if rows_valid is None else int(rows_valid)
        used = dict(sw=self.w.scale, sw_inv=self.w.scale_inv, sx=self.x_scale,
                    sx_inv=self.x_scale_inv, sg=self.g_scale, sg_inv=self.g_scale_inv)
        aw, ax, ag = amax_of(w_bits), amax_of(x_bits, rv), amax_of(g_bits, rv)
        self._finish_forward(aw, ax)
        self._finish_backward(ag)
        used.update(amax_w=aw, amax_x=ax, amax_g=ag)
        return used

    def state(self) -> dict:
        return dict(step=self.step, w_scale=self.w.scale,
                    w_scale_inv=self.w.scale_inv, hist=self.w.hist, idx=self.w.pos,
                    x_scale=self.x_scale, x_scale_inv=self.x_scale_inv,
                    g_scale=self.g_scale, g_scale_inv=self.g_scale_inv)


def current_scaled_forward(x_bits, w_bits):
    """Dynamic tensorwise scaling (SpecForge PR 2, Modifications: torchao
    Float8Linear with dynamic tensorwise scaling): amax first, then the scale
    from ``scale_from_amax`` with no delay, then the cast and the GEMM."""
    ax = amax_of(x_bits)
    aw = amax_of(w_bits)
    sx, sx_inv = scale_from_amax(ax)
    sw, sw_inv = scale_from_amax(aw)
    qx, qx_t, _ = quantize_tensorwise(x_bits, sx_inv)
    qw, qw_t, _ = quantize_tensorwise(w_bits, sw_inv)
    y = scaled_gemm(qx, qw, sx, sw)
    return dict(y=y, qx=qx, qx_t=qx_t, qw=qw, qw_t=qw_t, amax_x=ax, amax_w=aw,
                sx=sx, sx_inv=sx_inv, sw=sw, sw_inv=sw_inv)


def block_linear_step(x_bits, w_bits, g_bits, rows_valid=None):
    """Forward, dgrad and wgrad under the block recipe (see ``oracle.block``)."""
    M = x_bits.shape[0]
    rv = M if rows_valid is None else int(rows_valid)
    qx, qx_t, ax, sx, sx_t = blk.quantize_1x128(x_bits, rv)
    qw, qw_t, aw, sw, sw_t = blk.quantize_128x128(w_bits)
    qg, qg_t, ag, sg, sg_t = blk.quantize_1x128(g_bits, rv)
    y = blk.block_scaled_gemm(qx, qw, sx, sw, 128)
    dx = blk.block_scaled_gemm(qg, qw_t, sg, sw_t, 128)
    dw = blk.block_scaled_gemm(qg_t, qx_t, sg_t, sx_t, 1)
    y[rv:] = 0.0
    dx[rv:] = 0.0
    return dict(y=y, dx=dx, dw=dw, qx=qx, qx_t=qx_t, sx=sx, sx_t=sx_t, amax_x=ax,
                qw=qw, qw_t=qw_t, sw=sw, sw_t=sw_t, amax_w=aw,
                qg=qg, qg_t=qg_t, sg=sg, sg_t=sg_t, amax_g=ag)
