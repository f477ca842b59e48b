"""Host-side schedule of delayed scaling for one FP8 linear layer.

This is the bookkeeping of AstrAI's ``fp8_state.py`` (``FP8TensorMeta``,
``FP8State.step``, ``fp8_linear_forward`` / ``fp8_linear_backward``) laid over
the C ABI. All arithmetic runs in the library's kernels; this class only owns
the device tensors that hold the scales and the ring, the host-side ring index
and step counter, and the order of calls:

    begin_step()   step_count += 1; every 16th step: REFRESH the weight scale
    forward(x, w)  quantize W (scale_inv), RECORD amax_w, quantize x with the
                   delayed x scale, forward GEMM, FROM_AMAX(amax_x) -> next slot
    backward(g)    quantize g with the delayed g scale, dgrad (Qg, Qw^T),
                   wgrad (Qg^T, Qx^T with the scale that made Qx^T),
                   FROM_AMAX(amax_g) -> next slot (g in E4M3, or in E5M2 for
                   the hybrid format)
    end_step()     the next slots become current

Reading: the activation and gradient scales live in two slots (current,
next) so that wgrad multiplies Qx^T by the scale that produced it, while the
update for the next step is written as soon as amax is known. Each amax
buffer is folded into by its quantize pass (FP8_AMAX_ACCUMULATE) and cleared by
the update that reads it (FP8_SCALE_CLEAR_AMAX), so no pass needs a separate
launch to zero it first. Nothing here synchronizes with the device.
"""
from __future__ import annotations

import torch

from . import _abi
from ._abi import Slot


class _NoProbe:
    def __call__(self, tag):
        return self

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


class DelayedScalingLinear:
    """Delayed scaling for one linear layer (weight meta + activation/gradient scales).

    ``probe(tag)`` may be given to wrap each kernel call in a context manager
    (the benchmark records HIP events with it); tags are "quantize", "gemm"
    and "scale".
    """

    def __init__(self, device, update_interval: int = 16, probe=None, keep_amax: bool = False,
                 grad_format: str = "e4m3"):
        """``keep_amax``: leave each amax in its buffer after the update that reads it (every
        quantize pass then zeroes its buffer first: one more launch per pass); for
        inspecting the amaxes of a step. ``grad_format`` "e5m2": the hybrid format, with the
        output gradient coded in E5M2 (scales from 57344) and x, W in E4M3."""
        if grad_format not in ("e4m3", "e5m2"):
            raise ValueError(f"grad_format must be 'e4m3' or 'e5m2', not {grad_format!r}")
        self.grad_format = grad_format
        self._g5 = grad_format == "e5m2"
        self.probe = probe or _NoProbe()
        self.acc = not keep_amax
        f32 = dict(dtype=torch.float32, device=device)
        self.update_interval = update_interval
        self.step_count = 0
        self.w_scale = torch.ones(1, **f32)
        self.w_scale_inv = torch.ones(1, **f32)
        self.hist = torch.ones(update_interval, **f32)
        self.idx = 0
        # [slot] pairs for activations and gradients
        self.x_scale = torch.ones(2, **f32)
        self.x_scale_inv = torch.ones(2, **f32)
        self.g_scale = torch.ones(2, **f32)
        self.g_scale_inv = torch.ones(2, **f32)
        self.cur = 0
        # each amax is folded into by one quantize pass and cleared by the update that
        # reads it, so it is zero whenever a pass starts
        self.amax_w = torch.zeros(1, **f32)
        self.amax_x = torch.zeros(1, **f32)
        self.amax_g = torch.zeros(1, **f32)
        self._saved = None

    @property
    def nxt(self) -> int:
        return 1 - self.cur

    def begin_step(self, stream=None, refresh: bool | None = None) -> bool:
        """Advance one step; refresh the weight scale from the ring every update_interval
        steps (or as ``refresh`` says, when a caller keeps the step count globally)."""
        self.step_count += 1
        if refresh is None:
            refresh = self.step_count % self.update_interval == 0
        if refresh:
            with self.probe("scale"):
                _abi.fp8_scale_update(_abi.FP8_SCALE_REFRESH, hist=self.hist, scale=self.w_scale,
                                      scale_inv=self.w_scale_inv, stream=stream)
            return True
        return False

    def forward(self, x, w, rows_valid=None, out=None, bufs=None, stream=None, bias=None):
        """y = x W^T. ``bufs`` may hold preallocated qw, qw_t, qx, qx_t tensors."""
        b = bufs or {}
        p = self.probe
        with p("quantize"):
            qw, qw_t, _, _, _ = _abi.fp8_quantize_amax(
                w, scale_inv=self.w_scale_inv, q=b.get("qw"), q_t=b.get("qw_t"), amax=self.amax_w,
                amax_accumulate=self.acc, stream=stream)
        with p("scale"):
            _abi.fp8_scale_update(_abi.FP8_SCALE_RECORD, amax=self.amax_w, hist=self.hist,
                                  pos=self.idx, clear_amax=self.acc, stream=stream)
        self.idx = (self.idx + 1) % self.hist.numel()
        sx, sx_inv = Slot(self.x_scale, self.cur), Slot(self.x_scale_inv, self.cur)
        with p("quantize"):
            qx, qx_t, _, _, _ = _abi.fp8_quantize_amax(
                x, rows_valid=rows_valid, scale_inv=sx_inv, q=b.get("qx"), q_t=b.get("qx_t"),
                amax=self.amax_x, amax_accumulate=self.acc, stream=stream)
        with p("gemm"):
            y = _abi.fp8_linear_fwd(qx, qw, sx, self.w_scale, y=out, M_valid=rows_valid,
                                    stream=stream, bias=bias)
        with p("scale"):
            _abi.fp8_scale_update(_abi.FP8_SCALE_FROM_AMAX, amax=self.amax_x,
                                  scale=Slot(self.x_scale, self.nxt),
                                  scale_inv=Slot(self.x_scale_inv, self.nxt), clear_amax=self.acc,
                                  stream=stream)
        self._saved = (qx_t, qw_t, rows_valid)
        return y

    def backward(self, g, dx=None, dw=None, bufs=None, stream=None):
        """(dx, dW) for the output gradient g."""
        b = bufs or {}
        p = self.probe
        qx_t, qw_t, rows_valid = self._saved
        sg, sg_inv = Slot(self.g_scale, self.cur), Slot(self.g_scale_inv, self.cur)
        g5 = self._g5
        with p("quantize"):
            qg, qg_t, _, _, _ = _abi.fp8_quantize_amax(
                g, rows_valid=rows_valid, scale_inv=sg_inv, q=b.get("qg"), q_t=b.get("qg_t"),
                amax=self.amax_g, amax_accumulate=self.acc, e5m2=g5, stream=stream)
        with p("gemm"):
            dx = _abi.fp8_linear_dgrad(qg, qw_t, sg, self.w_scale, dx=dx, M_valid=rows_valid,
                                       stream=stream, a_e5m2=g5)
        with p("gemm"):
            dw = _abi.fp8_linear_wgrad(qg_t, qx_t, sg, Slot(self.x_scale, self.cur), dw=dw,
                                       stream=stream, a_e5m2=g5)
        with p("scale"):
            _abi.fp8_scale_update(_abi.FP8_SCALE_FROM_AMAX, amax=self.amax_g,
                                  scale=Slot(self.g_scale, self.nxt),
                                  scale_inv=Slot(self.g_scale_inv, self.nxt), clear_amax=self.acc,
                                  e5m2=g5, stream=stream)
        return dx, dw

    def end_step(self, g_updated: bool = True) -> None:
        """The next slots become current. ``g_updated`` False (a step without backward):
        the gradient scale carries over unchanged."""
        if not g_updated:
            self.g_scale[self.nxt:self.nxt + 1].copy_(self.g_scale[self.cur:self.cur + 1])
            self.g_scale_inv[self.nxt:self.nxt + 1].copy_(self.g_scale_inv[self.cur:self.cur + 1])
        self.cur = self.nxt

    _TENSORS = ("w_scale", "w_scale_inv", "hist", "x_scale", "x_scale_inv", "g_scale",
                "g_scale_inv")

    def state_dict(self) -> dict:
        """The whole schedule state: device tensors cloned, host counters as ints."""
        d = {k: getattr(self, k).detach().clone() for k in self._TENSORS}
        d.update(step_count=self.step_count, idx=self.idx, cur=self.cur,
                 update_interval=self.update_interval, grad_format=self.grad_format)
        return d

    def load_state_dict(self, d: dict) -> None:
        if int(d["update_interval"]) != self.update_interval:
            raise ValueError("update_interval differs from the saved state's")
        if d.get("grad_format", "e4m3") != self.grad_format:
            raise ValueError("grad_format differs from the saved state's")
        for k in self._TENSORS:
            getattr(self, k).copy_(d[k])
        self.step_count, self.idx, self.cur = int(d["step_count"]), int(d["idx"]), int(d["cur"])

    def state(self) -> dict:
        """Host copies of the schedule state (synchronizes; for tests)."""
        c = self.cur
        return dict(step=self.step_count, idx=self.idx, hist=self.hist.cpu().numpy().copy(),
                    w_scale=self.w_scale.item(), w_scale_inv=self.w_scale_inv.item(),
                    x_scale=self.x_scale[c].item(), x_scale_inv=self.x_scale_inv[c].item(),
                    g_scale=self.g_scale[c].item(), g_scale_inv=self.g_scale_inv[c].item())
