"""PyTorch autograd wrapper over the scaled FP8 linear layer.

[AstrAI] ``astrai/extension/fp8_state.py``: ``fp8_autocast()`` switches linears to the fp8
path and advances the scale-update counter once per entry, so that weight scales refresh
from their 16-step amax window on every 16th entry; ``fp8_linear_forward`` /
``fp8_linear_backward`` run the quantize and scaled GEMM kernels with the delayed scales;
``FP8State.reset`` clears the state. The pieces here:

    with fp8_autocast():          # one step: the counter advances once
        y = layer(x)              # Fp8Linear: quantize + fp8 GEMM (forward)
    y.backward(g)                 # dgrad + wgrad from the forward's transposed codes

Outside ``fp8_autocast`` an ``Fp8Linear`` is a plain bf16 linear. Every number of the fp8
path is computed in the library's kernels; this module only routes tensors and keeps the
host-side counters. A layer advances its own delayed-scaling state the first time it runs
in a step (refreshing its weight scale if a multiple of the interval was reached since its
last step), and ends the step after its backward; a step that runs no backward keeps the
gradient scale as it was. Each layer is meant to run once per step (one forward and at
most one backward), the schedule delayed scaling assumes ([NeMo]: one scale update per
step).
"""
from __future__ import annotations

import contextlib
import math

import torch
import torch.nn.functional as F

from . import _abi
from .state import DelayedScalingLinear


class Fp8State:
    """Global fp8 switch and step counter ([AstrAI] ``FP8State``)."""

    def __init__(self, update_interval: int = 16):
        self.enabled = False
        self.update_interval = update_interval
        self.step_count = 0
        self.generation = 0          # bumped by reset(): layers then start afresh

    def reset(self) -> None:
        self.enabled = False
        self.step_count = 0
        self.generation += 1

    def state_dict(self) -> dict:
        return {"step_count": self.step_count, "update_interval": self.update_interval}

    def load_state_dict(self, d: dict) -> None:
        self.step_count = int(d["step_count"])
        self.update_interval = int(d["update_interval"])


_state = Fp8State()


def fp8_state() -> Fp8State:
    return _state


@contextlib.contextmanager
def fp8_autocast(enabled: bool = True, update_interval: int = 16):
    """Run Fp8Linear layers on the fp8 path; the step counter advances once on entry."""
    st = _state
    prev = (st.enabled, st.update_interval)
    st.enabled, st.update_interval = enabled, update_interval
    try:
        if enabled:
            st.step_count += 1
        yield
    finally:
        st.enabled, st.update_interval = prev


class _Fp8LinearFn(torch.autograd.Function):
    """y = x W^T through the fp8 path; backward gives dx (dgrad) and dW (wgrad). A token
    count that is not a multiple of 16 is padded here (fp8_pad_tokens) for the kernels,
    with the padded rows kept out of amax and outputs (rows_valid), and cut off again."""

    @staticmethod
    def forward(ctx, x2d, weight, bias, layer):
        M = x2d.shape[0]
        xp, M_pad = _abi.fp8_pad_tokens(x2d) if M % 16 else (x2d, M)
        b = None if bias is None else bias.detach()
        y = layer._lin.forward(xp, weight.detach(), rows_valid=M, bias=b)
        ctx.layer, ctx.M, ctx.M_pad, ctx.has_bias = layer, M, M_pad, bias is not None
        return y[:M] if M_pad != M else y

    @staticmethod
    def backward(ctx, gy):
        layer = ctx.layer
        gy = gy.contiguous()
        if gy.dtype != torch.bfloat16:
            gy = gy.to(torch.bfloat16)
        if ctx.M_pad != ctx.M:
            gy, _ = _abi.fp8_pad_tokens(gy)
        dx, dw = layer._lin.backward(gy)
        db = _abi.fp8_bias_grad(gy, rows_valid=ctx.M) if ctx.has_bias else None
        layer._lin.end_step()
        layer._pending = False
        return (dx[:ctx.M] if ctx.M_pad != ctx.M else dx), dw, db, None


class Fp8Linear(torch.nn.Module):
    """A linear layer y = x W^T (+ b) with a bf16 weight [out, in] (and bias [out]) that
    runs as the scaled FP8 linear inside ``fp8_autocast`` (delayed scaling, e4m3 operands,
    the bias added in the GEMM's epilogue, bf16 out; the bias gradient is a column sum of
    the output gradient).

    in_features and out_features must be multiples of 16 for the fp8 path (the fp8 GEMMs
    need it); the token count need not be: the layer pads it with fp8_pad_tokens and keeps
    the padded rows out of amax and outputs. The delayed-scaling state (weight amax ring,
    scales, slots, counters) is saved and restored with the module's state_dict.
    """

    def __init__(self, in_features: int, out_features: int, bias: bool = False, device=None,
                 update_interval: int = 16, grad_format: str = "e4m3"):
        super().__init__()
        if grad_format not in ("e4m3", "e5m2"):
            raise ValueError(f"grad_format must be 'e4m3' or 'e5m2', not {grad_format!r}")
        self.grad_format = grad_format
        self.in_features, self.out_features = in_features, out_features
        self.weight = torch.nn.Parameter(
            torch.empty((out_features, in_features), dtype=torch.bfloat16, device=device))
        bound = 1.0 / math.sqrt(in_features)          # nn.Linear's default initialisation
        torch.nn.init.uniform_(self.weight, -bound, bound)
        if bias:
            self.bias = torch.nn.Parameter(
                torch.empty(out_features, dtype=torch.bfloat16, device=device))
            torch.nn.init.uniform_(self.bias, -bound, bound)
        else:
            self.register_parameter("bias", None)
        self.update_interval = update_interval
        self._lin = None
        self._generation = -1
        self._last_step = 0
        self._pending = False

    def _fp8_ok(self) -> bool:
        return self.in_features % 16 == 0 and self.out_features % 16 == 0

    def _begin(self) -> None:
        st = _state
        if self._lin is None or self._generation != st.generation:
            self._lin = DelayedScalingLinear(self.weight.device, self.update_interval,
                                             grad_format=self.grad_format)
            self._generation, self._last_step, self._pending = st.generation, 0, False
        if self._last_step == st.step_count:
            return
        if self._pending:                 # the previous step ran no backward
            self._lin.end_step(g_updated=False)
            self._pending = False
        ui = self.update_interval
        refresh = st.step_count // ui > self._last_step // ui
        self._lin.begin_step(refresh=refresh)
        self._last_step = st.step_count

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if not _state.enabled or not self._fp8_ok():
            return F.linear(x, self.weight, self.bias)
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected {self.in_features} input features, got {x.shape[-1]}")
        self._begin()
        lead = x.shape[:-1]
        x2d = x.reshape(-1, self.in_features)
        if x2d.dtype != torch.bfloat16:
            x2d = x2d.to(torch.bfloat16)
        x2d = x2d.contiguous()
        # the step ends after the backward, or (none run) when the layer's next step begins
        self._pending = True
        b = self.bias
        if torch.is_grad_enabled() and (x.requires_grad or self.weight.requires_grad or
                                        (b is not None and b.requires_grad)):
            y = _Fp8LinearFn.apply(x2d, self.weight, b, self)
        else:
            with torch.no_grad():
                y = _Fp8LinearFn.forward(_NoCtx(), x2d, self.weight, b, self)
        return y.reshape(*lead, self.out_features)

    # delayed-scaling state in the module's state_dict
    def get_extra_state(self):
        st = {"last_step": self._last_step, "pending": self._pending}
        if self._lin is not None:
            st["lin"] = {k: (v.cpu() if torch.is_tensor(v) else v)
                         for k, v in self._lin.state_dict().items()}
        return st

    def set_extra_state(self, state) -> None:
        if "lin" not in state:
            self._lin = None
            return
        self._lin = DelayedScalingLinear(self.weight.device, self.update_interval,
                                         grad_format=self.grad_format)
        self._lin.load_state_dict(state["lin"])
        self._generation = _state.generation
        self._last_step = int(state["last_step"])
        self._pending = bool(state["pending"])


class _NoCtx:
    """Stands in for autograd's context when the forward runs without a graph."""
