"""Scale arithmetic and the weight amax-history ring (test infrastructure only).

Source: AstrAI ``astrai/extension/fp8_state.py``.

* ``_update_delayed_scale``: ``a = clamp_min(float32(amax), 1e-12)``,
  ``scale = a / 448``, ``scale_inv = 448 / a``; written for the *next* call
  (activations and gradients are scaled one step late).
* ``FP8TensorMeta.__init__``: ``scale``, ``scale_inv`` start at 1.0; the amax
  history has ``update_interval`` (16) entries, all initialised to **1.0**;
  the ring index starts at 0.
* ``FP8TensorMeta.record``: ``hist[idx] = amax``; ``idx = (idx + 1) % len``.
* ``FP8TensorMeta.refresh``: ``m = max(hist)``; only if ``m > 0``:
  ``scale = m / 448``, ``scale_inv = 448 / m``.
* ``FP8State.step``: ``step_count += 1``; when ``step_count % 16 == 0`` every
  weight meta refreshes. ``fp8_autocast`` calls ``step`` once per entry, i.e.
  once per training step, before the forward.

Readings (the pages leave the rounding open):

* each quotient is ONE correctly rounded float32 division (numpy float32
  division is IEEE). PyTorch evaluates ``448.0 / tensor`` as a reciprocal
  followed by a multiply; the plain mathematical reading of the printed
  expression, one division, is used instead;
* the clamp keeps NaN (``clamp_min`` propagates NaN), so a NaN amax gives NaN
  scales; ``refresh`` skips a NaN window maximum because ``NaN > 0`` is false;
* 1e-12 is the float32 nearest to 1e-12 (bits 0x2B8CBCCC), as a Python float
  scalar meets a float32 tensor in ``clamp_min``.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = np.float32(448.0)
E5M2_MAX = np.float32(57344.0)   # gradients in the hybrid format: the E5M2 maximum
AMAX_FLOOR = np.float32(1e-12)
UPDATE_INTERVAL = 16


def scale_from_amax(amax, fmax=E4M3_MAX) -> tuple[np.float32, np.float32]:
    """``_update_delayed_scale``: (scale, scale_inv) from one amax value.
    ``fmax`` is the format's largest value: 448, or 57344 for E5M2 gradients."""
    a = np.float32(amax)
    fmax = np.float32(fmax)
    if not np.isnan(a) and a < AMAX_FLOOR:
        a = AMAX_FLOOR
    with np.errstate(invalid="ignore", divide="ignore"):
        scale = np.float32(a / fmax)
        scale_inv = np.float32(fmax / a)
    return scale, scale_inv


class WeightMeta:
    """The weight half of ``FP8TensorMeta``: scale, scale_inv and the ring."""

    def __init__(self, update_interval: int = UPDATE_INTERVAL):
        self.scale = np.float32(1.0)
        self.scale_inv = np.float32(1.0)
        self.hist = np.ones(update_interval, dtype=np.float32)
        self.idx = 0

    def record(self, amax) -> None:
        self.hist[self.idx] = np.float32(amax)
        self.idx = (self.idx + 1) % self.hist.size

    def refresh(self) -> None:
        m = np.float32(np.max(self.hist))       # NaN propagates through max
        if m > 0:                                # False for NaN: keep the old scale
            self.scale = np.float32(m / E4M3_MAX)
            self.scale_inv = np.float32(E4M3_MAX / m)


class StepCounter:
    """``FP8State.step``: one advance per training step."""

    def __init__(self, update_interval: int = UPDATE_INTERVAL):
        self.update_interval = update_interval
        self.step_count = 0

    def step(self) -> bool:
        """Advance; return True when the weight metas must refresh now."""
        self.step_count += 1
        return self.step_count % self.update_interval == 0
