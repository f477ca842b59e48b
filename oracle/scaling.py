"""Scale arithmetic and the weight amax window (test infrastructure only).

Source: AstrAI ``astrai/extension/fp8_state.py`` (``_update_delayed_scale``,
``FP8TensorMeta``, ``FP8State``, ``fp8_autocast``). What the schedule is, in
its own terms:

* a scale pair from one amax: ``a = max(amax, 1e-12)``, dequant scale
  ``a / 448`` and quantize multiplier ``448 / a``; activations and gradients
  take the pair of their previous step's amax (one step late);
* every weight keeps a window of its last 16 recorded amaxes; before any is
  recorded all 16 entries are 1.0. Each step records the amax of the weight
  it quantized, the i-th recorded amax (counting from 0) taking entry
  ``i mod 16``;
* the weight's scale pair starts at (1.0, 1.0) and is recomputed from the
  window's maximum m at the start of every step whose number (from 1) is a
  multiple of 16, before that step's forward; when m is not positive (or is
  NaN) the pair stays as it was.

Readings (the pages leave the rounding open):

* each quotient is ONE correctly rounded float32 division (numpy float32
  division is IEEE). PyTorch evaluates ``448.0 / tensor`` as a reciprocal
  followed by a multiply; the plain mathematical reading of the printed
  expression, one division, is used instead;
* the clamp keeps NaN (``clamp_min`` propagates NaN), so a NaN amax gives NaN
  scales; a NaN window maximum leaves the weight's pair unchanged;
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


def window_after(recorded, length: int = UPDATE_INTERVAL) -> np.ndarray:
    """The amax window after ``recorded`` (in order): ``length`` entries that start at 1.0,
    the i-th recorded amax (from 0) in entry ``i mod length``."""
    w = np.ones(length, dtype=np.float32)
    for i, a in enumerate(recorded):
        w[i % length] = np.float32(a)
    return w


def window_scale(window, fmax=E4M3_MAX):
    """The scale pair from a window's maximum m, or None when m is NaN or not positive (the
    weight then keeps the pair it had)."""
    m = np.float32(np.max(np.asarray(window, dtype=np.float32)))   # NaN propagates
    if not m > 0:
        return None
    fmax = np.float32(fmax)
    return np.float32(m / fmax), np.float32(fmax / m)


def refresh_due(step: int, interval: int = UPDATE_INTERVAL) -> bool:
    """Whether step ``step`` (numbered from 1) recomputes the weight scales first."""
    return step % interval == 0


class WeightScales:
    """A weight's scale pair and the amaxes recorded for it."""

    def __init__(self, length: int = UPDATE_INTERVAL):
        self.length = length
        self.scale = np.float32(1.0)
        self.scale_inv = np.float32(1.0)
        self.recorded = []

    @property
    def hist(self) -> np.ndarray:
        return window_after(self.recorded, self.length)

    @property
    def pos(self) -> int:
        """The window entry the next recorded amax goes to."""
        return len(self.recorded) % self.length

    def record(self, amax) -> None:
        self.recorded.append(np.float32(amax))

    def refresh(self) -> None:
        pair = window_scale(self.hist)
        if pair is not None:
            self.scale, self.scale_inv = pair
