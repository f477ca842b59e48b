"""Helpers for the GPU tests: host <-> device copies and case logging."""
import sys

import numpy as np
import torch


def note(msg: str) -> None:
    """Name the case before a GPU step (so a lost box still tells what ran)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """numpy uint16 bf16 patterns -> device bf16 tensor (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.cuda().view(torch.bfloat16)


def dev_f32(v) -> torch.Tensor:
    return torch.tensor(np.atleast_1d(np.asarray(v, dtype=np.float32)), device="cuda")


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.uint8).cpu().numpy()


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_bf16_f64(t: torch.Tensor) -> np.ndarray:
    b = host_bf16_bits(t).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_bits(v) -> int:
    return int(np.array(v, dtype=np.float32).view(np.uint32))


def assert_same_bytes(got: np.ndarray, want: np.ndarray, what: str) -> None:
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got.ravel() != want.ravel())
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {got.size} bytes differ; first at flat index "
                             f"{i}: got 0x{int(got.ravel()[i]):02x}, want 0x{int(want.ravel()[i]):02x}")


def assert_within(got: np.ndarray, exact: np.ndarray, bound: np.ndarray, what: str) -> float:
    """|got - exact| <= bound elementwise; returns the worst ratio err/bound."""
    err = np.abs(got - exact)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(np.max(ratio)) if ratio.size else 0.0
    assert worst <= 1.0, f"{what}: max |err|/bound = {worst:.3g}"
    return worst
