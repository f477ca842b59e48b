"""Seeded synthetic inputs for the scaled FP8 linear layer.

This module only draws random numbers and rounds them to bf16. It holds none of
the method's arithmetic (no quantize, no scale, no GEMM), and it is the one
module that both the CPU oracle's callers and the GPU path's callers use: the
tests and the benchmark generate bytes here and hand the SAME bytes to both.

Seeds: ``numpy.random.Generator(PCG64(SeedSequence([config, tensor, step, chunk])))``.
Large tensors are drawn in fixed chunks of ``CHUNK`` elements (each with its
own seed) so that the bytes do not depend on how many threads draw them.

The workloads stand in for the pages' data (LibriSpeech, ShareGPT, trained
Llama/Qwen weights), which are not used: shapes and value distributions follow
the configurations of the scaled FP8 linear benchmark (see ``CONFIGS``).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22

# tensor ids used in the seeds
T_X, T_W, T_G, T_H, T_WDOWN, T_GDOWN, T_DRIFT, T_LENS, T_WGATE, T_WUP, T_GGATE, T_GUP = range(1, 13)


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.asarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(config: int, tensor: int, step: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config, tensor, step, chunk])))


def _draw(kind: str, n: int, rng: np.random.Generator, p) -> np.ndarray:
    if kind == "normal":
        return rng.standard_normal(n, dtype=np.float32) * np.float32(p["std"])
    if kind == "student_t":
        return rng.standard_t(p["nu"], n).astype(np.float32)
    if kind == "outlier_normal":
        v = rng.standard_normal(n, dtype=np.float32)
        hit = rng.random(n) < p["rate"]
        return np.where(hit, v * np.float32(p["mult"]), v).astype(np.float32)
    raise ValueError(kind)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def sample(kind: str, shape, config: int, tensor: int, step: int = 0, **p) -> np.ndarray:
    """Seeded float32 samples of ``kind`` ('normal', 'student_t', 'outlier_normal')."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    starts = list(range(0, n, CHUNK))

    def fill(ci_s):
        ci, s = ci_s
        m = min(CHUNK, n - s)
        out[s:s + m] = _draw(kind, m, _rng(config, tensor, step, ci), p)

    if len(starts) <= 1:
        for item in enumerate(starts):
            fill(item)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, enumerate(starts)))
    return out.reshape(shape)


def bf16_tensor(kind: str, shape, config: int, tensor: int, step: int = 0, **p) -> np.ndarray:
    """Seeded bf16 bit patterns (uint16) of the given shape and distribution."""
    return f32_to_bf16(sample(kind, shape, config, tensor, step, **p))


def drift(w_bits: np.ndarray, config: int, step: int, std: float) -> np.ndarray:
    """Weight drift between steps: ``bf16(float32(W) + N(0, std))``."""
    d = sample("normal", w_bits.shape, config, T_DRIFT, step, std=std)
    return f32_to_bf16(bf16_to_f32(w_bits) + d)


def varlen_lengths(config: int, count: int = 64, lo: int = 32, hi: int = 2048) -> np.ndarray:
    """Sequence lengths uniform on the integers [lo, hi] (packed THD batch)."""
    return _rng(config, T_LENS, 0, 0).integers(lo, hi + 1, size=count)


# ---------------------------------------------------------------- configurations
CONFIGS = {
    1: dict(name="single fp8 linear forward, current tensorwise scaling",
            M=64, K=128, N=128, x=("normal", dict(std=1.0)), w=("normal", dict(std=1.0)),
            scaling="current"),
    2: dict(name="fp8 linear fwd+dgrad+wgrad, 32 steps of delayed scaling",
            M=4096, K=4096, N=4096, x=("normal", dict(std=1.0)), w=("normal", dict(std=0.02)),
            g=("normal", dict(std=1e-3)), drift=1e-4, steps=32, scaling="delayed"),
    3: dict(name="Llama-8B-shaped MLP block (gate, up, down), fwd+bwd",
            M=8192, K=4096, N=14336, x=("student_t", dict(nu=3)), w=("normal", dict(std=0.02)),
            g=("normal", dict(std=1e-3)), scaling="delayed"),
    4: dict(name="packed THD varlen batch padded to a multiple of 16, K=N=4096",
            K=4096, N=4096, seqs=64, len_lo=32, len_hi=2048, x=("normal", dict(std=1.0)),
            w=("normal", dict(std=0.02)), g=("normal", dict(std=1e-3)), scaling="delayed"),
    5: dict(name="block-scaled recipe (1x128 activations, 128x128 weights)",
            M=16384, K=8192, N=8192, x=("outlier_normal", dict(rate=0.01, mult=100.0)),
            w=("outlier_normal", dict(rate=0.01, mult=100.0)),
            g=("outlier_normal", dict(rate=0.01, mult=100.0)), scaling="block"),
}


def linear_inputs(config: int, step: int = 0, M: int | None = None, K: int | None = None,
                  N: int | None = None, rows: int | None = None):
    """x [rows, K], W [N, K], g [rows, N] (bf16 bits) for configs 1, 2, 4, 5.

    ``M``/``K``/``N`` override the configuration's sizes (small parity cases use
    the same distributions at smaller shapes). ``rows`` is the row count drawn
    for x and g (defaults to M).
    """
    c = CONFIGS[config]
    M = c.get("M") if M is None else M
    K = c["K"] if K is None else K
    N = c["N"] if N is None else N
    rows = M if rows is None else rows
    xk, xp = c["x"]
    wk, wp = c["w"]
    out = dict(x=bf16_tensor(xk, (rows, K), config, T_X, step, **xp),
               w=bf16_tensor(wk, (N, K), config, T_W, 0, **wp))
    if "g" in c:
        gk, gp = c["g"]
        out["g"] = bf16_tensor(gk, (rows, N), config, T_G, step, **gp)
    return out


def mlp_inputs(config: int = 3, M: int | None = None, K: int | None = None, N: int | None = None):
    """Config 3's block: x, h (down's input), the three weights and the three output grads."""
    c = CONFIGS[config]
    M = c["M"] if M is None else M
    K = c["K"] if K is None else K
    N = c["N"] if N is None else N
    xk, xp = c["x"]
    wk, wp = c["w"]
    gk, gp = c["g"]
    return dict(
        x=bf16_tensor(xk, (M, K), config, T_X, 0, **xp),
        h=bf16_tensor(xk, (M, N), config, T_H, 0, **xp),
        w_gate=bf16_tensor(wk, (N, K), config, T_WGATE, 0, **wp),
        w_up=bf16_tensor(wk, (N, K), config, T_WUP, 0, **wp),
        w_down=bf16_tensor(wk, (K, N), config, T_WDOWN, 0, **wp),
        g_gate=bf16_tensor(gk, (M, N), config, T_GGATE, 0, **gp),
        g_up=bf16_tensor(gk, (M, N), config, T_GUP, 0, **gp),
        g_down=bf16_tensor(gk, (M, K), config, T_GDOWN, 0, **gp),
    )


def varlen_batch(config: int = 4, K: int | None = None, N: int | None = None, step: int = 0,
                 count: int | None = None, len_hi: int | None = None):
    """Config 4: lengths, T = sum, and x [T, K], g [T, N], W [N, K] (bf16 bits)."""
    c = CONFIGS[config]
    K = c["K"] if K is None else K
    N = c["N"] if N is None else N
    lens = varlen_lengths(config, c["seqs"] if count is None else count, c["len_lo"],
                          c["len_hi"] if len_hi is None else len_hi)
    T = int(lens.sum())
    d = linear_inputs(config, step, M=T, K=K, N=N)
    d["lens"] = lens
    d["T"] = T
    return d
