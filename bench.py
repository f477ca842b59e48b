"""Benchmark: fp8 linear fwd+bwd TFLOP/s at 8192x4096x14336, and quantize+amax GB/s.

One step is one pass of the whole hot path over the Llama-8B-shaped MLP block
(tokens M = 8192; gate and up: K = 4096 -> N = 14336; down: 14336 -> 4096):
for each of the three linears the weight is quantized (with its amax recorded
in the 16-entry ring), the input is quantized with its delayed scale, the
forward GEMM runs, then the gradient is quantized and dgrad and wgrad run, and
the delayed scales are updated; the token count goes through the padding check
(8192 is already a multiple of 16, so no rows are added). Inputs are seeded
synthetic tensors already resident in HBM: activations Student-t(3), weights
N(0, 0.02), output gradients N(0, 1e-3). Timing: W untimed warm-up steps
(steady state of delayed scaling), then K steps between two device
synchronizations with nothing recorded in between (the headline); then the
same K steps again with HIP events around every kernel call, which give the
per-launch durations for the roofline figures.

Prints ONE JSON line. ``--gpus N`` with N > 1 exits: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the block-recipe and packed-varlen measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 512 MiB buffer three times (for scaling HBM byte counters)")
    ap.add_argument("--data-sensitivity", action="store_true",
                    help="only time one GEMM shape on random, constant and zero codes")
    ap.add_argument("--shape", default="8192,4096,14336",
                    help="M,N,K of the --data-sensitivity GEMM")
    ap.add_argument("--profile-gemms", action="store_true",
                    help="only run every GEMM launch shape of the step and of the block recipe "
                         "(5 launches each after 2 warm-up launches), for counter collection")
    ap.add_argument("--compare-hipblaslt", action="store_true",
                    help="only run each tensorwise GEMM launch shape of the step with this "
                         "library and with torch._scaled_mm (hipBLASLt) on the same codes: "
                         "bytes compared, 40 launches of each, for a kernel trace")
    return ap.parse_args()


def copy_calibration():
    """A plain device copy of known size: the reference for FETCH_SIZE / WRITE_SIZE."""
    import torch
    nbytes = 512 << 20
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": nbytes,
                                           "bytes_written_per_copy": nbytes, "copies": 3}}))


def data_sensitivity(launches=20, shape=(8192, 4096, 14336)):
    """The same GEMM launch (default M=8192, N=4096, K=14336) on three sets of operand codes: codes
    of normal data (as in the step), all codes 0x38 (1.0) and all codes 0. The instruction
    stream and memory traffic are identical; only the bits the matrix cores and data paths
    toggle differ, so a gap in time is a gap in clock (the chip's power limit)."""
    import torch
    import scaled_fp8_linear_amd as m
    m.load()
    dev = torch.device("cuda:0")
    M, N, K = shape
    gen = torch.Generator(device=dev).manual_seed(0)
    one = torch.ones(1, device=dev)
    res = {}
    for name in ("normal", "constant_1.0", "zeros", "normal_again"):
        if name.startswith("normal"):
            xa = torch.randn(M, K, device=dev, generator=gen).to(torch.bfloat16)
            xb = (torch.randn(N, K, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
            qa = m.fp8_quantize_amax(xa, scale_inv=448.0 / xa.abs().max().float().reshape(1),
                                     want_q_t=False)[0]
            qb = m.fp8_quantize_amax(xb, scale_inv=448.0 / xb.abs().max().float().reshape(1),
                                     want_q_t=False)[0]
            del xa, xb
        else:
            code = 0x38 if name.startswith("constant") else 0
            qa = torch.full((M, K), code, dtype=torch.uint8, device=dev)
            qb = torch.full((N, K), code, dtype=torch.uint8, device=dev)
        y = m.fp8_linear_fwd(qa, qb, one, one)
        for _ in range(3):
            m.fp8_linear_fwd(qa, qb, one, one, y=y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            m.fp8_linear_fwd(qa, qb, one, one, y=y)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / launches
        res[name] = {"us_per_launch": round(us, 1), "tflops": round(2.0 * M * N * K / us / 1e6, 1)}
        print(json.dumps({"data_sensitivity": name, **res[name]}), flush=True)
    print(json.dumps({"data_sensitivity": res, "shape": [M, N, K], "launches": launches}))


def profile_gemms(launches=5, warmup=2):
    """Every GEMM launch shape of the MLP step (tensorwise; the two 256x256-tile shapes and the
    two wgrad shapes with 224-row / 224-column tiles) and the block recipe's forward, dgrad and
    wgrad at M=16384, K=N=8192, on operand codes the library quantizes from N(0,1) data, with a
    scale that keeps the codes spread over the format. One line per shape with the event time
    per launch; meant to run under rocprofv3 counter collection."""
    import torch
    import scaled_fp8_linear_amd as m
    m.load()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(3)

    def codes(rows, cols):
        x = torch.randn(rows, cols, device=dev, generator=gen).to(torch.bfloat16)
        q = m.fp8_quantize_amax(x, scale_inv=torch.full((1,), 64.0, device=dev), want_q_t=False)[0]
        return q

    def timed(name, fn, flops):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(launches):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / launches
        print(json.dumps({"gemm": name, "us_per_launch": round(us, 1),
                          "tflops": round(flops / us / 1e6, 1)}), flush=True)

    one = torch.ones(1, device=dev)
    for M, N, K in ((8192, 14336, 4096), (8192, 4096, 14336), (14336, 4096, 8192),
                    (4096, 14336, 8192)):
        qa, qb = codes(M, K), codes(N, K)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        timed(f"tensorwise {M}x{N}x{K}", lambda: m.fp8_linear_fwd(qa, qb, one, one, y=y),
              2.0 * M * N * K)
        del qa, qb, y
    M, N, K = 16384, 8192, 8192
    B = m.FP8_BLOCK_1x128
    x = torch.randn(M, K, device=dev, generator=gen).to(torch.bfloat16)
    w = torch.randn(N, K, device=dev, generator=gen).to(torch.bfloat16)
    g = torch.randn(M, N, device=dev, generator=gen).to(torch.bfloat16)
    qx, qx_t, _, sx, sx_t = m.fp8_quantize_amax(x, gran=B)
    qw, qw_t, _, sw, sw_t = m.fp8_quantize_amax(w, gran=m.FP8_BLOCK_128x128)
    qg, qg_t, _, sg, sg_t = m.fp8_quantize_amax(g, gran=B)
    del x, w, g
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    f = 2.0 * M * N * K
    timed("block fwd 16384x8192x8192", lambda: m.fp8_linear_fwd(qx, qw, sx, sw, y=y, gran=B), f)
    timed("block dgrad 16384x8192x8192",
          lambda: m.fp8_linear_dgrad(qg, qw_t, sg, sw_t, dx=dx, gran=B), f)
    timed("block wgrad 8192x8192x16384",
          lambda: m.fp8_linear_wgrad(qg_t, qx_t, sg_t, sx_t, dw=dw, gran=B), f)


def compare_hipblaslt(blocks=4, per_block=10, warmup=3):
    """The step's four tensorwise GEMM launch shapes, each run with this library and with
    torch._scaled_mm (hipBLASLt's FP8 GEMM) on the same operand codes (quantized by the library
    from N(0, 1) and N(0, 0.02) data with the scales their amaxes give), in alternating blocks
    of launches so that neither meets a different clock. Prints, per shape, how many output
    elements differ in their bytes and the mean event time per launch of each; meant to run
    under a kernel trace as well."""
    import torch
    import scaled_fp8_linear_amd as m
    m.load()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(5)

    def block_us(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(per_block):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / per_block

    for M, N, K in ((8192, 14336, 4096), (8192, 4096, 14336), (14336, 4096, 8192),
                    (4096, 14336, 8192)):
        xa = torch.randn(M, K, device=dev, generator=gen).to(torch.bfloat16)
        xb = (torch.randn(N, K, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
        amax_a, amax_b = xa.abs().max().float(), xb.abs().max().float()
        sa, sb = (amax_a / 448).reshape(1), (amax_b / 448).reshape(1)
        qa = m.fp8_quantize_amax(xa, scale_inv=(448 / amax_a).reshape(1), want_q_t=False)[0]
        qb = m.fp8_quantize_amax(xb, scale_inv=(448 / amax_b).reshape(1), want_q_t=False)[0]
        del xa, xb
        fa, fb = qa.view(torch.float8_e4m3fn), qb.view(torch.float8_e4m3fn)
        y = m.fp8_linear_fwd(qa, qb, sa, sb)
        r = torch._scaled_mm(fa, fb.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        differ = int((y.view(torch.int16) != r.view(torch.int16)).sum())
        run = {"fp8lin": lambda: m.fp8_linear_fwd(qa, qb, sa, sb, y=y),
               "hipblaslt": lambda: torch._scaled_mm(fa, fb.t(), scale_a=sa, scale_b=sb,
                                                     out_dtype=torch.bfloat16)}
        for fn in run.values():
            for _ in range(warmup):
                fn()
        us = {k: 0.0 for k in run}
        for b in range(blocks):
            for k in (("fp8lin", "hipblaslt") if b % 2 == 0 else ("hipblaslt", "fp8lin")):
                us[k] += block_us(run[k]) / blocks
        ours, theirs = us["fp8lin"], us["hipblaslt"]
        print(json.dumps({"shape": [M, N, K], "elements": M * N, "elements_differing": differ,
                          "fp8lin_us": round(ours, 1), "hipblaslt_us": round(theirs, 1)}),
              flush=True)
        del qa, qb, fa, fb, y, r


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_mlp_8192x4096x14336.txt")


def source_digest(paths):
    """sha256 (first 16 hex digits) of C/HIP sources with comments and blank lines removed,
    so that an edit of comments alone keeps the digest while any change of code alters it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in paths:
        text = open(os.path.join(ROOT, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def counter_traffic(kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, scaled by the copy calibration; None when the summary is missing or the kernel's
    code (its sources without comments) has changed since the counters were taken."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    for block in text.split("\n\n"):
        kv = {}
        for ln in block.splitlines():
            if ln and not ln.startswith("#"):
                k, _, v = ln.partition(" ")
                kv[k] = v.strip()
        if kv.get("kernel") != kernel:
            continue
        try:
            digest = source_digest(kv["sources"].split())
        except OSError:
            return None
        if digest != kv["code_sha256"]:
            return None
        rd = float(kv["fetch_kib_mean"]) * float(kv["fetch_factor"]) * 1024
        wr = float(kv["write_kib_mean"]) * float(kv["write_factor"]) * 1024
        return {"bytes": int(rd + wr), "read_bytes": int(rd), "write_bytes": int(wr)}
    return None


class EventProbe:
    """Records a pair of HIP events (on the current stream) around each tagged kernel call."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}
        self.active = False
        self._tag = None

    def __call__(self, tag):
        self._tag = tag
        return self

    def __enter__(self):
        if self.active:
            e = self.torch.cuda.Event(enable_timing=True)
            e.record()
            self.pairs.setdefault(self._tag, []).append([e, None])
        return self

    def __exit__(self, *exc):
        if self.active:
            e = self.torch.cuda.Event(enable_timing=True)
            e.record()
            self.pairs[self._tag][-1][1] = e
        return False

    def durations_ms(self, tag):
        return [a.elapsed_time(b) for a, b in self.pairs.get(tag, [])]


def _oracle_quantize_slabs(bits, scale_inv, pool, slabs):
    """The oracle's tensorwise quantize of a bf16 [rows, cols] tensor, cut into row slabs
    that run on a thread pool (numpy releases the GIL inside its array operations); the
    transposed copy is put together from the slabs' transposes."""
    from oracle.quantize import quantize_tensorwise
    rows = bits.shape[0]
    bounds = np.linspace(0, rows, slabs + 1).astype(int)
    parts = list(pool.map(lambda i: quantize_tensorwise(bits[bounds[i]:bounds[i + 1]], scale_inv),
                          range(slabs)))
    q = np.concatenate([p[0] for p in parts])
    q_t = np.concatenate([p[1] for p in parts], axis=1)
    return q, q_t


def cpu_baseline(sample_tokens: int) -> dict:
    """The CPU oracle, as it is, on the benchmark's own step: the three linears of the MLP
    block (gate, up: 4096 -> 14336; down: 14336 -> 4096), each with amax, scale and quantize
    of its input, weight and output gradient (the oracle's quantize on row slabs, one per
    host core, in threads) and forward, dgrad and wgrad in float64 through numpy's BLAS.
    ``sample_tokens`` below 8192 restricts every linear to that many tokens and scales the
    time linearly (for slow hosts); at 8192 nothing is extrapolated.
    """
    from concurrent.futures import ThreadPoolExecutor

    import workloads
    from oracle import gemm
    from oracle.quantize import amax as o_amax
    from oracle.scaling import scale_from_amax

    M, K, N = 8192, 4096, 14336
    S = min(sample_tokens, M)
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = cores
    ST, W02, G13 = dict(nu=3), dict(std=0.02), dict(std=1e-3)
    linears = {   # x, W, g of each linear, drawn as the GPU step draws them
        "gate": (("student_t", (S, K), workloads.T_X, ST), ("normal", (N, K), workloads.T_WGATE, W02),
                 ("normal", (S, N), workloads.T_GGATE, G13)),
        "up": (("student_t", (S, K), workloads.T_X, ST), ("normal", (N, K), workloads.T_WUP, W02),
               ("normal", (S, N), workloads.T_GUP, G13)),
        "down": (("student_t", (S, N), workloads.T_H, ST), ("normal", (K, N), workloads.T_WDOWN, W02),
                 ("normal", (S, K), workloads.T_GDOWN, G13)),
    }
    t_q = t_g = 0.0
    elems = 0
    with ThreadPoolExecutor(cores) as pool:
        for spec in linears.values():
            bits = [workloads.bf16_tensor(kind, shape, 3, tid, 0, **p)
                    for kind, shape, tid, p in spec]
            t0 = time.perf_counter()
            qs = []
            for b in bits:
                s_, si = scale_from_amax(o_amax(b))
                qs.append((s_,) + _oracle_quantize_slabs(b, si, pool, cores))
                elems += b.size
            t_q += time.perf_counter() - t0
            (sx, qx, qx_t), (sw, qw, qw_t), (sg, qg, qg_t) = qs
            t0 = time.perf_counter()
            gemm.scaled_gemm(qx, qw, sx, sw)            # forward, contraction over inputs
            gemm.scaled_gemm(qg, qw_t, sg, sw)          # dgrad, contraction over outputs
            gemm.scaled_gemm(qg_t, qx_t, sg, sx)        # wgrad, contraction over tokens
            t_g += time.perf_counter() - t0
            del bits, qs
    t_step = (t_q + t_g) * (M / S)
    flops = 3 * 6.0 * M * N * K
    return {"value": round(flops / t_step / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(max(cores, blas_threads)), "kind": "oracle",
            "affinity_cores": cores, "blas_threads": int(blas_threads), "quantize_threads": cores,
            "quantize_gbs": round(4.0 * elems / t_q / 1e9, 3),
            "gemm_gflops": round(3 * 3 * 2.0 * S * N * K / t_g / 1e9, 1),
            "sample": (f"the whole step on {S} of {M} tokens: quantize of x, W, g of the 3 "
                       f"linears (oracle, {cores} row slabs on {cores} threads) and their fwd, "
                       f"dgrad, wgrad in float64 (BLAS, {blas_threads} threads); measured "
                       f"{t_q + t_g:.1f} s (quantize {t_q:.1f} s, GEMMs {t_g:.1f} s)"
                       + ("" if S == M else f", scaled x{M / S:g} to the full step"))}


def _time_steps(torch, step, steps, warmup):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def measure_config1(torch, m, workloads, iters=200, repeats=7):
    """Config 1: one fp8 linear forward with current tensorwise scaling, x [64, 128],
    W [128, 128], N(0, 1): for each operand an amax pass, the scale from that amax (no
    delay), the cast with it; then the GEMM (7 launches). Latency per forward, as launched
    eagerly from Python and as one captured HIP graph (replayed; checked byte for byte
    against the eager result)."""
    d = workloads.linear_inputs(1)
    dev = torch.device("cuda:0")

    def up(b):
        return torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)

    x, w = up(d["x"]), up(d["w"])
    f32 = dict(dtype=torch.float32, device=dev)
    amax = {n: torch.zeros(1, **f32) for n in "xw"}
    sc = {n: torch.ones(1, **f32) for n in "xw"}
    si = {n: torch.ones(1, **f32) for n in "xw"}
    q = {"x": torch.empty((64, 128), dtype=torch.uint8, device=dev),
         "w": torch.empty((128, 128), dtype=torch.uint8, device=dev)}
    y = torch.empty((64, 128), dtype=torch.bfloat16, device=dev)
    src = {"x": x, "w": w}

    def forward():
        for n in "xw":
            # amax folded into a cleared buffer; the scale update reads it and clears it
            m.fp8_quantize_amax(src[n], amax=amax[n], amax_accumulate=True, want_q=False,
                                want_q_t=False)
            m.fp8_scale_update(m.FP8_SCALE_FROM_AMAX, amax=amax[n], scale=sc[n],
                               scale_inv=si[n], clear_amax=True)
            m.fp8_quantize_amax(src[n], scale_inv=si[n], q=q[n], want_q_t=False,
                                want_amax=False)
        m.fp8_linear_fwd(q["x"], q["w"], sc["x"], sc["w"], y=y)

    def per_call_us(fn, iters=iters):
        for _ in range(20):
            fn()
        out = []
        for _ in range(repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3 / iters)
        return float(np.median(out))

    eager_us = per_call_us(forward)
    ref = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        forward()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        forward()
    y.zero_()
    graph.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(y.view(torch.int16), ref.view(torch.int16)))
    graph_us = per_call_us(graph.replay)
    # the same forward as one launch (amaxes, scales, casts and GEMM, one workgroup per tile)
    y1 = torch.empty((64, 128), dtype=torch.bfloat16, device=dev)
    sc1 = torch.empty(4, **f32)
    q1 = {"x": torch.empty((64, 128), dtype=torch.uint8, device=dev),
          "w": torch.empty((128, 128), dtype=torch.uint8, device=dev)}

    def fused():
        m.fp8_linear_fwd_current(x, w, y=y1, scales=sc1, qx=q1["x"], qw=q1["w"])

    fused_us = per_call_us(fused)
    torch.cuda.synchronize()
    fused_same = bool(torch.equal(q1["x"], q["x"]) and torch.equal(q1["w"], q["w"]) and
                      torch.equal(sc1[:2], torch.cat([sc["x"], sc["w"]])) and
                      torch.equal(sc1[2:], torch.cat([si["x"], si["w"]])))
    gf = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fused()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(gf):
        fused()
    fused_graph_us = per_call_us(gf.replay)
    # GPU time per forward: one graph of back-to-back forwards, so neither the host nor a
    # replay's own start is in the figure
    chain = 32
    gc = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gc):
        for _ in range(chain):
            fused()
    chain_us = per_call_us(gc.replay, iters=20) / chain
    flops = 2.0 * 64 * 128 * 128
    return {"workload": "one fp8 linear forward, current tensorwise scaling, x [64,128], "
                        "W [128,128] N(0,1): amax pass, scale, cast for x and W, then the GEMM",
            "launches": 7, "us_per_forward_eager": round(eager_us, 2),
            "us_per_forward_hip_graph": round(graph_us, 2),
            "graph_matches_eager": same,
            "gflops_hip_graph": round(flops / (graph_us * 1e-6) / 1e9, 2),
            "one_launch": {"entry": "fp8_linear_fwd_current",
                           "us_per_forward_eager": round(fused_us, 2),
                           "us_per_forward_hip_graph": round(fused_graph_us, 2),
                           "us_per_forward_gpu": round(chain_us, 2),
                           "gpu_time_of": f"one HIP graph of {chain} forwards back to back",
                           "codes_and_scales_match_seven_launches": fused_same,
                           "gflops_hip_graph": round(flops / (fused_graph_us * 1e-6) / 1e9, 2)}}


def measure_config2(torch, m, repeats=5):
    """Config 2: fp8 linear fwd + dgrad + wgrad at M = K = N = 4096 for 32 steps of delayed
    scaling (16-step weight amax ring, one-step-delayed activation and gradient scales):
    x ~ N(0,1) and g ~ N(0,1e-3) fresh every step, W ~ N(0,0.02) drifting by N(0,1e-4) per
    step; every step's tensors are resident in HBM before timing (drawn on the device).
    Each repeat runs the 32 steps from a fresh schedule; the median repeat is reported."""
    M = K = N = 4096
    steps = 32
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(2)
    bf = dict(dtype=torch.bfloat16, device=dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    xs = [torch.randn(M, K, device=dev, generator=gen).to(torch.bfloat16) for _ in range(steps)]
    gs = [(torch.randn(M, N, device=dev, generator=gen) * 1e-3).to(torch.bfloat16)
          for _ in range(steps)]
    ws = [(torch.randn(N, K, device=dev, generator=gen) * 0.02).to(torch.bfloat16)]
    for _ in range(steps - 1):
        ws.append((ws[-1].float() + torch.randn(N, K, device=dev, generator=gen) * 1e-4)
                  .to(torch.bfloat16))
    bufs = dict(qw=torch.empty((N, K), **u8), qw_t=torch.empty((K, N), **u8),
                qx=torch.empty((M, K), **u8), qx_t=torch.empty((K, M), **u8),
                qg=torch.empty((M, N), **u8), qg_t=torch.empty((N, M), **u8))
    y, dx, dw = (torch.empty((M, N), **bf), torch.empty((M, K), **bf),
                 torch.empty((N, K), **bf))

    def run(lin):
        for t in range(steps):
            lin.begin_step()
            lin.forward(xs[t], ws[t], out=y, bufs=bufs)
            lin.backward(gs[t], dx=dx, dw=dw, bufs=bufs)
            lin.end_step()

    run(m.DelayedScalingLinear(dev))                      # warm-up
    times = []
    for _ in range(repeats):
        lin = m.DelayedScalingLinear(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        run(lin)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    flops = steps * 6.0 * M * N * K
    return {"workload": "fp8 linear fwd+dgrad+wgrad, M=K=N=4096, 32 steps of delayed scaling, "
                        "x N(0,1), W N(0,0.02) drifting N(0,1e-4), g N(0,1e-3)",
            "steps": steps, "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "ms_per_32_steps": round(ms, 4), "ms_per_step": round(ms / steps, 4),
            "repeats": repeats}


def measure_bf16_step(torch, fp8_ms, steps=10, warmup=3):
    """The same nine GEMMs of the MLP step in bf16 through torch (hipBLASLt), for context
    beside the pages' expectation of about 2x from FP8 over bf16 when compute-bound: no
    quantize, no scales, bf16 in and out, float32 accumulation. Right operands are
    contiguous (the forward takes W^T stored as such); the wgrad's left operand is the
    transposed view of g. Inputs are random bf16 of the step's shapes."""
    M, K, N = 8192, 4096, 14336
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(9)

    def r(*shape):
        return torch.randn(*shape, device=dev, generator=gen).to(torch.bfloat16)

    x, h = r(M, K), r(M, N)
    wg, wu, wd = r(N, K), r(N, K), r(K, N)
    wgt, wut, wdt = wg.t().contiguous(), wu.t().contiguous(), wd.t().contiguous()
    gg, gu, gd = r(M, N), r(M, N), r(M, K)

    def e(*shape):
        return torch.empty(*shape, dtype=torch.bfloat16, device=dev)

    yg, yu, yd = e(M, N), e(M, N), e(M, K)
    dxg, dxu, dh = e(M, K), e(M, K), e(M, N)
    dwg, dwu, dwd = e(N, K), e(N, K), e(K, N)

    def step():
        torch.mm(x, wgt, out=yg)
        torch.mm(x, wut, out=yu)
        torch.mm(h, wdt, out=yd)
        torch.mm(gg, wg, out=dxg)
        torch.mm(gu, wu, out=dxu)
        torch.mm(gd, wd, out=dh)
        torch.mm(gg.t(), x, out=dwg)
        torch.mm(gu.t(), x, out=dwu)
        torch.mm(gd.t(), h, out=dwd)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    flops = 18.0 * M * N * K
    return {"workload": "the MLP step's nine GEMMs in bf16 (torch.mm, hipBLASLt), no quantize",
            "ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / 2500.0, 4),
            "fp8_step_speedup": round(ms / fp8_ms, 3), "steps": steps}


def measure_quantize_vs_copy(torch, m, reps=5):
    """The quantize pass on every tensor shape of the step (and the packed varlen batch),
    beside a copy of the same bytes at the same access width: the library's padding kernel
    copying the bf16 tensor into a second buffer (2 B read and 2 B written per element,
    16-byte loads and stores), which is the rate an HBM stream of this mix reaches on the
    box. Buffers rotate through enough sets (at least 1.5 GB) that no launch finds its
    data in the 256 MB Infinity Cache."""
    import math
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(7)
    out = {}
    for name, (rows, cols) in (("x", (8192, 4096)), ("w_gate_up", (14336, 4096)),
                               ("w_down", (4096, 14336)), ("g_gate_up_and_h", (8192, 14336)),
                               ("varlen_54672", (54672, 4096))):
        per_set = 4 * rows * cols
        sets = max(2, math.ceil(1.5e9 / per_set))
        xs = [torch.randn(rows, cols, device=dev, generator=gen).to(torch.bfloat16)
              for _ in range(sets)]
        si = torch.full((1,), 64.0, device=dev)
        amax = torch.zeros(1, device=dev)
        qs = [torch.empty((rows, cols), dtype=torch.uint8, device=dev) for _ in range(sets)]
        qts = [torch.empty((cols, rows), dtype=torch.uint8, device=dev) for _ in range(sets)]
        ds = [torch.empty_like(t) for t in xs]

        def timed(fn):
            for i in range(sets):
                fn(i)
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(3):
                    for i in range(sets):
                        fn(i)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / (3 * sets))
            return float(np.median(ts))

        q_us = timed(lambda i: m.fp8_quantize_amax(xs[i], scale_inv=si, q=qs[i], q_t=qts[i],
                                                   amax=amax, amax_accumulate=True))
        c_us = timed(lambda i: m.fp8_pad_tokens(xs[i], x_pad=ds[i]))
        out[name] = {"shape": [rows, cols], "quantize_us": round(q_us, 2),
                     "quantize_tbs": round(per_set / q_us / 1e6, 3),
                     "copy_us": round(c_us, 2), "copy_tbs": round(per_set / c_us / 1e6, 3),
                     "quantize_over_copy": round(c_us / q_us, 3)}
        del xs, qs, qts, ds
        torch.cuda.empty_cache()
    return out


def measure_block_recipe(torch, m, workloads, steps, warmup):
    """Block recipe (1x128 activation/gradient tiles, 128x128 weight tiles, current
    scaling) at M=16384, K=N=8192: quantize x, W, g and the three GEMMs per step."""
    M, K, N = 16384, 8192, 8192
    d = workloads.linear_inputs(5, 0)
    dev = torch.device("cuda:0")

    def up(b):
        return torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)

    x, w, g = up(d["x"]), up(d["w"]), up(d["g"])
    del d
    B, W128 = m.FP8_BLOCK_1x128, m.FP8_BLOCK_128x128
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    buf = dict(qx=torch.empty((M, K), **u8), qxt=torch.empty((K, M), **u8),
               sx=torch.empty((M, K // 128), **f32), sxt=torch.empty((K, M // 128), **f32),
               qw=torch.empty((N, K), **u8), qwt=torch.empty((K, N), **u8),
               sw=torch.empty((N // 128, K // 128), **f32), swt=torch.empty((K // 128, N // 128), **f32),
               qg=torch.empty((M, N), **u8), qgt=torch.empty((N, M), **u8),
               sg=torch.empty((M, N // 128), **f32), sgt=torch.empty((N, M // 128), **f32),
               y=torch.empty((M, N), **bf), dx=torch.empty((M, K), **bf), dw=torch.empty((N, K), **bf))
    gemm_ev, q_ev = [], []
    instrument = [False]

    def ev(lst, fn):
        if not instrument[0]:
            fn()
            return
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        lst.append((a, b))

    def step():
        b = buf
        ev(q_ev, lambda: m.fp8_quantize_amax(x, gran=B, q=b["qx"], q_t=b["qxt"], scale=b["sx"],
                                             scale_t=b["sxt"], want_amax=False))
        ev(q_ev, lambda: m.fp8_quantize_amax(w, gran=W128, q=b["qw"], q_t=b["qwt"], scale=b["sw"],
                                             scale_t=b["swt"], want_amax=False))
        ev(q_ev, lambda: m.fp8_quantize_amax(g, gran=B, q=b["qg"], q_t=b["qgt"], scale=b["sg"],
                                             scale_t=b["sgt"], want_amax=False))
        ev(gemm_ev, lambda: m.fp8_linear_fwd(b["qx"], b["qw"], b["sx"], b["sw"], y=b["y"], gran=B))
        ev(gemm_ev, lambda: m.fp8_linear_dgrad(b["qg"], b["qwt"], b["sg"], b["swt"], dx=b["dx"],
                                               gran=B))
        ev(gemm_ev, lambda: m.fp8_linear_wgrad(b["qgt"], b["qxt"], b["sgt"], b["sxt"], dw=b["dw"],
                                               gran=B))

    ms = _time_steps(torch, step, steps, warmup)      # uninstrumented
    instrument[0] = True                               # then per-call HIP events
    _time_steps(torch, step, steps, 0)
    gemm_ev, q_ev = gemm_ev[-3 * steps:], q_ev[-3 * steps:]
    g_ms = [a.elapsed_time(b) for a, b in gemm_ev]
    q_ms = [a.elapsed_time(b) for a, b in q_ev]
    flops = 6.0 * M * N * K
    q_bytes = 4 * (M * K + N * K + M * N)        # bf16 in, codes + transposed codes out
    return {"workload": "block recipe linear fwd+dgrad+wgrad, M=16384 K=N=8192, N(0,1) with 1% x100",
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1), "ms_per_step": round(ms, 4),
            "gemm_tflops_per_launch": round(2.0 * M * N * K / (np.mean(g_ms) * 1e-3) / 1e12, 1),
            "gemm_frac_of_fp8_peak": round(2.0 * M * N * K / (np.mean(g_ms) * 1e-3) / 1e12
                                           / PEAK_FP8_TFLOPS, 4),
            "quantize_gbs": round(q_bytes / (np.sum(q_ms) / steps * 1e-3) / 1e9, 1),
            "quantize_frac_of_hbm_peak": round(q_bytes / (np.sum(q_ms) / steps * 1e-3) / 1e9
                                               / PEAK_HBM_GBS, 4)}


def measure_varlen(torch, m, workloads, steps, warmup):
    """Packed varlen batch: 64 sequences of U{32..2048} tokens, padded to a multiple of 16,
    K = N = 4096, one linear fwd+bwd with delayed scaling and rows_valid = T."""
    d = workloads.varlen_batch(4)
    T = d["T"]
    dev = torch.device("cuda:0")

    def up(b):
        return torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)

    x, w, g = up(d["x"]), up(d["w"]), up(d["g"])
    del d
    _, T_pad = m.fp8_pad_tokens(x, query_only=True)
    xp = torch.empty((T_pad, x.shape[1]), dtype=x.dtype, device=dev)
    gp = torch.empty((T_pad, g.shape[1]), dtype=g.dtype, device=dev)
    # the packed batches as a loader would hand them over: in buffers with room for T_pad
    # rows, the tail holding whatever was there before
    xb = torch.full((T_pad, x.shape[1]), float("nan"), dtype=x.dtype, device=dev)
    gb = torch.full((T_pad, g.shape[1]), float("nan"), dtype=g.dtype, device=dev)
    xb[:T].copy_(x)
    gb[:T].copy_(g)
    lin = m.DelayedScalingLinear(dev)

    def step_in_place():
        m.fp8_pad_tokens(xb, T=T, x_pad=xb)         # zero rows [T, T_pad) of the batch
        m.fp8_pad_tokens(gb, T=T, x_pad=gb)
        lin.begin_step()
        lin.forward(xb, w, rows_valid=T)
        lin.backward(gb)
        lin.end_step()

    def step_copy():
        m.fp8_pad_tokens(x, x_pad=xp)               # copy [T] rows into a [T_pad] buffer
        m.fp8_pad_tokens(g, x_pad=gp)
        lin.begin_step()
        lin.forward(xp, w, rows_valid=T)
        lin.backward(gp)
        lin.end_step()

    ms = _time_steps(torch, step_in_place, steps, warmup)
    ms_copy = _time_steps(torch, step_copy, steps, warmup)
    flops = 6.0 * T_pad * 4096 * 4096

    # per-sequence alignment for tp = cp = 2 (THD): every sequence to a multiple of 4, the
    # batch to a multiple of 64; pad and unpad timed per launch with HIP events
    sm, tm = m.fp8_align_multiple(m.FP8_LAYOUT_THD, 1, 2, 2)
    lens = workloads.varlen_lengths(4)
    cu = np.concatenate([[0], np.cumsum(lens)])
    _, cu_pad, T_al = m.fp8_pad_varlen(x, cu, sm, tm, query_only=True)
    xa = torch.empty((T_al, x.shape[1]), dtype=x.dtype, device=dev)
    xu = torch.empty_like(x)

    def per_launch_ms(fn, n=20):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    pad_ms = per_launch_ms(lambda: m.fp8_pad_varlen(x, cu, sm, tm, x_pad=xa))
    unpad_ms = per_launch_ms(lambda: m.fp8_unpad_varlen(xa, cu, cu_pad, x=xu))
    cols = x.shape[1]
    pad_bytes = 2 * T * cols + 2 * T_al * cols
    unpad_bytes = 4 * T * cols
    return {"workload": "packed THD batch, 64 seqs U{32..2048}, K=N=4096, delayed scaling",
            "tokens": T, "tokens_padded": T_pad, "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "ms_per_step": round(ms, 4), "padding": "in place (tail rows of the batch zeroed)",
            "ms_per_step_padding_by_copy": round(ms_copy, 4),
            "per_sequence_alignment": {
                "rule": "THD, tp = cp = 2: each sequence to a multiple of %d, the batch to %d"
                        % (sm, tm),
                "tokens_aligned": T_al,
                "pad_us": round(pad_ms * 1e3, 1),
                "pad_gbs": round(pad_bytes / (pad_ms * 1e-3) / 1e9, 1),
                "unpad_us": round(unpad_ms * 1e3, 1),
                "unpad_gbs": round(unpad_bytes / (unpad_ms * 1e-3) / 1e9, 1)}}


def measure_f1(torch, m, steps, warmup):
    """The autograd wrapper with bias at the gate linear's shape (tokens 8192, 4096 -> 14336):
    the forward GEMM with and without the bias epilogue (HIP events per launch), the bias
    gradient pass (GB/s), and whole Fp8Linear fwd+bwd steps through torch.autograd."""
    M, K, N = 8192, 4096, 14336
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(1)
    x = torch.randn(M, K, device=dev, generator=gen).to(torch.bfloat16)
    g = (torch.randn(M, N, device=dev, generator=gen) * 1e-3).to(torch.bfloat16)
    layer = m.Fp8Linear(K, N, bias=True, device=dev)
    qx = m.fp8_quantize_amax(x, scale_inv=torch.ones(1, device=dev), want_q_t=False)[0]
    qw = m.fp8_quantize_amax(layer.weight.detach(), scale_inv=torch.full((1,), 64.0, device=dev),
                             want_q_t=False)[0]
    one = torch.ones(1, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    b = layer.bias.detach()

    def per_launch_us(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for a, c in ev:
            a.record()
            fn()
            c.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(c) for a, c in ev])) * 1e3

    us_plain = per_launch_us(lambda: m.fp8_linear_fwd(qx, qw, one, one, y=y), steps)
    us_bias = per_launch_us(lambda: m.fp8_linear_fwd(qx, qw, one, one, y=y, bias=b), steps)
    db = torch.empty(N, dtype=torch.bfloat16, device=dev)
    us_db = per_launch_us(lambda: m.fp8_bias_grad(g, db=db), steps)

    m.fp8_state().reset()
    xr = x.detach().requires_grad_(True)

    def step():
        layer.weight.grad = None
        layer.bias.grad = None
        xr.grad = None
        with m.fp8_autocast():
            out = layer(xr)
        out.backward(g)

    ms = _time_steps(torch, step, steps, warmup)
    m.fp8_state().reset()
    flops = 6.0 * M * N * K
    return {"workload": "Fp8Linear(4096 -> 14336, bias) fwd+bwd through torch.autograd, tokens 8192",
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1), "ms_per_step": round(ms, 4),
            "fwd_gemm_us": round(us_plain, 1), "fwd_gemm_with_bias_us": round(us_bias, 1),
            "bias_epilogue_overhead": round(us_bias / us_plain - 1.0, 4),
            "bias_grad_us": round(us_db, 1),
            "bias_grad_gbs": round(2.0 * M * N / (us_db * 1e-6) / 1e9, 1),
            "bias_grad_frac_of_hbm_peak": round(2.0 * M * N / (us_db * 1e-6) / 1e9 / PEAK_HBM_GBS,
                                                4)}


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "bench.py measures one GPU: the hot path runs on one "
                                   "device and has no cross-GPU step; run with --gpus 1"}))
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.data_sensitivity:
        data_sensitivity(shape=tuple(int(v) for v in args.shape.split(",")))
        return
    if args.profile_gemms:
        profile_gemms()
        return
    if args.compare_hipblaslt:
        compare_hipblaslt()
        return

    import torch

    import scaled_fp8_linear_amd as m
    import workloads

    m.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    M, K, N = 8192, 4096, 14336

    host = workloads.mlp_inputs(3)

    def up(b):
        return torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)

    t = {k: up(v) for k, v in host.items()}
    del host
    probe = EventProbe(torch)
    lins = {n: m.DelayedScalingLinear(dev, probe=probe) for n in ("gate", "up", "down")}
    shapes = {"gate": (K, N), "up": (K, N), "down": (N, K)}     # (in, out)
    u8 = dict(dtype=torch.uint8, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    bufs, outs = {}, {}
    for n, (kin, kout) in shapes.items():
        bufs[n] = dict(qw=torch.empty((kout, kin), **u8), qw_t=torch.empty((kin, kout), **u8),
                       qx=torch.empty((M, kin), **u8), qx_t=torch.empty((kin, M), **u8),
                       qg=torch.empty((M, kout), **u8), qg_t=torch.empty((kout, M), **u8))
        outs[n] = dict(y=torch.empty((M, kout), **bf), dx=torch.empty((M, kin), **bf),
                       dw=torch.empty((kout, kin), **bf))
    inp = {"gate": t["x"], "up": t["x"], "down": t["h"]}
    wts = {"gate": t["w_gate"], "up": t["w_up"], "down": t["w_down"]}
    grads = {"gate": t["g_gate"], "up": t["g_up"], "down": t["g_down"]}

    def step(layers=lins):
        # token-count padding check (8192 is a multiple of 16: nothing to add)
        _, T_pad = m.fp8_pad_tokens(t["x"], query_only=True)
        assert T_pad == M
        for n in ("gate", "up", "down"):
            layers[n].begin_step()
        for n in ("gate", "up", "down"):
            layers[n].forward(inp[n], wts[n], out=outs[n]["y"], bufs=bufs[n])
        for n in ("down", "up", "gate"):
            layers[n].backward(grads[n], dx=outs[n]["dx"], dw=outs[n]["dw"], bufs=bufs[n])
        for n in ("gate", "up", "down"):
            layers[n].end_step()

    for _ in range(args.warmup):
        step()

    def timed_steps(layers=lins, steps=args.steps):
        """(median ms per step, mean ms per step, wall seconds): an event at every step
        boundary (none between the kernels of a step)."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            step(layers)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return float(np.median(per)), ev[0].elapsed_time(ev[-1]) / steps, \
            time.perf_counter() - t0

    # the timed region: K steps with nothing recorded between the kernels of a step
    ms_step, ms_step_mean, wall_s = timed_steps()
    # the same K steps again with a pair of HIP events around every kernel call (on the
    # launch stream): the per-launch durations of the roofline figures. Each event record
    # costs the stream a few microseconds, so this pass is slower as a whole.
    probe.active = True
    ms_step_instr, _, _ = timed_steps()
    probe.active = False
    flops_step = 3 * 6.0 * M * N * K
    value = flops_step / (ms_step * 1e-3) / 1e12

    gemm_ms = probe.durations_ms("gemm")
    q_ms = probe.durations_ms("quantize")
    s_ms = probe.durations_ms("scale")
    gemm_avg = float(np.mean(gemm_ms))
    gemm_flops = 2.0 * M * N * K                   # every one of the 9 GEMMs has this count
    gemm_tflops = gemm_flops / (gemm_avg * 1e-3) / 1e12
    q_elems_step = 3 * (M * K + N * K + M * N)     # per linear: x, W, g (equal across the three)
    q_bytes_step = 4 * q_elems_step                # 2 B read + 1 B Q + 1 B Q^T per element
    q_ms_step = float(np.sum(q_ms)) / args.steps
    q_gbs = q_bytes_step / (q_ms_step * 1e-3) / 1e9
    g_traffic = counter_traffic("gemm_fp8_mx16_kernel")
    q_traffic = counter_traffic("quantize_tensorwise_kernel")
    line = {
        "metric": "fp8 linear fwd+bwd TFLOP/s at 8192x4096x14336; quantize+amax GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_mean": round(ms_step_mean, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": "Llama-8B-shaped MLP block fwd+bwd (gate, up: 4096->14336; "
                               "down: 14336->4096), delayed tensorwise scaling",
                   "tokens": M, "K": K, "N": N, "linears": 3, "flops_per_step": flops_step},
        "roofline": {"bound": "mfma", "kernel": "gemm_fp8_mx16_kernel",
                     "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": g_traffic and g_traffic["bytes"],
                     "traffic_detail": g_traffic,
                     # A + B codes (1 B) in, D (bf16) out, averaged over fwd / dgrad / wgrad
                     "algorithmic_bytes_per_launch": 4 * (M * K + N * K + M * N) // 3,
                     "avg_launch_us": round(gemm_avg * 1e3, 2),
                     "launches": len(gemm_ms)},
        "quantize_amax": {"achieved": round(q_gbs, 1), "unit": "GB/s", "peak": PEAK_HBM_GBS,
                          "frac": round(q_gbs / PEAK_HBM_GBS, 4),
                          "avg_launch_us": round(float(np.mean(q_ms)) * 1e3, 2),
                          "bytes_per_step": q_bytes_step,
                          "traffic": q_traffic and q_traffic["bytes"],
                          "algorithmic_bytes_per_launch": q_bytes_step // 9},
        "breakdown_ms_per_step": {"gemm": round(float(np.sum(gemm_ms)) / args.steps, 4),
                                  "quantize": round(q_ms_step, 4),
                                  "scale_update": round(float(np.sum(s_ms)) / args.steps, 4)},
        "gemm_only_tflops": round(9 * gemm_flops / (float(np.sum(gemm_ms)) / args.steps * 1e-3)
                                  / 1e12, 2),
        "instrumented_pass": {"steps": args.steps, "ms_per_step": round(ms_step_instr, 4),
                              "events": "a HIP event pair around every kernel call; source of "
                                        "roofline, quantize_amax and breakdown_ms_per_step"},
        "wall_s_timed": round(wall_s, 3),
        "device": torch.cuda.get_device_name(0),
    }
    if not args.headline_only:
        # the hybrid format on the same inputs and buffers: gradients in E5M2
        hprobe = EventProbe(torch)
        hyb = {n: m.DelayedScalingLinear(dev, probe=hprobe, grad_format="e5m2")
               for n in ("gate", "up", "down")}
        hsteps = max(3, args.steps // 3)
        for _ in range(2):
            step(hyb)
        ms_h, _, _ = timed_steps(hyb, hsteps)
        hprobe.active = True
        timed_steps(hyb, hsteps)
        hprobe.active = False
        h_gemm = hprobe.durations_ms("gemm")
        # per step: 3 forward GEMMs (E4M3 x E4M3), then dgrad and wgrad of each linear
        bwd = [d for i, d in enumerate(h_gemm) if i % 9 >= 3]
        line["hybrid_e5m2_gradients"] = {
            "workload": "the same MLP block with the output gradients coded in E5M2 "
                        "(x, W in E4M3; dgrad/wgrad on the mixed-format MFMA)",
            "tflops": round(flops_step / (ms_h * 1e-3) / 1e12, 2),
            "ms_per_step": round(ms_h, 4),
            "gemm_tflops_per_launch": round(gemm_flops / (float(np.mean(h_gemm)) * 1e-3) / 1e12, 2),
            "backward_gemm_tflops_per_launch": round(
                gemm_flops / (float(np.mean(bwd)) * 1e-3) / 1e12, 2),
        }
        del hyb
    del t, bufs, outs, lins
    if not args.headline_only:
        torch.cuda.empty_cache()
        line["other_rows"] = {
            "config1_current_scaling": measure_config1(torch, m, workloads),
            "config2_delayed_4096": measure_config2(torch, m),
            "quantize_vs_copy": measure_quantize_vs_copy(torch, m),
            "block_recipe": measure_block_recipe(torch, m, workloads, max(3, args.steps // 3), 2),
            "packed_varlen_padding": measure_varlen(torch, m, workloads, max(3, args.steps // 3), 2),
            "autograd_bias_f1": measure_f1(torch, m, max(3, args.steps // 3), 2),
            "bf16_gemm_step": measure_bf16_step(torch, line["ms_per_step"]),
        }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_sample_tokens)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
