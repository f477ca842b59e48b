"""A current-scaling forward captured as one HIP graph and replayed.

Config 1 (x [64, 128], W [128, 128], N(0, 1)): per operand an amax pass folded into a
cleared buffer, the scale from that amax (which clears the buffer again), the cast; then the
GEMM. The graph is replayed several times, with other eager work and synchronizations in
between; every replay must give the eager result byte for byte (codes, scales, y), and that
result must match the oracle (codes and scales bit-exact, y within both GEMM bounds). The
library clears buffers with kernels, never with memset nodes.
"""
import numpy as np
import pytest

import workloads
from oracle import gemm
from oracle.linear import current_scaled_forward
from tests.gpu_util import (assert_same_bytes, assert_within, dev_bf16, f32_bits, host_bf16_f64,
                            host_u8, note)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_fp8_linear_amd as m
    m.load()
    return m


def test_config1_forward_graph_replays(lib):
    d = workloads.linear_inputs(1)
    x, w = dev_bf16(d["x"]), dev_bf16(d["w"])
    f32 = dict(dtype=torch.float32, device="cuda")
    amax = {n: torch.zeros(1, **f32) for n in "xw"}
    sc = {n: torch.ones(1, **f32) for n in "xw"}
    si = {n: torch.ones(1, **f32) for n in "xw"}
    q = {"x": torch.empty((64, 128), dtype=torch.uint8, device="cuda"),
         "w": torch.empty((128, 128), dtype=torch.uint8, device="cuda")}
    y = torch.empty((64, 128), dtype=torch.bfloat16, device="cuda")
    src = {"x": x, "w": w}

    def forward():
        for n in "xw":
            lib.fp8_quantize_amax(src[n], amax=amax[n], amax_accumulate=True, want_q=False,
                                  want_q_t=False)
            lib.fp8_scale_update(lib.FP8_SCALE_FROM_AMAX, amax=amax[n], scale=sc[n],
                                 scale_inv=si[n], clear_amax=True)
            lib.fp8_quantize_amax(src[n], scale_inv=si[n], q=q[n], want_q_t=False,
                                  want_amax=False)
        lib.fp8_linear_fwd(q["x"], q["w"], sc["x"], sc["w"], y=y)

    def snapshot():
        torch.cuda.synchronize()
        return dict(qx=host_u8(q["x"]), qw=host_u8(q["w"]), y=host_bf16_f64(y),
                    s=[f32_bits(t.item()) for t in (sc["x"], sc["w"], si["x"], si["w"])],
                    amax=[f32_bits(t.item()) for t in (amax["x"], amax["w"])])

    note("graph: eager config-1 forward")
    forward()
    eager = snapshot()
    ref = current_scaled_forward(d["x"], d["w"])
    assert_same_bytes(eager["qx"], ref["qx"], "qx")
    assert_same_bytes(eager["qw"], ref["qw"], "qw")
    assert eager["s"] == [f32_bits(v) for v in (ref["sx"], ref["sw"], ref["sx_inv"],
                                                ref["sw_inv"])]
    assert eager["amax"] == [0, 0]                  # cleared by the scale updates
    D, tight = gemm.fp32_bound(ref["qx"], ref["qw"], ref["sx"], ref["sw"])
    assert_within(eager["y"], D, gemm.error_bound(ref["qx"], ref["qw"], ref["sx"], ref["sw"]), "y")
    assert_within(eager["y"], D, tight, "y (float32 accumulation)")

    note("graph: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        forward()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        forward()
    other = torch.randn(256, 512, device="cuda").to(torch.bfloat16)
    for r in range(5):
        note(f"graph: replay {r}")
        y.fill_(7.0)
        for t in q.values():
            t.fill_(0x55)
        for t in list(sc.values()) + list(si.values()):
            t.fill_(3.0)
        graph.replay()
        got = snapshot()
        assert_same_bytes(got["qx"], eager["qx"], f"qx replay {r}")
        assert_same_bytes(got["qw"], eager["qw"], f"qw replay {r}")
        assert got["s"] == eager["s"] and got["amax"] == [0, 0], r
        assert np.array_equal(got["y"], eager["y"]), r
        # eager work of the program between replays
        qo, _, _, _, _ = lib.fp8_quantize_amax(other, scale_inv=torch.ones(1, **f32),
                                               want_q_t=False)
        lib.fp8_linear_fwd(qo, qo, torch.ones(1, **f32), torch.ones(1, **f32))
        torch.cuda.synchronize()


def test_calls_without_a_stream_use_torch_current_stream(lib):
    """A call given no stream is enqueued on torch's current stream: the default stream, a side
    stream made current (checked here), and the capture stream (the replays above)."""
    from scaled_fp8_linear_amd import _abi
    note("binding stream resolution")
    assert _abi._stream(None) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert _abi._stream(None) == side.cuda_stream
        d = workloads.linear_inputs(1)
        y, sc, _, _ = lib.fp8_linear_fwd_current(dev_bf16(d["x"]), dev_bf16(d["w"]))
    torch.cuda.current_stream().wait_stream(side)
    assert _abi._stream(None) == torch.cuda.current_stream().cuda_stream
    y2, sc2, _, _ = lib.fp8_linear_fwd_current(dev_bf16(d["x"]), dev_bf16(d["w"]))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)) and torch.equal(sc, sc2)
