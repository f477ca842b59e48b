"""GPU parity for per-sequence padding of packed batches (TP/SP/CP alignment).

* fp8_pad_varlen / fp8_unpad_varlen bit-exact with the oracle's loops: the packed-varlen
  lengths (64 sequences U{32..2048}) under the THD multiples for tp = cp = 2, several
  hundred sequences (more than one launch's table) with empty ones among them, no sequences
  at all; the padding rows are zero even where the output buffer held NaN;
* a layer step on a per-sequence padded batch: the zero padding rows quantize to 0x00, keep
  out of amax and give zero output rows, and the unpadded outputs match the oracle.
"""
import numpy as np
import pytest

import workloads
from oracle import gemm, padding
from oracle.linear import DelayedLinear
from tests.gpu_util import (assert_same_bytes, assert_within, dev_bf16, f32_bits,
                            host_bf16_bits, host_bf16_f64, note)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import scaled_fp8_linear_amd as m
    m.load()
    return m


def _round_trip(m, lens, cols, sm, tm, seed):
    lens = [int(v) for v in lens]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    x = workloads.bf16_tensor("normal", (max(T, 1), cols), 99, seed, cols, std=1.0)[:T]
    want, ocu = padding.pad_varlen(x, lens, sm, tm)
    xd = dev_bf16(x) if T else torch.empty((0, cols), dtype=torch.bfloat16, device="cuda")
    _, _, T_pad = m.fp8_pad_varlen(xd, cu, sm, tm, query_only=True)
    x_pad = torch.full((T_pad, cols), float("nan"), dtype=torch.bfloat16, device="cuda")
    note(f"pad_varlen nseq={len(lens)} T={T} cols={cols} seq_multiple={sm} total={tm}")
    x_pad, cu_pad, T_pad = m.fp8_pad_varlen(xd, cu, sm, tm, x_pad=x_pad)
    torch.cuda.synchronize()
    assert cu_pad == list(ocu) and T_pad == want.shape[0]
    assert_same_bytes(host_bf16_bits(x_pad), want, "x_pad")
    note(f"unpad_varlen nseq={len(lens)}")
    back = m.fp8_unpad_varlen(x_pad, cu, cu_pad)
    torch.cuda.synchronize()
    assert_same_bytes(host_bf16_bits(back), padding.unpad_varlen(want, lens, ocu), "unpad")
    assert_same_bytes(host_bf16_bits(back), x, "unpad = input")


def test_packed_varlen_lengths_thd_cp2_tp2(lib):
    sm, tm = padding.align_multiples(padding.THD, tp=2, cp=2)
    assert (sm, tm) == (4, 64)
    _round_trip(lib, workloads.varlen_lengths(4), 64, sm, tm, 1)


@pytest.mark.parametrize("nseq,cols,sm,tm", [(300, 16, 8, 16), (129, 48, 3, 5), (128, 32, 1, 16),
                                             (1, 4096, 2, 128)])
def test_many_sequences_and_empty_ones(lib, nseq, cols, sm, tm):
    rng = np.random.default_rng(nseq)
    lens = rng.integers(0, 40, nseq)
    lens[::7] = 0
    _round_trip(lib, lens, cols, sm, tm, nseq)


def test_no_sequences(lib):
    _round_trip(lib, [], 16, 4, 16, 0)


def test_bshd_batch_through_the_layer(lib):
    """B = 6 sequences of T = 37 tokens under tp = 4 (BSHD): each is padded to the lcm rule's
    multiple, the layer runs on the padded batch, outputs at padding rows are exactly zero
    and the unpadded outputs match the oracle on the same padded batch."""
    B, T, tp, K, N = 6, 37, 4, 128, 160
    sm, tm = lib.fp8_align_multiple(lib.FP8_LAYOUT_BSHD, B, tp)
    assert (sm, tm) == padding.align_multiples(padding.BSHD, B, tp)
    lens = [T] * B
    cu = np.arange(B + 1, dtype=np.int64) * T
    d = workloads.linear_inputs(2, 1, M=B * T, K=K, N=N)
    x_pad, cu_pad, T_pad = lib.fp8_pad_varlen(dev_bf16(d["x"]), cu, sm, tm)
    Tp = cu_pad[1]
    assert Tp % tp == 0 and (B * Tp) % (16 * tp) == 0 and T_pad == B * Tp
    ox, _ = padding.pad_varlen(d["x"], lens, sm, tm)
    gfull = workloads.linear_inputs(2, 2, M=T_pad, K=K, N=N)["g"]
    og, _ = padding.pad_varlen(padding.unpad_varlen(gfull, lens, cu_pad), lens, sm, tm)
    lin = lib.DelayedScalingLinear("cuda", keep_amax=True)
    ref = DelayedLinear()
    for step in range(3):
        note(f"BSHD padded layer step {step}")
        lin.begin_step()
        ref.begin_step()
        y = lin.forward(x_pad, dev_bf16(d["w"]))
        dx, dw = lin.backward(dev_bf16(og))
        torch.cuda.synchronize()
        f = ref.forward(ox, d["w"])
        b = ref.backward(og)
        assert f32_bits(lin.amax_x.item()) == f32_bits(f["amax_x"])
        assert f32_bits(lin.amax_g.item()) == f32_bits(b["amax_g"])
        yh = host_bf16_f64(y)
        pad_rows = np.ones(T_pad, bool)
        for i in range(B):
            pad_rows[cu_pad[i]:cu_pad[i] + T] = False
        assert np.all(yh[pad_rows] == 0) and np.all(host_bf16_f64(dx)[pad_rows] == 0)
        assert_within(yh, f["y"], gemm.error_bound(f["qx"], f["qw"], f["sx"], f["sw"]), "y")
        assert_within(host_bf16_f64(dw), b["dw"],
                      gemm.error_bound(b["qg_t"], f["qx_t"], b["sg"], f["sx"]), "dw")
        y_packed = lib.fp8_unpad_varlen(y, cu, cu_pad)
        torch.cuda.synchronize()
        assert_same_bytes(host_bf16_bits(y_packed),
                          padding.unpad_varlen(host_bf16_bits(y), lens, cu_pad), "y unpadded")
        lin.end_step()


def test_full_size_packed_batch_as_benchmarked(lib):
    """The benchmark's launch: the 54 657-token packed batch, 4096 columns, THD with
    tp = cp = 2 (each sequence to a multiple of 4, the batch to 64), pad and unpad bit-exact
    with the oracle over every row."""
    sm, tm = lib.fp8_align_multiple(lib.FP8_LAYOUT_THD, 1, 2, 2)
    lens = workloads.varlen_lengths(4)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    x = workloads.bf16_tensor("normal", (T, 4096), 4, 98, 0, std=1.0)
    want, ocu = padding.pad_varlen(x, lens, sm, tm)
    note(f"full-size pad_varlen T={T} cols=4096")
    x_pad, cu_pad, T_pad = lib.fp8_pad_varlen(dev_bf16(x), cu, sm, tm)
    torch.cuda.synchronize()
    assert cu_pad == list(ocu) and T_pad == want.shape[0] == 54784
    assert_same_bytes(host_bf16_bits(x_pad), want, "x_pad")
    back = lib.fp8_unpad_varlen(x_pad, cu, cu_pad)
    torch.cuda.synchronize()
    assert_same_bytes(host_bf16_bits(back), x, "unpad")
