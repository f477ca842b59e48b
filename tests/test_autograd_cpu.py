"""Host logic of the autograd wrapper: the autocast counter, the bf16 path outside
fp8_autocast, and the delayed-scaling state's save/restore (no GPU needed)."""
import pytest

torch = pytest.importorskip("torch")

import scaled_fp8_linear_amd as m  # noqa: E402
from scaled_fp8_linear_amd.state import DelayedScalingLinear  # noqa: E402


def test_autocast_advances_once_per_entry():
    st = m.fp8_state()
    st.reset()
    assert not st.enabled
    for k in range(1, 4):
        with m.fp8_autocast():
            assert st.enabled and st.step_count == k
        assert not st.enabled
    with m.fp8_autocast(enabled=False):
        assert not st.enabled and st.step_count == 3
    st.reset()
    assert st.step_count == 0


def test_bf16_path_outside_autocast_and_for_unaligned_features():
    torch.manual_seed(0)
    for fin, fout in [(32, 48), (20, 48)]:
        layer = m.Fp8Linear(fin, fout)
        x = torch.randn(5, fin, dtype=torch.bfloat16)
        want = torch.nn.functional.linear(x, layer.weight)
        assert torch.equal(layer(x), want)
        if fin % 16:
            with m.fp8_autocast():      # features not a multiple of 16 stay bf16
                assert torch.equal(layer(x), want)
    m.fp8_state().reset()


def test_schedule_state_round_trip():
    a = DelayedScalingLinear("cpu")
    a.hist.copy_(torch.arange(16, dtype=torch.float32))
    a.w_scale.fill_(0.25)
    a.x_scale.copy_(torch.tensor([2.0, 3.0]))
    a.g_scale.copy_(torch.tensor([5.0, 7.0]))
    a.step_count, a.idx, a.cur = 37, 5, 1
    b = DelayedScalingLinear("cpu")
    b.load_state_dict(a.state_dict())
    assert (b.step_count, b.idx, b.cur) == (37, 5, 1)
    for k in a._TENSORS:
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    with pytest.raises(ValueError):
        DelayedScalingLinear("cpu", update_interval=8).load_state_dict(a.state_dict())


def test_step_without_backward_keeps_gradient_scale():
    a = DelayedScalingLinear("cpu")
    a.g_scale.copy_(torch.tensor([5.0, 7.0]))
    a.g_scale_inv.copy_(torch.tensor([0.2, 1 / 7]))
    a.cur = 0
    a.end_step(g_updated=False)
    assert a.cur == 1 and a.g_scale[1].item() == 5.0 and a.g_scale_inv[1].item() == pytest.approx(0.2)


def test_module_state_keeps_the_gradient_format():
    """Fp8Linear's saved schedule restores into a layer with the same grad_format (the
    restored schedule codes gradients in E5M2 again), and is refused by one with the
    other format."""
    from scaled_fp8_linear_amd import Fp8Linear
    a = Fp8Linear(32, 48, grad_format="e5m2")
    a._lin = DelayedScalingLinear("cpu", grad_format="e5m2")
    a._lin.step_count, a._lin.idx = 9, 9
    sd = a.state_dict()
    b = Fp8Linear(32, 48, grad_format="e5m2")
    b.load_state_dict(sd)
    assert b._lin.grad_format == "e5m2" and b._lin.step_count == 9
    with pytest.raises(ValueError):
        Fp8Linear(32, 48).load_state_dict(sd)
    with pytest.raises(ValueError):
        Fp8Linear(32, 48, grad_format="e4m2")
