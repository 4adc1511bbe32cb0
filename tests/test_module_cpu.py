"""Host-side checks of the trainable layer: parameter shapes and initialisation,
argument validation, and that a CPU tensor is refused (there is no CPU path)."""
import pytest
import torch

from memory_bound_depthwise_amd import WTConvError
from memory_bound_depthwise_amd.module import WTConv2d


def test_parameters_and_init():
    m = WTConv2d(6, 5, 3)
    assert m.weight.shape == (6, 5, 5) and m.bias.shape == (6,) and m.scale.shape == (6,)
    assert m.level_weight.shape == (3, 6, 4, 5, 5) and m.level_scale.shape == (3, 6, 4)
    assert float(m.weight.detach().abs().max()) <= 1 / 5 and float(m.level_weight.detach().abs().max()) <= 1 / 5
    assert torch.all(m.scale == 1) and torch.all(m.level_scale == 1) and torch.all(m.bias == 0)
    assert all(p.dtype == torch.float32 for p in m.parameters())
    assert sum(p.numel() for p in m.parameters()) == 6 * 25 + 6 + 6 + 3 * 6 * 4 * 25 + 3 * 6 * 4


def test_base_only_and_no_bias():
    m = WTConv2d(4, 7, 0, bias=False)
    assert m.level_weight is None and m.level_scale is None and m.bias is None
    assert [n for n, _ in m.named_parameters()] == ["weight", "scale"]


@pytest.mark.parametrize("kw", [dict(kernel_size=4), dict(levels=-1), dict(levels=9)])
def test_rejects_bad_arguments(kw):
    with pytest.raises(ValueError):
        WTConv2d(4, **{"kernel_size": 5, "levels": 1, **kw})


def test_cpu_tensor_is_refused():
    m = WTConv2d(2, 5, 1)
    with pytest.raises(WTConvError):
        m(torch.zeros(1, 2, 8, 8))
