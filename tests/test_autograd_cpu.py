"""The autograd entry without a GPU: it has no CPU path, so host tensors are
refused before anything reaches the library."""
import pytest

torch = pytest.importorskip("torch")

from numerics_safe_softmax_amd import autograd


def test_host_tensors_are_refused():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(ValueError, match="GPU"):
        autograd.attention(q, q, q)


def test_layer_shapes_and_init_without_running():
    layer = autograd.GPT2Attention(d_model=768, n_head=12, device="cpu", seed=3)
    assert layer.w_qkv.shape == (2304, 768) and layer.w_out.shape == (768, 768)
    assert layer.w_qkv.dtype == torch.bfloat16
    assert float(layer.b_qkv.float().abs().sum()) == 0.0
    std = float(layer.w_qkv.float().std())
    assert 0.018 < std < 0.022
    with pytest.raises(ValueError):
        autograd.GPT2Attention(d_model=100, n_head=12)
