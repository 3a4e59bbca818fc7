"""The PyTorch operator over the C ABI (CPU part: registration, shape propagation, errors)."""
import pytest
import torch

from transformer_encoder_bert_amd import torch_op


def test_operator_is_registered():
    assert hasattr(torch.ops.ftx, "encoder_forward")


def test_fake_implementation_propagates_shape():
    x = torch.empty(2, 33, 768, dtype=torch.float16, device="meta")
    y = torch.ops.ftx.encoder_forward(x, None, 12345)
    assert y.shape == x.shape and y.dtype == x.dtype and y.device.type == "meta"


def test_unknown_id_is_an_error():
    with pytest.raises(ValueError):
        torch.ops.ftx.encoder_forward(torch.zeros(1, 32, 128), None, 987654)


def test_register_and_unregister():
    sentinel = object()
    i = torch_op.register(sentinel)
    assert torch_op._lookup(i) is sentinel
    torch_op.unregister(i)
    with pytest.raises(ValueError):
        torch_op._lookup(i)
