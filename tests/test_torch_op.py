"""The PyTorch operator over the C ABI (CPU part: registration, shape propagation, errors)."""
import pytest
import torch

from transformer_encoder_bert_amd import torch_op


def test_operator_is_registered():
    assert hasattr(torch.ops.ftx, "encoder_forward")


class _StandIn:
    """What the operator needs of a registered encoder for shape propagation."""
    shape = (2, 33, 768)


def test_fake_implementation_propagates_shape():
    i = torch_op.register(_StandIn())
    try:
        x = torch.empty(2, 33, 768, dtype=torch.float16, device="meta")
        y = torch.ops.ftx.encoder_forward(x, None, i)
        assert y.shape == x.shape and y.dtype == x.dtype and y.device.type == "meta"
        assert y.is_contiguous()
        # an input that is not [B][S][H] is refused, not given a wrong output shape
        with pytest.raises(ValueError):
            torch.ops.ftx.encoder_forward(x.view(66, 768), None, i)
        with pytest.raises(ValueError):
            torch.ops.ftx.encoder_forward(torch.empty(1, 33, 768, device="meta"), None, i)
    finally:
        torch_op.unregister(i)


def test_seq_lens_must_cover_the_batch():
    """Encoder.forward refuses a seq_lens tensor that does not hold one length per sequence
    (the kernels read lens[b] for every b), before anything reaches the library."""
    from transformer_encoder_bert_amd import ftx
    enc = ftx.Encoder.__new__(ftx.Encoder)   # argument checks only: no handle, no GPU
    enc.shape, enc.dtype, enc.handle = (4, 32, 128), torch.float16, None
    x = torch.zeros(4, 32, 128, dtype=torch.float16)
    with pytest.raises(ValueError, match="seq_lens has 3 elements"):
        enc.forward(x, torch.full((3,), 32, dtype=torch.int32))
    with pytest.raises(ValueError, match="seq_lens has dtype"):
        enc.forward(x, torch.full((4,), 32, dtype=torch.int64))


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
