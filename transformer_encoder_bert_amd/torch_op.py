"""The encoder forward as a PyTorch operator, ``torch.ops.ftx.encoder_forward``.

The Faster Transformer article (cloud.tencent.com/developer/article/1490359, section
"Faster Transformer 优化原理") ships its encoder as a TensorFlow op that a graph uses after
loading the shared library.  This is the PyTorch counterpart: a custom operator over the C
ABI of libftx.so, so the forward can sit inside a model as one opaque op (with a fake
implementation for shape propagation).  Argument marshalling only -- the computation is
ftx_forward.

A handle cannot travel through an operator's schema, so encoders are registered under an
integer id: ``op_id = register(encoder)``, then
``torch.ops.ftx.encoder_forward(x, seq_lens, op_id)`` (``seq_lens`` may be None).
"""
from __future__ import annotations

import itertools
import threading
from typing import Dict, Optional

import torch

from .ftx import Encoder

_lock = threading.Lock()
_ids = itertools.count(1)
_encoders: Dict[int, Encoder] = {}


def register(encoder: Encoder) -> int:
    """Make ``encoder`` callable through the operator; returns its id."""
    with _lock:
        i = next(_ids)
        _encoders[i] = encoder
    return i


def unregister(op_id: int) -> None:
    with _lock:
        _encoders.pop(op_id, None)


def _lookup(op_id: int) -> Encoder:
    try:
        return _encoders[op_id]
    except KeyError:
        raise ValueError(f"no ftx encoder registered under id {op_id}") from None


def _checked(x: torch.Tensor, op_id: int) -> Encoder:
    enc = _lookup(op_id)
    if tuple(x.shape) != tuple(enc.shape):
        raise ValueError(f"input has shape {tuple(x.shape)}, the encoder takes [B][S][H] = {enc.shape}")
    return enc


@torch.library.custom_op("ftx::encoder_forward", mutates_args=())
def encoder_forward(x: torch.Tensor, seq_lens: Optional[torch.Tensor], op_id: int) -> torch.Tensor:
    """[B][S][H] -> [B][S][H] (a new contiguous tensor): the L-layer encoder forward of the
    registered handle, on the current stream."""
    return _checked(x, op_id).forward(x.contiguous(), seq_lens)


@encoder_forward.register_fake
def _(x, seq_lens, op_id):
    return x.new_empty(_checked(x, op_id).shape)


class EncoderModule(torch.nn.Module):
    """An ``nn.Module`` around one handle: ``module(x, seq_lens=None)`` calls the operator.

    Weights are given once (per layer, dicts of device tensors named as in ftx_layer_weights)
    and copied into the handle; the module keeps no tensors of its own."""

    def __init__(self, encoder: Encoder):
        super().__init__()
        self.encoder = encoder
        self.op_id = register(encoder)

    def forward(self, x: torch.Tensor, seq_lens: Optional[torch.Tensor] = None) -> torch.Tensor:
        return torch.ops.ftx.encoder_forward(x, seq_lens, self.op_id)

    def close(self) -> None:
        unregister(self.op_id)
        self.encoder.close()
