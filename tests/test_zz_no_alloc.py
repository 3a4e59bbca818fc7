"""ftx_forward_static_workspace, the entry point that allocates nothing (its workspace is the
library's static per-GPU scratch), against ftx_forward through the C ABI.

Two calls in a row, the second on a smaller input (a smaller handle, a ragged length that
takes the padded-copy path, bf16 with its fp32 copies), each compared with ftx_forward on the
same handle (same kernels and plans: bitwise equal) and with the fp64 oracle at the stack bar.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_util import announce, assert_within, dev_layer, dev_lens, need_gpu, to_dev, to_f64
from transformer_encoder_bert_amd import ftx

pytestmark = pytest.mark.gpu

STATIC_BYTES = 64 << 20


@pytest.fixture(autouse=True)
def _gpu(request):
    need_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _handle(shape, seed, lens_range):
    c = si.custom_case(shape, seed, params="random_affine", lens_range=lens_range)
    layers = list(c.layers())
    enc = ftx.Encoder(shape.batch, shape.seq_len, shape.head_num, shape.size_per_head,
                      shape.num_layers, shape.dtype)
    for l, w in enumerate(layers):
        enc.set_weights(l, dev_layer(w, shape.dtype))
    torch.cuda.synchronize()
    return c, layers, enc


def _bar(dtype):
    return {"fp16": (5e-2, 0.0), "bf16": (5e-2, 2.0 ** -8)}[dtype]


def test_static_workspace_matches_forward_on_two_calls():
    cases = [
        # the first call: BERT-base heads, 8 sequences of 32 (split-K partials in the scratch)
        (si.Shape(8, 32, 12, 64, 2, "fp16"), 901, (1, 32)),
        # the second, smaller: 3 sequences of 50 (padded to 64 inside the handle), bf16
        (si.Shape(3, 50, 4, 64, 2, "bf16"), 902, (1, 50)),
    ]
    handles = [_handle(sh, seed, lr) for sh, seed, lr in cases]
    outs = []
    for (sh, _, _), (c, layers, enc) in zip(cases, handles):
        x, lens = to_dev(c.x, sh.dtype), dev_lens(c.lens)
        out = torch.full_like(x, float("nan"))
        enc.forward_static_workspace(x, lens, out)   # a call straight after the previous one
        outs.append(out)
    torch.cuda.synchronize()
    for (sh, _, _), (c, layers, enc), got in zip(cases, handles, outs):
        x, lens = to_dev(c.x, sh.dtype), dev_lens(c.lens)
        ref = enc.forward(x, lens)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{sh}: static workspace differs from ftx_forward"
        oref = oracle.encoder(c.x, layers, c.lens, sh.head_num)
        print(sh, assert_within(to_f64(got), oref, *_bar(sh.dtype), f"{sh} vs oracle"))
    # the first handle again, after the second has used the scratch
    c, layers, enc = handles[0]
    x, lens = to_dev(c.x, "fp16"), dev_lens(c.lens)
    again = torch.empty_like(x)
    enc.forward_static_workspace(x, lens, again)
    torch.cuda.synchronize()
    assert torch.equal(again, outs[0])
    for _, _, enc in handles:
        enc.close()


def test_static_workspace_with_the_folded_layernorm():
    """Shapes where the first LayerNorm folds into FFN-in (2048 rows, hidden 768 fp16 and
    hidden 1024 bf16): the per-tile row statistics and Z1 live in the scratch too.  Two calls
    in a row, the second on a different handle; each equals ftx_forward bitwise and meets the
    oracle's stack bar."""
    cases = [(si.Shape(64, 32, 12, 64, 1, "fp16"), 911, (1, 32)),
             (si.Shape(16, 128, 16, 64, 1, "bf16"), 912, (1, 128))]
    handles = [_handle(sh, seed, lr) for sh, seed, lr in cases]
    outs = []
    for (sh, _, _), (c, layers, enc) in zip(cases, handles):
        x, lens = to_dev(c.x, sh.dtype), dev_lens(c.lens)
        out = torch.full_like(x, float("nan"))
        enc.forward_static_workspace(x, lens, out)
        outs.append(out)
    torch.cuda.synchronize()
    for (sh, _, _), (c, layers, enc), got in zip(cases, handles, outs):
        x, lens = to_dev(c.x, sh.dtype), dev_lens(c.lens)
        enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
        ref = enc.forward(x, lens)
        t = enc.kernel_times()
        enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 0)
        assert t["ln1"][1] == 0, f"{sh}: the LayerNorm did not fold"
        assert torch.equal(got, ref), f"{sh}: static workspace differs from ftx_forward"
        oref = oracle.encoder(c.x, layers, c.lens, sh.head_num)
        print(sh, assert_within(to_f64(got), oref, *_bar(sh.dtype), f"{sh} vs oracle"))
    for _, _, enc in handles:
        enc.close()


def test_static_workspace_refuses_a_larger_forward():
    """A handle whose workspace exceeds the static scratch is refused before anything is
    enqueued: BERT-base fp16 at 256 sequences of 32 needs about 120 MiB."""
    sh = si.Shape(256, 32, 12, 64, 1, "fp16")
    c, layers, enc = _handle(sh, 903, None)
    x = to_dev(c.x, "fp16")
    out = torch.zeros_like(x)
    with pytest.raises(ftx.FtxError) as e:
        enc.forward_static_workspace(x, None, out)
    assert e.value.status == ftx.FTX_ERR_UNSUPPORTED
    assert "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not out.any()
    enc.close()
