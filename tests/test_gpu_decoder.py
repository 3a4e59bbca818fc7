"""Decoder parity of ftx_decoder_forward (and of the masked-attention step it is built on)
against the fp64 decoder oracle, through the C ABI.

Bars: the encoder's (tests/test_gpu_encoder.py) -- fp32 |gpu - oracle| / max(|oracle|, 1)
<= 1e-4; fp16 |gpu - oracle| <= 1e-2 per layer and <= 5e-2 per stack; bf16 the same plus
one ulp of the output, 2^-8 |oracle|.  Per layer: a one-layer handle fed the oracle's
previous-layer output rounded to the storage format.  Attention steps: the bar of the
encoder's attention step (fp32 accumulation, one output rounding).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_util import DEV, TORCH, UNIT, announce, assert_within, dev_lens, need_gpu, to_dev, to_f64
from transformer_encoder_bert_amd import ftx

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16"]


@pytest.fixture(autouse=True)
def _gpu(request):
    need_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def check(g, o, dtype, tol, what):
    if dtype == "fp32":
        rel = np.abs(g - o) / np.maximum(np.abs(o), 1.0)
        assert np.all(np.isfinite(g))
        assert rel.max() <= 1e-4, f"{what}: fp32 max relative error {rel.max():.3g} > 1e-4"
        return
    atol, rtol = tol
    assert_within(g, o, atol, rtol, what)


LAYER_TOL = {"fp32": None, "fp16": (1e-2, 0.0), "bf16": (1e-2, 2.0 ** -8)}
STACK_TOL = {"fp32": None, "fp16": (5e-2, 0.0), "bf16": (5e-2, 2.0 ** -8)}


# ------------------------------------------------------------------ masked attention step

ATTN = [
    # B, Sq, Sk, n, d, causal, key_lens
    (2, 32, 32, 3, 64, True, None),          # causal, S = 32 (the kernel without LDS)
    (2, 64, 64, 2, 64, True, None),          # causal across key tiles
    (1, 128, 128, 2, 32, True, None),
    (1, 512, 512, 1, 64, True, None),        # causal over several softmax chunks
    (2, 32, 96, 2, 64, False, [96, 40]),     # cross: fewer queries than keys
    (2, 128, 32, 2, 64, False, [32, 7]),     # cross: more queries than keys
    (1, 64, 512, 2, 64, False, [300]),       # cross, long memory
    (70, 32, 32, 32, 64, True, None),        # causal, over 2048 heads: the LDS kernel at S = 32
    (8, 512, 512, 2, 64, True, None),        # causal, 16 heads: query groups renumbered by XCD
    (4, 512, 256, 2, 32, False, [256, 1, 129, 200]),  # cross: four query groups over two key chunks
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B,Sq,Sk,n,d,causal,lens", ATTN)
def test_masked_attention(dtype, B, Sq, Sk, n, d, causal, lens):
    rng = np.random.default_rng(B * 1000 + Sq * 7 + Sk + n + d + causal)
    r = lambda shape: si.round_to(rng.normal(size=shape), dtype)
    q, k, v = r((B, n, Sq, d)), r((B, n, Sk, d)), r((B, n, Sk, d))
    lens_np = None if lens is None else np.array(lens, dtype=np.int32)
    s = oracle.scaled_scores(q, k)
    p = oracle.causal_softmax(s) if causal else oracle.masked_softmax(s, lens_np)
    ref = oracle.merge_heads(oracle.context(p, v))
    ctx = torch.empty((B, Sq, n * d), dtype=TORCH[dtype], device=DEV)
    ftx.ftx_step_masked_attention(B, Sq, Sk, n, d, to_dev(q, dtype), to_dev(k, dtype),
                                  to_dev(np.ascontiguousarray(np.swapaxes(v, -1, -2)), dtype),
                                  dev_lens(lens_np), causal, ctx)
    # the bar of the encoder's attention step: probabilities rounded to the storage format
    # before the P V product (relative 2u of each |v| term), one output rounding
    u = UNIT[dtype]
    atol = (2 * u if dtype != "fp32" else 1e-6) * np.abs(v).max() + 1e-6
    assert_within(to_f64(ctx), ref, atol, 2 * u, "masked attention")


# ------------------------------------------------------------------ decoder layers

CASES = [
    # B, Sd, Se, n, d, layers, dtype, mem_lens_range, params
    (2, 32, 64, 4, 32, 2, "fp32", (20, 64), "random_affine"),
    (2, 64, 32, 4, 32, 2, "fp16", (5, 32), "random_affine"),
    (3, 32, 96, 12, 64, 2, "fp16", (40, 96), "bert"),
    (2, 64, 128, 4, 64, 2, "bf16", (64, 128), "random_affine"),
    # 512 target rows at hidden 768: the three projections before a LayerNorm split K over
    # 384 tiles of 32 x 32, and the LayerNorms sum the partials
    (16, 32, 32, 12, 64, 1, "fp16", (8, 32), "random_affine"),
]


@functools.lru_cache(maxsize=4)
def _case(B, Sd, Se, n, d, L, dtype, mlr, params):
    sh = si.DecoderShape(B, Sd, Se, n, d, L, dtype)
    c = si.make_decoder_case(sh, 7 + B + Sd + Se, params=params, mem_lens_range=mlr)
    return c, list(c.layers())


def _decoder(shape, layers):
    dec = ftx.Decoder(shape.batch, shape.tgt_len, shape.mem_len, shape.head_num,
                      shape.size_per_head, len(layers), shape.dtype)
    for l, w in enumerate(layers):
        dec.set_weights(l, {k: to_dev(w[k], shape.dtype) for k in si.DECODER_WEIGHT_NAMES})
    torch.cuda.synchronize()
    return dec


@pytest.mark.parametrize("case", CASES)
def test_every_layer(case):
    c, layers = _case(*case)
    sh = c.shape
    lens = dev_lens(c.mem_lens)
    mem = to_dev(c.mem, sh.dtype)
    x = c.x
    for l, w in enumerate(layers):
        dec = _decoder(si.DecoderShape(sh.batch, sh.tgt_len, sh.mem_len, sh.head_num,
                                       sh.size_per_head, 1, sh.dtype), [w])
        got = to_f64(dec.forward(to_dev(x, sh.dtype), mem, lens))
        dec.close()
        ref = oracle.decoder_layer(x, c.mem, w, c.mem_lens, sh.head_num)
        check(got, ref, sh.dtype, LAYER_TOL[sh.dtype], f"layer {l}")
        x = si.round_to(ref, sh.dtype)


@pytest.mark.parametrize("case", CASES)
def test_stack(case):
    c, layers = _case(*case)
    sh = c.shape
    dec = _decoder(sh, layers)
    got = to_f64(dec.forward(to_dev(c.x, sh.dtype), to_dev(c.mem, sh.dtype), dev_lens(c.mem_lens)))
    dec.close()
    ref = oracle.decoder(c.x, c.mem, layers, c.mem_lens, sh.head_num)
    check(got, ref, sh.dtype, STACK_TOL[sh.dtype], "stack")


@pytest.mark.parametrize("Sd,Se,dtype,with_lens", [
    (1, 1, "fp16", False), (17, 40, "fp16", True), (33, 100, "bf16", True),
    (70, 33, "fp32", False), (5, 511, "fp16", True), (100, 7, "bf16", False)])
def test_ragged_lengths(Sd, Se, dtype, with_lens):
    """Lengths that are not multiples of 32: padded inside the handle, compared with the
    oracle at the caller's lengths."""
    sh = si.DecoderShape(2, Sd, Se, 4, 32, 2, dtype)
    c = si.make_decoder_case(sh, 31 + Sd + Se, params="random_affine",
                             mem_lens_range=(1, Se) if with_lens else None)
    layers = list(c.layers())
    dec = _decoder(sh, layers)
    got = to_f64(dec.forward(to_dev(c.x, dtype), to_dev(c.mem, dtype), dev_lens(c.mem_lens)))
    dec.close()
    ref = oracle.decoder(c.x, c.mem, layers, c.mem_lens, sh.head_num)
    check(got, ref, dtype, STACK_TOL[dtype], f"Sd={Sd} Se={Se}")


def test_later_positions_do_not_reach_earlier_rows():
    """Causality on the GPU: rows i+1.. of the input perturbed, rows 0..i of the output
    unchanged bit for bit."""
    c, layers = _case(*CASES[1])
    sh = c.shape
    dec = _decoder(sh, layers)
    mem, lens = to_dev(c.mem, sh.dtype), dev_lens(c.mem_lens)
    base = to_f64(dec.forward(to_dev(c.x, sh.dtype), mem, lens))
    rng = np.random.default_rng(3)
    for i in (0, 17, 40):
        x1 = c.x.copy()
        x1[:, i + 1:] = si.round_to(rng.normal(size=x1[:, i + 1:].shape) * 3, sh.dtype)
        out = to_f64(dec.forward(to_dev(x1, sh.dtype), mem, lens))
        np.testing.assert_array_equal(out[:, : i + 1], base[:, : i + 1])
        assert not np.array_equal(out[:, i + 1:], base[:, i + 1:])
    dec.close()


def test_padded_memory_does_not_reach_outputs():
    c, layers = _case(*CASES[2])
    sh = c.shape
    dec = _decoder(sh, layers)
    x, lens = to_dev(c.x, sh.dtype), dev_lens(c.mem_lens)
    base = to_f64(dec.forward(x, to_dev(c.mem, sh.dtype), lens))
    m1 = c.mem.copy()
    rng = np.random.default_rng(9)
    for b, L in enumerate(c.mem_lens):
        m1[b, L:] = si.round_to(rng.normal(size=m1[b, L:].shape) * 5, sh.dtype)
    out = to_f64(dec.forward(x, to_dev(m1, sh.dtype), lens))
    dec.close()
    np.testing.assert_array_equal(out, base)


def test_deterministic_and_inputs_untouched():
    c, layers = _case(*CASES[2])
    sh = c.shape
    dec = _decoder(sh, layers)
    x, mem, lens = to_dev(c.x, sh.dtype), to_dev(c.mem, sh.dtype), dev_lens(c.mem_lens)
    x0, m0 = x.clone(), mem.clone()
    a = dec.forward(x, mem, lens).clone()
    b = dec.forward(x, mem, lens)
    dec.close()
    assert torch.equal(a, b) and torch.equal(x, x0) and torch.equal(mem, m0)


@pytest.mark.parametrize("Sd,Se,d,dtype", [(32, 64, 64, "fp16"), (64, 32, 64, "bf16"), (100, 40, 64, "fp16"),
                                          (32, 32, 32, "fp16")])
def test_fused_self_attention_matches_oracle(Sd, Se, d, dtype):
    """FTX_OPT_FUSED_ATTENTION = 2: the causal self-attention inside the self Q/K/V
    projection (Sd = 100 is padded to 128; d = 32 puts two heads in a tile)."""
    sh = si.DecoderShape(3, Sd, Se, 2, d, 2, dtype)
    c = si.make_decoder_case(sh, 41 + Sd + Se, params="random_affine", mem_lens_range=(1, Se))
    layers = list(c.layers())
    dec = ftx.Decoder(sh.batch, sh.tgt_len, sh.mem_len, sh.head_num, sh.size_per_head, 2, dtype)
    dec.set_option(ftx.FTX_OPT_FUSED_ATTENTION, 2)
    dec.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
    for l, w in enumerate(layers):
        dec.set_weights(l, {k: to_dev(w[k], dtype) for k in si.DECODER_WEIGHT_NAMES})
    got = to_f64(dec.forward(to_dev(c.x, dtype), to_dev(c.mem, dtype), dev_lens(c.mem_lens)))
    t = dec.kernel_times()
    dec.close()
    assert t["self_qkv_attention"][1] == 2 and t["self_attention"][1] == 0
    ref = oracle.decoder(c.x, c.mem, layers, c.mem_lens, sh.head_num)
    check(got, ref, dtype, STACK_TOL[dtype], f"fused self-attention Sd={Sd}")


def test_fused_self_attention_is_causal():
    """Rows after i perturbed: rows 0..i of the output unchanged bit for bit, fused path."""
    sh = si.DecoderShape(2, 64, 32, 2, 64, 2, "fp16")
    c = si.make_decoder_case(sh, 5, params="random_affine", mem_lens_range=(5, 32))
    layers = list(c.layers())
    dec = ftx.Decoder(2, 64, 32, 2, 64, 2, "fp16")
    dec.set_option(ftx.FTX_OPT_FUSED_ATTENTION, 2)
    for l, w in enumerate(layers):
        dec.set_weights(l, {k: to_dev(w[k], "fp16") for k in si.DECODER_WEIGHT_NAMES})
    mem, lens = to_dev(c.mem, "fp16"), dev_lens(c.mem_lens)
    base = to_f64(dec.forward(to_dev(c.x, "fp16"), mem, lens))
    rng = np.random.default_rng(3)
    for i in (0, 31, 40):
        x1 = c.x.copy()
        x1[:, i + 1:] = si.round_to(rng.normal(size=x1[:, i + 1:].shape) * 3, "fp16")
        out = to_f64(dec.forward(to_dev(x1, "fp16"), mem, lens))
        np.testing.assert_array_equal(out[:, : i + 1], base[:, : i + 1])
        assert not np.array_equal(out[:, i + 1:], base[:, i + 1:])
    dec.close()


def test_decoder_errors_on_device():
    c, layers = _case(*CASES[1])
    sh = c.shape
    dec = ftx.Decoder(sh.batch, sh.tgt_len, sh.mem_len, sh.head_num, sh.size_per_head, 2, sh.dtype)
    dec.set_weights(0, {k: to_dev(layers[0][k], sh.dtype) for k in si.DECODER_WEIGHT_NAMES})
    x, mem = to_dev(c.x, sh.dtype), to_dev(c.mem, sh.dtype)
    with pytest.raises(ftx.FtxError) as e:
        dec.forward(x, mem)                       # layer 1 has no weights
    assert e.value.status == ftx.FTX_ERR_NOT_READY
    with pytest.raises(ftx.FtxError) as e:
        ftx.ftx_decoder_forward(dec.handle, x, mem, None, x)   # output aliases the input
    assert e.value.status == ftx.FTX_ERR_INVALID_ARG
    dec.close()


def test_full_size_sampled_rows():
    """The decoder workload at batch 512 in the launch configuration the benchmark times (the
    causal self-attention inside the projection); the oracle checks sampled sequences
    (sequences are independent)."""
    wd = si.DECODER_WORKLOAD
    sh = si.DecoderShape(512, wd["tgt_len"], wd["mem_len"], wd["head_num"], wd["size_per_head"],
                         wd["num_layers"], wd["dtype"])
    c = si.make_decoder_case(sh, wd["seed"], mem_lens_range=wd["mem_lens_range"])
    layers = list(c.layers())
    dec = _decoder(sh, layers)
    dec.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
    out = dec.forward(to_dev(c.x, sh.dtype), to_dev(c.mem, sh.dtype), dev_lens(c.mem_lens))
    t = dec.kernel_times()
    rows = [0, 255, 511]
    got = to_f64(out[rows])
    dec.close()
    assert t["self_qkv_attention"][1] == sh.num_layers
    ref = oracle.decoder(c.x[rows], c.mem[rows], layers, c.mem_lens[rows], sh.head_num)
    check(got, ref, sh.dtype, STACK_TOL[sh.dtype], f"decoder B512 rows {rows}")
