"""Encoder-level parity of ftx_forward against the fp64 oracle, through the C ABI.

Bars (max over all B x S x H outputs):
* fp32: |gpu - oracle| / max(|oracle|, 1) <= 1e-4;
* fp16: |gpu - oracle| <= 1e-2 per layer and <= 5e-2 after the whole stack;
* bf16: |gpu - oracle| <= 1e-2 + 2^-8 |oracle| per layer and <= 5e-2 + 2^-8 |oracle| per
  stack.  The bare 1e-2 is below bf16's own rounding of outputs |y| >= 4 (half an ulp
  there is 2^-9 * 4 = 7.8e-3, one ulp 1.6e-2), so one ulp of the output, 2^-8 |oracle|, is
  added.  (The library keeps the residual Y1 in fp32 in bf16 mode; with Y1 stored in bf16
  an exact fp64 model of the storage roundings already exceeds this bar.)
Per layer means: a one-layer handle fed the oracle's previous-layer output rounded to the
storage format, compared with the oracle's layer on that same input.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from gpu_util import (DEV, TORCH, announce, assert_within, dev_layer, dev_lens, need_gpu, rnd,
                      to_dev, to_f64)
from transformer_encoder_bert_amd import ftx

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(request):
    need_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def layer_tol(dtype):
    return {"fp32": (0.0, 0.0), "fp16": (1e-2, 0.0), "bf16": (1e-2, 2.0 ** -8)}[dtype]


def stack_tol(dtype):
    return {"fp32": (0.0, 0.0), "fp16": (5e-2, 0.0), "bf16": (5e-2, 2.0 ** -8)}[dtype]


def check(g, o, dtype, tol, what):
    if dtype == "fp32":
        rel = np.abs(g - o) / np.maximum(np.abs(o), 1.0)
        assert np.all(np.isfinite(g))
        assert rel.max() <= 1e-4, f"{what}: fp32 max relative error {rel.max():.3g} > 1e-4"
        return dict(max_rel1=float(rel.max()))
    atol, rtol = tol
    return assert_within(g, o, atol, rtol, what)


@functools.lru_cache(maxsize=4)
def _case(workload, batch, params="bert", num_layers=None):
    c = si.make_case(workload, batch, params=params, num_layers=num_layers)
    layers = list(c.layers())
    return c, layers


@functools.lru_cache(maxsize=4)
def _oracle_states(workload, batch, params="bert", num_layers=None):
    """Oracle output after every layer, [L+1] list starting with the input."""
    c, layers = _case(workload, batch, params, num_layers)
    states = [c.x]
    for w in layers:
        states.append(oracle.encoder_layer(states[-1], w, c.lens, c.shape.head_num))
    return states


def _encoder(shape, layers):
    enc = ftx.Encoder(shape.batch, shape.seq_len, shape.head_num, shape.size_per_head,
                      len(layers), shape.dtype)
    for l, w in enumerate(layers):
        enc.set_weights(l, dev_layer(w, shape.dtype))
    torch.cuda.synchronize()
    return enc


SMALL = [
    ("single_layer_fp32", 1, "bert"),
    ("single_layer_fp32", 1, "random_affine"),
    ("bert_base_fp16_s32", 1, "bert"),
    ("bert_base_fp16_s32", 8, "random_affine"),
    ("pruned_fp16_s32", 64, "bert"),
    ("bert_base_fp16_s64_varlen", 1, "bert"),
    ("bert_base_fp16_s128_varlen", 4, "random_affine"),
    ("bert_large_bf16_s128", 2, "bert"),
    ("bert_large_bf16_s512", 1, "random_affine"),
]


@pytest.mark.parametrize("workload,batch,params", SMALL)
def test_every_layer(workload, batch, params):
    """Each layer of the stack, on the oracle's previous output, within the per-layer bar."""
    c, layers = _case(workload, batch, params)
    states = _oracle_states(workload, batch, params)
    dt = c.shape.dtype
    enc = ftx.Encoder(c.shape.batch, c.shape.seq_len, c.shape.head_num, c.shape.size_per_head, 1, dt)
    lens = dev_lens(c.lens)
    worst = 0.0
    for l, w in enumerate(layers):
        enc.set_weights(0, dev_layer(w, dt))
        x_in = rnd(states[l], dt)
        ref = oracle.encoder_layer(x_in, w, c.lens, c.shape.head_num)
        out = to_f64(enc.forward(to_dev(x_in, dt), lens))
        rep = check(out, ref, dt, layer_tol(dt), f"{workload} B={batch} layer {l}")
        worst = max(worst, rep.get("max_abs", rep.get("max_rel1", 0.0)))
    enc.close()
    print(f"worst per-layer error {worst:.3g}")


@pytest.mark.parametrize("fused", [1, 0])
@pytest.mark.parametrize("workload,batch,params", SMALL)
def test_stack(workload, batch, params, fused):
    c, layers = _case(workload, batch, params)
    ref = _oracle_states(workload, batch, params)[-1]
    enc = _encoder(c.shape, layers)
    enc.set_option(ftx.FTX_OPT_FUSED_EPILOGUES, fused)
    out = to_f64(enc.forward(to_dev(c.x, c.shape.dtype), dev_lens(c.lens)))
    enc.close()
    rep = check(out, ref, c.shape.dtype, stack_tol(c.shape.dtype), f"{workload} B={batch} stack")
    print(rep)


def test_fused_and_unfused_paths_agree():
    c, layers = _case("bert_base_fp16_s64_varlen", 1, "bert")
    enc = _encoder(c.shape, layers)
    x = to_dev(c.x, "fp16")
    lens = dev_lens(c.lens)
    a = to_f64(enc.forward(x, lens))
    enc.set_option(ftx.FTX_OPT_FUSED_EPILOGUES, 0)
    b = to_f64(enc.forward(x, lens))
    enc.close()
    assert_within(a, b, 2e-2, 0.0, "fused vs unfused")


@pytest.mark.parametrize("batch", [1, 8, 64])
def test_deterministic_and_input_untouched(batch):
    """Repeated forwards are bitwise equal.  At batches 1 and 8 the projections split K: the
    split-K reduction and the split-K LayerNorm sum the partials in split order, and their
    row statistics in a fixed order, so nothing depends on which block finishes first.  At
    64 the first LayerNorm is folded: its per-tile statistics are each one block's, merged in
    tile order."""
    c, layers = _case("bert_base_fp16_s32", batch, "random_affine")
    enc = _encoder(c.shape, layers)
    x = to_dev(c.x, "fp16")
    x0 = x.clone()
    a = enc.forward(x).clone()
    b = enc.forward(x).clone()
    d = enc.forward(x)
    enc.close()
    assert torch.equal(a, b) and torch.equal(a, d)
    assert torch.equal(x, x0)


def test_batch_slices_match_the_batch():
    """Sequence b run alone equals sequence b run inside the batch (batch independence).

    The two runs take different GEMM tilings (one sequence is 128 rows, which the planner
    splits along K), so they agree to rounding, not bit for bit: after 12 fp16 layers a few
    outputs near 6 differ by 4 ulp (0.016).  A leak across sequences moves outputs by O(1),
    so the bar is the stack tolerance each run meets against the oracle."""
    c, layers = _case("bert_base_fp16_s128_varlen", 4, "random_affine")
    enc = _encoder(c.shape, layers)
    full = to_f64(enc.forward(to_dev(c.x, "fp16"), dev_lens(c.lens)))
    enc.close()
    one = si.Shape(1, c.shape.seq_len, c.shape.head_num, c.shape.size_per_head, c.shape.num_layers, "fp16")
    enc1 = _encoder(one, layers)
    for b in (0, 3):
        o = to_f64(enc1.forward(to_dev(c.x[b:b + 1], "fp16"), dev_lens(c.lens[b:b + 1])))
        assert_within(o[0], full[b], 5e-2, 0.0, f"sequence {b}")
    enc1.close()


def test_padded_positions_do_not_reach_valid_rows():
    c, layers = _case("bert_base_fp16_s128_varlen", 4, "random_affine")
    enc = _encoder(c.shape, layers)
    lens = dev_lens(c.lens)
    a = to_f64(enc.forward(to_dev(c.x, "fp16"), lens))
    x1 = c.x.copy()
    rng = np.random.default_rng(5)
    for b, L in enumerate(c.lens):
        x1[b, L:] = rnd(rng.normal(size=x1[b, L:].shape) * 3, "fp16")
    b_out = to_f64(enc.forward(to_dev(x1, "fp16"), lens))
    enc.close()
    for b, L in enumerate(c.lens):
        np.testing.assert_array_equal(b_out[b, :L], a[b, :L])


def test_null_lens_equals_full_lens():
    c, layers = _case("bert_base_fp16_s32", 1, "bert")
    enc = _encoder(c.shape, layers)
    x = to_dev(c.x, "fp16")
    a = enc.forward(x, None).clone()
    b = enc.forward(x, dev_lens(np.array([32], dtype=np.int32)))
    enc.close()
    assert torch.equal(a, b)


def test_zero_weights_reduce_to_layernorm():
    """All projection weights and biases zero: X' = LN(LN(X)) (computed here from the oracle's
    LayerNorm, which the CPU tests pin to torch's)."""
    shape = si.Shape(2, 64, 12, 64, 1, "fp16")
    c = si.custom_case(shape, 11, lens=np.array([64, 9]))
    w = {k: (np.zeros_like(v) if k.startswith(("w_", "b_")) else v) for k, v in c.layer(0).items()}
    enc = _encoder(shape, [w])
    out = to_f64(enc.forward(to_dev(c.x, "fp16"), dev_lens(c.lens)))
    enc.close()
    ones, zeros = np.ones(shape.hidden), np.zeros(shape.hidden)
    ref = oracle.layer_norm(rnd(oracle.layer_norm(c.x, ones, zeros), "fp16"), ones, zeros)
    assert_within(out, ref, 1e-2, 0.0, "zero weights")


def test_max_hidden_and_odd_heads():
    """Hidden 4096 (64 heads x 64, the largest supported) and an odd head count."""
    for shape in (si.Shape(1, 32, 64, 64, 1, "fp16"), si.Shape(3, 96, 5, 32, 2, "bf16")):
        c = si.custom_case(shape, 21, lens_range=(1, shape.seq_len), params="random_affine")
        layers = list(c.layers())
        ref = oracle.encoder(c.x, layers, c.lens, shape.head_num)
        enc = _encoder(shape, layers)
        out = to_f64(enc.forward(to_dev(c.x, shape.dtype), dev_lens(c.lens)))
        enc.close()
        tol = stack_tol(shape.dtype) if shape.num_layers > 1 else layer_tol(shape.dtype)
        check(out, ref, shape.dtype, tol, f"{shape}")


@pytest.mark.parametrize("shape", [
    si.Shape(1, 32, 24, 64, 1, "fp16"),  # hidden 1536, one sequence
    si.Shape(2, 32, 24, 64, 1, "bf16"),  # the same with the fp32 residual stream
    si.Shape(1, 32, 4, 64, 1, "fp32"),   # fp32, hidden 256
    si.Shape(3, 32, 48, 32, 1, "fp16"),  # size per head 32
    si.Shape(16, 32, 12, 64, 1, "fp16"),  # BERT-base, 512 rows: 384 tiles of 32 x 32
    si.Shape(12, 32, 12, 64, 1, "bf16"),  # 384 rows: 288 tiles of 32 x 32
    si.Shape(1, 512, 16, 64, 1, "bf16"),  # BERT-large, 512 rows: 512 tiles of 32 x 32
])
def test_split_k_paths(shape):
    """The small-batch path: at the first four shapes every projection splits K; the Q/K/V
    head split and the GELU finish their partials in the reduction, the attention-output and
    FFN-out partials are summed by the LayerNorm after them.  At the last three only the
    attention-output and FFN-out projections split (more 32 x 32 tiles than CUs, fewer
    waves than SIMDs).  One layer at the layer bar."""
    c = si.custom_case(shape, 31, lens_range=(1, shape.seq_len), params="random_affine")
    layers = list(c.layers())
    ref = oracle.encoder(c.x, layers, c.lens, shape.head_num)
    enc = _encoder(shape, layers)
    enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
    out = to_f64(enc.forward(to_dev(c.x, shape.dtype), dev_lens(c.lens)))
    enc.close()
    check(out, ref, shape.dtype, layer_tol(shape.dtype), f"{shape}")


@pytest.mark.parametrize("shape,fused", [
    (si.Shape(1, 32, 12, 64, 2, "fp16"), True),    # BERT-base heads, one sequence
    (si.Shape(2, 32, 12, 64, 1, "bf16"), True),    # the fp32 residual stream
    (si.Shape(1, 32, 24, 32, 1, "fp16"), True),    # size per head 32, hidden 768
    (si.Shape(1, 20, 16, 64, 1, "bf16"), True),    # hidden 1024 (four workgroups per head), S padded
    (si.Shape(8, 32, 12, 64, 1, "fp16"), False),   # 9 MiB of per-head partials: separate kernels
])
def test_attention_with_output_projection_partials(shape, fused):
    """Small batches at S = 32: the attention kernel also computes each head's share of the
    attention-output projection (split-K partials split by head, summed by the LayerNorm in
    head order); one launch replaces the attention and the projection (while the per-head
    partials stay within 4 MiB).  Against the oracle at the layer (one layer) or stack bar,
    with padded lengths."""
    c = si.custom_case(shape, 61 + shape.batch, lens_range=(1, shape.seq_len), params="random_affine")
    layers = list(c.layers())
    ref = oracle.encoder(c.x, layers, c.lens, shape.head_num)
    enc = _encoder(shape, layers)
    enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
    out = to_f64(enc.forward(to_dev(c.x, shape.dtype), dev_lens(c.lens)))
    t = enc.kernel_times()
    enc.close()
    assert t["attention"][1] == shape.num_layers and t["ln1"][1] == shape.num_layers
    assert t["attn_out_gemm"][1] == (0 if fused else shape.num_layers)
    tol = stack_tol(shape.dtype) if shape.num_layers > 1 else layer_tol(shape.dtype)
    print(check(out, ref, shape.dtype, tol, f"{shape}"))


@pytest.mark.parametrize("shape", [
    si.Shape(256, 32, 4, 32, 2, "fp16"),  # 8192 rows: 128 tiles of 64
    si.Shape(257, 32, 4, 32, 1, "bf16"),  # the fp32 residual stream; a partial last tile
    si.Shape(128, 64, 2, 64, 1, "fp32"),
])
def test_hidden_128_layernorm_in_the_projection(shape):
    """Hidden size 128 with at least 128 row tiles: the attention-output and FFN-out
    projections run the bias + residual + LayerNorm in their epilogue (a 64 x 128 tile holds
    whole rows); against the oracle at the stack bar, and no LayerNorm launch of its own."""
    c = si.custom_case(shape, 41, lens_range=(1, shape.seq_len), params="random_affine")
    layers = list(c.layers())
    ref = oracle.encoder(c.x, layers, c.lens, shape.head_num)
    enc = _encoder(shape, layers)
    enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
    out = to_f64(enc.forward(to_dev(c.x, shape.dtype), dev_lens(c.lens)))
    t = enc.kernel_times()
    enc.close()
    assert t["ln1"][1] == 0 and t["ln2"][1] == 0
    assert t["attn_out_gemm"][1] == shape.num_layers and t["ffn2_gemm"][1] == shape.num_layers
    check(out, ref, shape.dtype, stack_tol(shape.dtype), f"{shape}")


@pytest.mark.parametrize("shape", [
    si.Shape(64, 32, 12, 64, 2, "fp16"),   # 2048 rows: 64 x 64 attention-output tiles, 12 per row
    si.Shape(33, 64, 16, 64, 1, "fp16"),   # hidden 1024, 2112 rows: 128 x 128 tiles, last one partial
    si.Shape(20, 200, 12, 64, 1, "fp16"),  # padded length 224, ragged lengths, 4480 rows
    si.Shape(16, 128, 16, 64, 2, "bf16"),  # bf16 (Z1 also in fp32), hidden 1024, 64 x 64 tiles
    si.Shape(10, 512, 16, 64, 1, "bf16"),  # S = 512, 5120 rows: 128 x 128 attention-output tiles
    si.Shape(32, 512, 16, 64, 1, "fp16"),  # fp16 hidden 1024 at 16384 rows: 256 x 256 tiles
    si.Shape(128, 32, 12, 64, 1, "fp16"),  # 4096 rows: 128 x 96 attention-output tiles, 8 per row
    si.Shape(32, 128, 12, 64, 1, "bf16"),  # the same tiling in bf16, ragged lengths
])
def test_layernorm_fold(shape):
    """FTX_OPT_FOLD_LAYERNORM: the first LayerNorm folded into the FFN-in projection (gamma in
    the weights, beta in the bias, the row statistics from the attention-output projection's
    per-tile pairs) and rebuilt by the second LayerNorm.  No LayerNorm-1 launch; against the
    oracle at the layer / stack bar; with the fold off the LayerNorm runs on its own and the
    two agree within the stack bar.  New weights set on the handle are folded again."""
    c = si.custom_case(shape, 91 + shape.batch, lens_range=(1, shape.seq_len), params="random_affine")
    layers = list(c.layers())
    ref = oracle.encoder(c.x, layers, c.lens, shape.head_num)
    enc = _encoder(shape, layers)
    enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
    x, lens = to_dev(c.x, shape.dtype), dev_lens(c.lens)
    out = to_f64(enc.forward(x, lens))
    t = enc.kernel_times()
    assert t["ln1"][1] == 0 and t["ln2"][1] == shape.num_layers
    assert t["attn_out_gemm"][1] == shape.num_layers and t["ffn1_gemm"][1] == shape.num_layers
    tol = stack_tol(shape.dtype) if shape.num_layers > 1 else layer_tol(shape.dtype)
    print("fold", check(out, ref, shape.dtype, tol, f"{shape} fold"))
    enc.set_option(ftx.FTX_OPT_FOLD_LAYERNORM, 0)
    plain = to_f64(enc.forward(x, lens))
    t = enc.kernel_times()
    assert t["ln1"][1] == shape.num_layers
    check(plain, ref, shape.dtype, tol, f"{shape} no fold")
    assert_within(out, plain, 5e-2, 0.0 if shape.dtype == "fp16" else 2.0 ** -7, "fold vs no fold")
    # other weights into the same handle: folded again at set_weights
    c2 = si.custom_case(shape, 191 + shape.batch, lens_range=(1, shape.seq_len), params="random_affine")
    layers2 = list(c2.layers())
    for l, w in enumerate(layers2):
        enc.set_weights(l, dev_layer(w, shape.dtype))
    enc.set_option(ftx.FTX_OPT_FOLD_LAYERNORM, 1)
    out2 = to_f64(enc.forward(x, lens))
    enc.close()
    check(out2, oracle.encoder(c.x, layers2, c.lens, shape.head_num), shape.dtype, tol,
          f"{shape} fold, new weights")


@pytest.mark.parametrize("shape,auto", [
    (si.Shape(256, 32, 12, 64, 2, "fp16"), True),   # 8192 rows: FFN-out on 512 128 x 96 tiles
    (si.Shape(64, 32, 12, 64, 1, "bf16"), False),   # 2048 rows: 64 x 64 tiles, no prefetch
    (si.Shape(20, 200, 12, 64, 1, "fp16"), False),  # 4480 rows (ragged lengths): 280 tiles
])
def test_weight_prefetch(shape, auto):
    """FTX_OPT_PREFETCH_WEIGHTS: a kernel that reads W2 ahead of the second FFN projection on
    the folded path.  Automatic (1): one launch per layer where that projection runs on
    128-row tiles, at least 1.5 per CU, else none; forced (2): one per layer; never (0):
    none.  It writes nothing, so the three outputs are equal bit for bit, and they match the
    oracle at the stack bar.  Modes outside 0..2 are refused."""
    c = si.custom_case(shape, 57 + shape.batch, lens_range=(1, shape.seq_len), params="random_affine")
    layers = list(c.layers())
    enc = _encoder(shape, layers)
    enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
    x, lens = to_dev(c.x, shape.dtype), dev_lens(c.lens)
    outs = {}
    for mode in (1, 2, 0):
        enc.set_option(ftx.FTX_OPT_PREFETCH_WEIGHTS, mode)
        outs[mode] = enc.forward(x, lens).clone()
        t = enc.kernel_times()
        assert t["ln1"][1] == 0, "the prefetch runs on the folded path"
        want = shape.num_layers if mode == 2 or (mode == 1 and auto) else 0
        assert t["weight_prefetch"][1] == want, (mode, t["weight_prefetch"])
    with pytest.raises(ftx.FtxError):
        enc.set_option(ftx.FTX_OPT_PREFETCH_WEIGHTS, 3)
    enc.close()
    assert torch.equal(outs[1], outs[0]) and torch.equal(outs[2], outs[0])
    ref = oracle.encoder(c.x, layers, c.lens, shape.head_num)
    tol = stack_tol(shape.dtype) if shape.num_layers > 1 else layer_tol(shape.dtype)
    print("prefetch", check(to_f64(outs[1]), ref, shape.dtype, tol, f"{shape} prefetch"))


@pytest.mark.parametrize("shape,with_lens", [
    (si.Shape(3, 100, 4, 32, 2, "fp16"), True),
    (si.Shape(2, 100, 4, 32, 2, "fp16"), False),   # no seq_lens: keys limited to 100
    (si.Shape(2, 1, 12, 64, 1, "fp32"), False),    # a single token
    (si.Shape(2, 33, 2, 64, 2, "bf16"), True),
    (si.Shape(1, 511, 2, 64, 1, "fp16"), True),
    (si.Shape(4, 70, 12, 64, 1, "fp32"), True),
])
def test_ragged_sequence_lengths(shape, with_lens):
    """Sequence lengths that are not a multiple of 32 (padded inside the handle)."""
    c = si.custom_case(shape, 31 + shape.seq_len, params="random_affine",
                       lens_range=(1, shape.seq_len) if with_lens else None)
    layers = list(c.layers())
    ref = oracle.encoder(c.x, layers, c.lens, shape.head_num)
    enc = _encoder(shape, layers)
    out = to_f64(enc.forward(to_dev(c.x, shape.dtype), dev_lens(c.lens)))
    enc.close()
    tol = stack_tol(shape.dtype) if shape.num_layers > 1 else layer_tol(shape.dtype)
    check(out, ref, shape.dtype, tol, f"{shape} lens={with_lens}")


@pytest.mark.parametrize("workload,batch,seq", [("bert_base_fp16_s32", 8, None),
                                                ("bert_base_fp16_s128_varlen", 2, None),
                                                ("bert_base_fp16_s32", 3, 100),
                                                ("bert_base_fp16_s32", 64, None)])  # folded LN
def test_graph_mode_replays_match_eager(workload, batch, seq):
    """FTX_OPT_GRAPH: every replay equals the eager forward bitwise, with eager work on the
    same stream between replays; new buffers trigger a new capture."""
    c, layers = _case(workload, batch, "random_affine")
    shape = c.shape if seq is None else si.Shape(batch, seq, c.shape.head_num, c.shape.size_per_head,
                                                  c.shape.num_layers, c.shape.dtype)
    if seq is not None:
        c = si.custom_case(shape, 77, params="random_affine", lens_range=(1, seq))
        layers = list(c.layers())
    enc = _encoder(shape, layers)
    x = to_dev(c.x, shape.dtype)
    lens = dev_lens(c.lens)
    ref = enc.forward(x, lens).clone()
    oref = oracle.encoder(c.x, layers, c.lens, shape.head_num)
    print("eager", check(to_f64(ref), oref, shape.dtype, stack_tol(shape.dtype), "eager"))
    enc.set_option(ftx.FTX_OPT_GRAPH, 1)
    out = torch.empty_like(ref)
    for i in range(4):
        out.fill_(float("nan"))
        enc.forward(x, lens, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        check(to_f64(out), oref, shape.dtype, stack_tol(shape.dtype), f"replay {i}")
        junk = (x.float() * 3).sum()  # eager work on the stream between replays
        torch.cuda.synchronize()
    out2 = torch.empty_like(ref)
    enc.forward(x, lens, out2)           # new output buffer: captured again
    torch.cuda.synchronize()
    assert torch.equal(out2, ref)
    check(to_f64(out2), oref, shape.dtype, stack_tol(shape.dtype), "new capture")
    enc.set_option(ftx.FTX_OPT_GRAPH, 0)
    assert torch.equal(enc.forward(x, lens), ref)
    enc.close()
    del junk


def test_fold_option_under_graph_replay():
    """Switching FTX_OPT_FOLD_LAYERNORM while graph replay is on drops the captured forward:
    each replay equals the eager forward of the path the option selects, bit for bit."""
    c, layers = _case("bert_base_fp16_s32", 64, "random_affine")
    enc = _encoder(c.shape, layers)
    x, lens = to_dev(c.x, "fp16"), dev_lens(c.lens)
    folded = enc.forward(x, lens).clone()
    enc.set_option(ftx.FTX_OPT_FOLD_LAYERNORM, 0)
    plain = enc.forward(x, lens).clone()
    assert not torch.equal(folded, plain)  # the two paths round differently
    enc.set_option(ftx.FTX_OPT_FOLD_LAYERNORM, 1)
    enc.set_option(ftx.FTX_OPT_GRAPH, 1)
    out = torch.empty_like(folded)
    for fold, ref in ((1, folded), (0, plain), (1, folded)):
        enc.set_option(ftx.FTX_OPT_FOLD_LAYERNORM, fold)
        for _ in range(2):
            out.fill_(float("nan"))
            enc.forward(x, lens, out)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"fold={fold}"
    enc.close()


def test_torch_operator_matches_the_oracle_and_the_c_abi():
    """torch.ops.ftx.encoder_forward (and the nn.Module around it) against the fp64 oracle at
    the stack bar, on padded lengths, and bitwise equal to ftx_forward."""
    from transformer_encoder_bert_amd import torch_op
    c, layers = _case("bert_base_fp16_s128_varlen", 4, "random_affine")
    enc = _encoder(c.shape, layers)
    x = to_dev(c.x, "fp16")
    lens = dev_lens(c.lens)
    ref = enc.forward(x, lens).clone()
    mod = torch_op.EncoderModule(enc)
    got = mod(x, lens)
    oref = oracle.encoder(c.x, layers, c.lens, c.shape.head_num)
    print(check(to_f64(got), oref, "fp16", stack_tol("fp16"), "torch operator"))
    assert torch.equal(got, ref)
    got2 = torch.ops.ftx.encoder_forward(x, lens, mod.op_id)
    check(to_f64(got2), oref, "fp16", stack_tol("fp16"), "torch operator, direct call")
    assert torch.equal(got2, ref)
    with pytest.raises(ValueError):     # not [B][S][H]
        torch.ops.ftx.encoder_forward(x.view(-1, x.shape[-1]), lens, mod.op_id)
    mod.close()


def test_errors_on_device():
    c, layers = _case("single_layer_fp32", 1, "bert")
    enc = ftx.Encoder(1, 32, 4, 32, 1, "fp32")
    x = to_dev(c.x, "fp32")
    with pytest.raises(ftx.FtxError) as e:
        enc.forward(x)
    assert e.value.status == ftx.FTX_ERR_NOT_READY
    enc.set_weights(0, dev_layer(layers[0], "fp32"))
    with pytest.raises(ftx.FtxError) as e:     # output aliasing the input
        ftx.ftx_forward(enc.handle, x, None, x)
    assert e.value.status == ftx.FTX_ERR_INVALID_ARG
    with pytest.raises(ftx.FtxError):          # layer out of range
        enc.set_weights(1, dev_layer(layers[0], "fp32"))
    enc.close()


def test_kernel_timing_counts_launches():
    c, layers = _case("bert_base_fp16_s32", 1, "bert")
    enc = _encoder(c.shape, layers)
    enc.set_option(ftx.FTX_OPT_KERNEL_TIMING, 1)
    x = to_dev(c.x, "fp16")
    enc.forward(x)
    t = enc.kernel_times()
    assert t["qkv_gemm"][1] == 12 and t["ln2"][1] == 12 and t["bias_gelu"][1] == 0
    assert all(ms >= 0 for ms, _ in t.values())
    enc.set_option(ftx.FTX_OPT_FUSED_EPILOGUES, 0)
    enc.forward(x)
    t = enc.kernel_times()
    assert t["bias_gelu"][1] == 12 and t["bias_qkv_split"][1] == 12
    enc.close()


# ------------------------------------------------------------------ full sizes, sampled rows

def tile_sample(batch: int, seq_len: int, seed: int):
    """Sequences the oracle checks at a full batch: all of them up to 64 sequences; above,
    one seeded sequence from every 256-row tile of the projections (256 / seq_len sequences
    per tile, at least one), so every tile of the benchmark's grid is covered."""
    if batch <= 64:
        return list(range(batch))
    per_tile = max(1, 256 // seq_len)
    rng = np.random.default_rng(seed)
    rows = []
    for first in range(0, batch, per_tile):
        rows.append(first + int(rng.integers(0, min(per_tile, batch - first))))
    return rows


# Every (workload, batch) the benchmark reports, in the launch configuration it times
# (default options).  BERT-large checks two sequences: its oracle takes about a second per
# sequence, where BERT-base takes 20 ms.
FULL = [
    ("bert_base_fp16_s32", 512, None),
    ("bert_base_fp16_s32", 256, None),
    ("bert_base_fp16_s32", 128, None),
    ("bert_base_fp16_s32", 64, None),
    ("bert_base_fp16_s32", 8, None),
    ("bert_base_fp16_s32", 1, None),
    ("pruned_fp16_s32", 512, None),
    ("pruned_fp16_s32", 64, None),
    ("pruned_fp16_s32", 1, None),
    ("bert_base_fp16_s64_varlen", 64, None),
    ("bert_base_fp16_s64_varlen", 1, None),
    ("bert_base_fp16_s128_varlen", 64, None),
    ("bert_base_fp16_s128_varlen", 1, None),
    ("bert_large_bf16_s128", 256, [0, 200]),
    ("bert_large_bf16_s512", 32, [7, 31]),
    ("bert_large_bf16_s512", 1, None),   # FFN-out partials on 64x64 tiles, 32x32 on three stages
]


@pytest.mark.parametrize("workload,batch,rows", FULL)
def test_full_size_sampled_rows(workload, batch, rows):
    """The whole batch at its full size, in the launch configuration the benchmark times;
    the oracle checks the sampled sequences (sequences are independent)."""
    c, layers = _case(workload, batch)
    if rows is None:
        rows = tile_sample(batch, c.shape.seq_len, seed=batch + c.shape.seq_len)
    enc = _encoder(c.shape, layers)
    out = enc.forward(to_dev(c.x, c.shape.dtype), dev_lens(c.lens))
    got = to_f64(out[rows])
    enc.close()
    ref = oracle.encoder_rows(c.x, layers, c.lens, c.shape.head_num, rows)
    rep = check(got, ref, c.shape.dtype, stack_tol(c.shape.dtype),
                f"{workload} B={batch} {len(rows)} sequences")
    print(f"{workload} B={batch}: {len(rows)} of {batch} sequences checked, {rep}")
