"""Per-step parity of the HIP kernels against the fp64 oracle, through the C ABI's
step entry points (include/ftx_steps.h).

Tolerances are derived from the arithmetic, with u the storage format's unit roundoff:
* every output is rounded once to the storage format: rtol = 2u (one ulp);
* projections accumulate in fp32 in any order: the recursive-summation bound
  gamma_K * (|A| |W|) with gamma_K = K u32 / (1 - K u32), u32 = 2^-24, elementwise;
* attention feeds the probabilities to the P V product in the storage format, which adds
  at most u * max|v| per output: atol = 2u * max|v| (+1e-6 for the fp32 exp);
* LayerNorm statistics in fp32: atol = 2e-5 on O(1) normalised outputs.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (DEV, TORCH, UNIT, announce, assert_within, dev_lens, need_gpu, rnd, to_dev,
                      to_f64)
from transformer_encoder_bert_amd import ftx

pytestmark = pytest.mark.gpu
DTYPES = ["fp32", "fp16", "bf16"]


@pytest.fixture(autouse=True)
def _gpu(request):
    need_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _rand(rng, shape, dtype, scale=1.0):
    return rnd(rng.normal(size=shape) * scale, dtype)


def _sum_bound(K, abs_products):
    """Rounding bound of an fp32 sum of K products in any order: gamma_K * sum |a_k w_k|."""
    u32 = 2.0 ** -24
    return K * u32 / (1 - K * u32) * abs_products


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,cols", [(1, 1), (7, 13), (64, 64), (768, 3072), (100, 33)])
def test_transpose_exact(dtype, rows, cols):
    rng = np.random.default_rng(rows * 1000 + cols)
    a = _rand(rng, (rows, cols), dtype)
    out = torch.empty((cols, rows), dtype=TORCH[dtype], device=DEV)
    ftx.ftx_step_transpose(to_dev(a, dtype), out)
    np.testing.assert_array_equal(to_f64(out), a.T)


# ------------------------------------------------------------------------------ projections

LINEAR_SHAPES = [
    (32, 384, 128),      # single-layer config QKV
    (32, 128, 512),      # single-layer config FFN-out
    (1, 64, 64),         # one row
    (33, 72, 40),        # ragged M, N and K tails
    (257, 136, 200),     # ragged, several 64x64 tiles
    (1024, 768, 768),    # 128x128 tiles
    (2048, 3072, 768),   # FFN-in shape family
    (4096, 2312, 768),   # 256x192 tiles with a ragged N tail
    (16416, 768, 768),   # 256x128 tiles with a ragged M tail
    (16384, 3072, 768),  # 256x256 tiles (BERT-base FFN-in at batch 512)
    # 256-row tiles with 12 slabs or more take the ping-pong K loop (16-bit dtypes; so do the
    # 256x256 and 256x192 shapes above)
    (16384, 768, 3072),  # 256x192 tiles (BERT-base FFN-out at batch 512)
    (16416, 768, 3072),  # 256x256 tiles with a ragged M tail
    (4000, 4040, 2048),  # 256x256 tiles with ragged M and N tails
    # 128x128 tiles with no more blocks than CUs and 12 slabs or more: three LDS stages;
    # where N is a multiple of 96 and that grid also fits the CUs, 128x96 tiles
    (4096, 768, 3072),   # BERT-base FFN-out at 4096 rows (256 tiles of 128 x 96)
    (3000, 768, 768),    # 128 x 96 with a ragged M tail (192 tiles)
    (6000, 768, 3072),   # 128 x 96, two blocks per CU (376 tiles), ragged M
    (4000, 776, 1576),   # ragged M, N and K tails (224 tiles of 128 x 128)
    # 64x64 tiles with 12 slabs or more keep two slabs in flight (three LDS stages)
    (2048, 768, 768),    # BERT-base attention output at batch 64 (12 slabs)
    (2048, 768, 3072),   # BERT-base FFN-out at batch 64
    (2000, 776, 1576),   # ragged M, N and K tails (the last slab is partly zeroed)
    # the small-M kernel (K split over the 4 waves of one workgroup per tile, whole slabs):
    # 32-row tiles ...
    (32, 2304, 768),     # BERT-base Q/K/V at batch 1
    (31, 3072, 768),     # FFN-in with a ragged last row tile
    (64, 768, 1024),     # 16 slabs: four per wave
    # ... and 64-row tiles where 32-row tiles would outnumber the CUs
    (128, 2304, 768),    # Q/K/V at 128 rows (BERT-base S128 batch 1)
    (96, 3072, 768),     # 64-row tiles with an empty second row tile in the last one
    (160, 2304, 512),    # three row tiles of 64, the last one half empty
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N,K", LINEAR_SHAPES)
@pytest.mark.parametrize("epi", ["none", "bias", "bias_gelu"])
def test_linear(dtype, M, N, K, epi):
    rng = np.random.default_rng(M * 7 + N * 11 + K)
    a = _rand(rng, (M, K), dtype)
    w = _rand(rng, (K, N), dtype, 0.05)
    b = _rand(rng, (N,), dtype, 0.5)
    bias = None if epi == "none" else b
    ref = oracle.linear(a, w, bias if bias is not None else np.zeros(N))
    if epi == "bias_gelu":
        ref = oracle.gelu_tanh(ref)
    c = torch.empty((M, N), dtype=TORCH[dtype], device=DEV)
    ftx.ftx_step_linear(to_dev(a, dtype), to_dev(np.ascontiguousarray(w.T), dtype),
                        None if bias is None else to_dev(bias, dtype), epi == "bias_gelu", c)
    u = UNIT[dtype]
    # GELU has slope <= 1.13, so the summation bound carries through it
    atol = 1.13 * _sum_bound(K, np.abs(a) @ np.abs(w)) + 1e-7
    assert_within(to_f64(c), ref, atol=atol, rtol=2 * u + (4e-6 if dtype == "fp32" else 0), what="linear")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B,S,n,d", [(1, 32, 4, 32), (2, 64, 3, 64), (3, 128, 2, 32), (1, 512, 2, 64),
                                     (64, 128, 12, 64), (32, 32, 12, 64)])
def test_qkv_projection(dtype, B, S, n, d):
    H = n * d
    rng = np.random.default_rng(B + S + n + d)
    x = _rand(rng, (B, S, H), dtype)
    wq, wk, wv = (_rand(rng, (H, H), dtype, 0.05) for _ in range(3))
    bq, bk, bv = (_rand(rng, (H,), dtype, 0.5) for _ in range(3))
    q_ref = oracle.split_heads(oracle.linear(x, wq, bq), n)
    k_ref = oracle.split_heads(oracle.linear(x, wk, bk), n)
    v_ref = oracle.split_heads(oracle.linear(x, wv, bv), n)
    w_t = np.concatenate([wq.T, wk.T, wv.T], axis=0)
    q = torch.empty((B, n, S, d), dtype=TORCH[dtype], device=DEV)
    k = torch.empty_like(q)
    vt = torch.empty((B, n, d, S), dtype=TORCH[dtype], device=DEV)
    ftx.ftx_step_qkv_projection(B, S, n, d, to_dev(x, dtype), to_dev(w_t, dtype),
                                to_dev(np.concatenate([bq, bk, bv]), dtype), q, k, vt)
    u = UNIT[dtype]
    bnd = lambda wm: oracle.split_heads(_sum_bound(H, np.abs(x) @ np.abs(wm)), n) + 1e-7
    assert_within(to_f64(q), q_ref, bnd(wq), 2 * u, "q")
    assert_within(to_f64(k), k_ref, bnd(wk), 2 * u, "k")
    assert_within(to_f64(vt), np.swapaxes(v_ref, -1, -2), np.swapaxes(bnd(wv), -1, -2), 2 * u, "v_t")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B,S,n,d", [(1, 32, 4, 32), (2, 64, 3, 64), (2, 128, 12, 64)])
def test_bias_qkv_split(dtype, B, S, n, d):
    H = n * d
    rng = np.random.default_rng(3 * B + S + n + d)
    qkv = _rand(rng, (B * S, 3 * H), dtype)
    b = _rand(rng, (3 * H,), dtype)
    ref = rnd(qkv + b, dtype).reshape(B, S, 3 * H)
    q = torch.empty((B, n, S, d), dtype=TORCH[dtype], device=DEV)
    k = torch.empty_like(q)
    vt = torch.empty((B, n, d, S), dtype=TORCH[dtype], device=DEV)
    ftx.ftx_step_bias_qkv_split(B, S, n, d, to_dev(qkv, dtype), to_dev(b, dtype), q, k, vt)
    u = UNIT[dtype]
    assert_within(to_f64(q), oracle.split_heads(ref[..., :H], n), 0, 2 * u, "q")
    assert_within(to_f64(k), oracle.split_heads(ref[..., H:2 * H], n), 0, 2 * u, "k")
    assert_within(to_f64(vt), np.swapaxes(oracle.split_heads(ref[..., 2 * H:], n), -1, -2), 0, 2 * u, "v_t")


# ------------------------------------------------------------------------------ attention

ATTN_CASES = [
    (1, 32, 4, 32, None),
    (1, 32, 4, 32, [17]),
    (2, 64, 3, 64, [1, 64]),         # one-key sequence (one-hot), full sequence
    (3, 128, 2, 64, [33, 96, 128]),  # ragged key tails across tiles
    (2, 128, 2, 32, [128, 5]),
    (2, 512, 2, 64, [512, 200]),     # several softmax chunks
    (1, 512, 1, 64, [64]),
    (2, 96, 2, 64, [96, 40]),        # S not a power of two
    (2, 32, 3, 64, [32, 9]),         # S = 32, few heads: the kernel without LDS
    (172, 32, 12, 64, None),         # S = 32, over 2048 heads: the LDS kernel
    (9, 512, 1, 32, [1, 127, 128, 129, 256, 257, 384, 385, 512]),  # every count of 128-key chunks
    (8, 256, 2, 64, [256, 1, 100, 129, 200, 33, 255, 64]),          # 16 heads: query groups renumbered by XCD
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("B,S,n,d,lens", ATTN_CASES)
def test_attention(dtype, B, S, n, d, lens):
    rng = np.random.default_rng(B * 100 + S + n * 7 + d)
    q = _rand(rng, (B, n, S, d), dtype, 1.0)
    k = _rand(rng, (B, n, S, d), dtype, 1.0)
    v = _rand(rng, (B, n, S, d), dtype, 1.0)
    lens_np = None if lens is None else np.array(lens, dtype=np.int32)
    ref = oracle.merge_heads(oracle.context(oracle.masked_softmax(oracle.scaled_scores(q, k), lens_np), v))
    ctx = torch.empty((B, S, n * d), dtype=TORCH[dtype], device=DEV)
    ftx.ftx_step_attention(B, S, n, d, to_dev(q, dtype), to_dev(k, dtype),
                           to_dev(np.ascontiguousarray(np.swapaxes(v, -1, -2)), dtype),
                           dev_lens(lens_np), ctx)
    u = UNIT[dtype]
    vmax = np.abs(v).max()
    atol = (2 * u if dtype != "fp32" else 1e-6) * vmax + 1e-6
    assert_within(to_f64(ctx), ref, atol, 2 * u, "ctx")


@pytest.mark.parametrize("dtype", ["fp16"])
def test_attention_lens_are_clamped(dtype):
    """Lengths outside [1, S] are clamped on the device: 0 behaves as 1, S+5 as S."""
    B, S, n, d = 2, 64, 2, 64
    rng = np.random.default_rng(9)
    q, k, v = (_rand(rng, (B, n, S, d), dtype) for _ in range(3))
    args = [to_dev(q, dtype), to_dev(k, dtype), to_dev(np.ascontiguousarray(np.swapaxes(v, -1, -2)), dtype)]
    outs = []
    for lens in ([0, S + 5], [1, S]):
        ctx = torch.empty((B, S, n * d), dtype=TORCH[dtype], device=DEV)
        ftx.ftx_step_attention(B, S, n, d, *args, dev_lens(np.array(lens, dtype=np.int32)), ctx)
        outs.append(to_f64(ctx))
    np.testing.assert_array_equal(outs[0], outs[1])


# ------------------------------------------------------------------------------ LayerNorm, GELU

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,cols", [(1, 128), (33, 768), (64, 1024), (5, 96), (7, 2048), (3, 4096),
                                       (4, 200), (2, 36), (3, 260), (2, 1000), (9, 384), (5, 512)])
def test_bias_residual_layernorm(dtype, rows, cols):
    rng = np.random.default_rng(rows * 3 + cols)
    x = _rand(rng, (rows, cols), dtype)
    a = _rand(rng, (rows, cols), dtype, 0.5)
    b = _rand(rng, (cols,), dtype, 0.2)
    g = _rand(rng, (cols,), dtype, 0.3) + 1.0
    g = rnd(g, dtype)
    be = _rand(rng, (cols,), dtype, 0.2)
    ref = oracle.layer_norm(x + a + b, g, be)
    y = torch.empty((rows, cols), dtype=TORCH[dtype], device=DEV)
    ftx.ftx_step_bias_residual_layernorm(to_dev(x, dtype), to_dev(a, dtype), to_dev(b, dtype),
                                         to_dev(g, dtype), to_dev(be, dtype), y)
    assert_within(to_f64(y), ref, 2e-5, 2 * UNIT[dtype], "layernorm")


@pytest.mark.parametrize("dtype", DTYPES)
def test_layernorm_in_place_and_moments(dtype):
    rows, cols = 16, 768
    rng = np.random.default_rng(77)
    x = _rand(rng, (rows, cols), dtype, 3.0)
    zeros = np.zeros(cols)
    ones = np.ones(cols)
    xd = to_dev(x, dtype)
    ad = to_dev(np.zeros((rows, cols)), dtype)
    ftx.ftx_step_bias_residual_layernorm(xd, ad, to_dev(zeros, dtype), to_dev(ones, dtype),
                                         to_dev(zeros, dtype), xd)  # y aliases x
    y = to_f64(xd)
    assert np.abs(y.mean(-1)).max() < 4 * UNIT[dtype] + 1e-6
    var = x.var(-1)
    np.testing.assert_allclose(y.var(-1), var / (var + 1e-6), rtol=8 * UNIT[dtype] + 1e-5)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,cols", [(1, 8), (32, 512), (100, 3072), (3, 4096)])
def test_bias_gelu(dtype, rows, cols):
    rng = np.random.default_rng(rows + cols)
    u = _rand(rng, (rows, cols), dtype, 3.0)
    b = _rand(rng, (cols,), dtype, 0.5)
    ref = oracle.gelu_tanh(u + b)
    g = torch.empty((rows, cols), dtype=TORCH[dtype], device=DEV)
    ftx.ftx_step_bias_gelu(to_dev(u, dtype), to_dev(b, dtype), g)
    assert_within(to_f64(g), ref, 1e-6, 2 * UNIT[dtype] + 2e-6, "bias_gelu")
