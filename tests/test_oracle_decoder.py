"""Pins of the fp64 decoder oracle against things other than itself (CPU only).

The decoder is a reading (the FT article's section "什么是 Faster Transformer" names it only
as a roadmap item): the encoder layer of the same article with a causal mask on the
self-attention and a post-LN cross-attention sub-layer over the memory.  Pinned against:

* an independent library routine: ``torch.nn.TransformerDecoderLayer`` in float64 (post-LN,
  tanh GELU, eps 1e-6, causal target mask, memory key-padding mask);
* brute-force scalar loops on a tiny shape;
* invariants the definition fixes exactly: causality (later decoder rows do not reach
  earlier outputs), padded memory rows do not reach any output, the causal mask's
  structure;
* special cases that reduce to simpler computations: one decoder position (self-attention
  is the value projection), one valid memory key (every query's cross context is that
  key's value), the last causal row (equal to unmasked attention), zero weights
  (LayerNorm only).

``test_planted_mistakes`` plants plausible slips in the oracle and checks a pin notices.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.fp64_decoder as dec
from synthetic_inputs import DecoderShape, make_decoder_case


def _case(B=2, Sd=5, Se=6, n=2, d=4, L=2, seed=11, mem_lens=(4, 6), params="random_affine", std=0.4):
    sh = DecoderShape(B, Sd, Se, n, d, L, "fp32")
    return make_decoder_case(sh, seed, params=params, weight_std=std,
                             mem_lens=None if mem_lens is None else np.array(mem_lens))


# ------------------------------------------------------------------- library routine

def _torch_decoder_layer(x, mem, w, mem_lens, n):
    H = x.shape[-1]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    layer = torch.nn.TransformerDecoderLayer(
        d_model=H, nhead=n, dim_feedforward=4 * H, dropout=0.0,
        activation=lambda u: F.gelu(u, approximate="tanh"), layer_norm_eps=1e-6,
        batch_first=True, norm_first=False, dtype=torch.float64)
    layer.eval()
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(t(np.concatenate([w["w_q"].T, w["w_k"].T, w["w_v"].T], 0)))
        layer.self_attn.in_proj_bias.copy_(t(np.concatenate([w["b_q"], w["b_k"], w["b_v"]])))
        layer.self_attn.out_proj.weight.copy_(t(w["w_o"].T))
        layer.self_attn.out_proj.bias.copy_(t(w["b_o"]))
        layer.multihead_attn.in_proj_weight.copy_(t(np.concatenate([w["w_q2"].T, w["w_k2"].T, w["w_v2"].T], 0)))
        layer.multihead_attn.in_proj_bias.copy_(t(np.concatenate([w["b_q2"], w["b_k2"], w["b_v2"]])))
        layer.multihead_attn.out_proj.weight.copy_(t(w["w_o2"].T))
        layer.multihead_attn.out_proj.bias.copy_(t(w["b_o2"]))
        layer.linear1.weight.copy_(t(w["w_ffn1"].T))
        layer.linear1.bias.copy_(t(w["b_ffn1"]))
        layer.linear2.weight.copy_(t(w["w_ffn2"].T))
        layer.linear2.bias.copy_(t(w["b_ffn2"]))
        for i in (1, 2, 3):
            getattr(layer, f"norm{i}").weight.copy_(t(w[f"ln{i}_gamma"]))
            getattr(layer, f"norm{i}").bias.copy_(t(w[f"ln{i}_beta"]))
    Sd, Se = x.shape[1], mem.shape[1]
    causal = torch.triu(torch.full((Sd, Sd), float("-inf"), dtype=torch.float64), diagonal=1)
    pad = None
    if mem_lens is not None:
        pad = torch.from_numpy(np.arange(Se)[None, :] >= np.asarray(mem_lens)[:, None])
    with torch.no_grad():
        y = layer(t(x), t(mem), tgt_mask=causal, memory_key_padding_mask=pad)
    return y.numpy()


@pytest.mark.parametrize("mem_lens", [(4, 6), None, (1, 2)])
def test_matches_torch_decoder_layer(mem_lens):
    c = _case(mem_lens=mem_lens)
    for w in c.layers():
        got = oracle.decoder_layer(c.x, c.mem, w, c.mem_lens, c.shape.head_num)
        ref = _torch_decoder_layer(c.x, c.mem, w, c.mem_lens, c.shape.head_num)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


def test_stack_matches_torch_layer_by_layer():
    c = _case(L=3)
    h = c.x
    for w in c.layers():
        h = _torch_decoder_layer(h, c.mem, w, c.mem_lens, c.shape.head_num)
    got = oracle.decoder(c.x, c.mem, list(c.layers()), c.mem_lens, c.shape.head_num)
    np.testing.assert_allclose(got, h, rtol=0, atol=1e-10)


# ------------------------------------------------------------------- brute force

def _bf_layer(x, mem, w, mem_len, n):
    """Scalar loops over one sequence: x [Sd][H], mem [Se][H] as nested lists."""
    Sd, Se, H = len(x), len(mem), len(x[0])
    d = H // n

    def lin(rows, W, b):
        return [[sum(r[i] * W[i][j] for i in range(len(r))) + b[j] for j in range(len(b))] for r in rows]

    def ln(rows, g, bb):
        out = []
        for r in rows:
            mu = sum(r) / H
            var = sum((v - mu) ** 2 for v in r) / H
            out.append([g[j] * (r[j] - mu) / math.sqrt(var + 1e-6) + bb[j] for j in range(H)])
        return out

    def attn(Q, K, V, allowed):
        ctx = [[0.0] * H for _ in Q]
        for h in range(n):
            for i in range(len(Q)):
                keys = [j for j in range(len(K)) if allowed(i, j)]
                s = [sum(Q[i][h * d + e] * K[j][h * d + e] for e in range(d)) / math.sqrt(d) for j in keys]
                m = max(s)
                ex = [math.exp(v - m) for v in s]
                tot = sum(ex)
                for e in range(d):
                    ctx[i][h * d + e] = sum(ex[t] / tot * V[keys[t]][h * d + e] for t in range(len(keys)))
        return ctx

    g = lambda u: 0.5 * u * (1 + math.tanh(math.sqrt(2 / math.pi) * (u + 0.044715 * u * u * u)))
    L = lambda k: w[k].tolist()
    q, k, v = lin(x, L("w_q"), L("b_q")), lin(x, L("w_k"), L("b_k")), lin(x, L("w_v"), L("b_v"))
    a = lin(attn(q, k, v, lambda i, j: j <= i), L("w_o"), L("b_o"))
    y1 = ln([[x[i][j] + a[i][j] for j in range(H)] for i in range(Sd)], L("ln1_gamma"), L("ln1_beta"))
    q2 = lin(y1, L("w_q2"), L("b_q2"))
    k2, v2 = lin(mem, L("w_k2"), L("b_k2")), lin(mem, L("w_v2"), L("b_v2"))
    c2 = lin(attn(q2, k2, v2, lambda i, j: j < mem_len), L("w_o2"), L("b_o2"))
    y2 = ln([[y1[i][j] + c2[i][j] for j in range(H)] for i in range(Sd)], L("ln2_gamma"), L("ln2_beta"))
    u = lin(y2, L("w_ffn1"), L("b_ffn1"))
    z = lin([[g(t) for t in r] for r in u], L("w_ffn2"), L("b_ffn2"))
    return ln([[y2[i][j] + z[i][j] for j in range(H)] for i in range(Sd)], L("ln3_gamma"), L("ln3_beta"))


def test_brute_force_tiny():
    c = _case(B=2, Sd=3, Se=4, n=2, d=2, L=1, mem_lens=(3, 4))
    w = c.layer(0)
    got = oracle.decoder_layer(c.x, c.mem, w, c.mem_lens, 2)
    for b in range(2):
        ref = np.array(_bf_layer(c.x[b].tolist(), c.mem[b].tolist(), w, int(c.mem_lens[b]), 2))
        np.testing.assert_allclose(got[b], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------- exact invariants

def test_causal_softmax_structure():
    rng = np.random.default_rng(3)
    s = rng.normal(size=(2, 3, 6, 6)) * 4
    p = oracle.causal_softmax(s)
    assert np.all(np.triu(p[..., :, :], k=1) == 0.0)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-15)
    assert np.all(p[..., 0, 0] == 1.0)
    # row i equals the plain softmax of its first i + 1 scores
    for i in range(6):
        e = np.exp(s[..., i, : i + 1] - s[..., i, : i + 1].max(-1, keepdims=True))
        np.testing.assert_allclose(p[..., i, : i + 1], e / e.sum(-1, keepdims=True), rtol=1e-14, atol=0)


def test_causality_exact():
    c = _case(Sd=6)
    layers = list(c.layers())
    base = oracle.decoder(c.x, c.mem, layers, c.mem_lens, c.shape.head_num)
    rng = np.random.default_rng(5)
    for i in range(c.shape.tgt_len - 1):
        x1 = c.x.copy()
        x1[:, i + 1:] = rng.normal(size=x1[:, i + 1:].shape) * 3
        out = oracle.decoder(x1, c.mem, layers, c.mem_lens, c.shape.head_num)
        np.testing.assert_array_equal(out[:, : i + 1], base[:, : i + 1])
        assert not np.allclose(out[:, i + 1:], base[:, i + 1:])


def test_padded_memory_rows_do_not_reach_outputs():
    c = _case(mem_lens=(2, 5))
    layers = list(c.layers())
    base = oracle.decoder(c.x, c.mem, layers, c.mem_lens, c.shape.head_num)
    m1 = c.mem.copy()
    rng = np.random.default_rng(8)
    for b, L in enumerate(c.mem_lens):
        m1[b, L:] = rng.normal(size=m1[b, L:].shape) * 5
    np.testing.assert_array_equal(oracle.decoder(c.x, m1, layers, c.mem_lens, c.shape.head_num), base)


# ------------------------------------------------------------------- special cases

def test_single_position_self_attention_is_the_value_projection():
    c = _case(Sd=1)
    w = c.layer(0)
    st = oracle.decoder_layer_steps(c.x, c.mem, w, c.mem_lens, c.shape.head_num)
    v_proj = oracle.linear(oracle.linear(c.x, w["w_v"], w["b_v"]), w["w_o"], w["b_o"])
    np.testing.assert_allclose(st["attn"], v_proj, rtol=1e-14, atol=1e-14)


def test_one_valid_memory_key():
    c = _case(mem_lens=(1, 1))
    w = c.layer(0)
    st = oracle.decoder_layer_steps(c.x, c.mem, w, c.mem_lens, c.shape.head_num)
    # every query's cross context is the projected value of memory position 0
    v0 = oracle.linear(c.mem[:, :1], w["w_v2"], w["b_v2"])
    np.testing.assert_allclose(st["ctx2"], np.broadcast_to(v0, st["ctx2"].shape), rtol=0, atol=1e-14)


def test_last_causal_row_is_unmasked_attention():
    c = _case()
    w = c.layer(0)
    st = oracle.decoder_layer_steps(c.x, c.mem, w, c.mem_lens, c.shape.head_num)
    full = oracle.layer_steps(c.x, w, None, c.shape.head_num)  # the encoder's unmasked attention
    np.testing.assert_allclose(st["ctx"][:, -1], full["ctx"][:, -1], rtol=0, atol=1e-14)
    assert not np.allclose(st["ctx"][:, 0], full["ctx"][:, 0])


def test_zero_weights_reduce_to_layernorm():
    c = _case(params="bert")
    w = {k: np.zeros_like(v) if k.startswith(("w_", "b_")) else v for k, v in c.layer(0).items()}
    out = oracle.decoder_layer(c.x, c.mem, w, c.mem_lens, c.shape.head_num)
    # three LayerNorms of LN(x): each leaves unit variance up to epsilon
    np.testing.assert_allclose(out, oracle.layer_norm(c.x, np.ones(8), np.zeros(8)), rtol=0, atol=1e-5)


# ------------------------------------------------------------------- planted mistakes

def _unmasked_softmax(s):
    e = np.exp(s - s.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


def _strict_causal_softmax(s):
    """Off by one: keys j < i (row 0 keeps key 0)."""
    S = s.shape[-1]
    allowed = np.arange(S)[None, :] < np.arange(S)[:, None]
    allowed[0, 0] = True
    e = np.where(allowed, np.exp(np.where(allowed, s, 0.0) - np.where(allowed, s, -np.inf).max(-1, keepdims=True)), 0.0)
    return e / e.sum(-1, keepdims=True)


@pytest.mark.parametrize("slip", ["no_causal_mask", "strict_causal_mask", "no_memory_mask", "no_layernorm"])
def test_planted_mistakes(monkeypatch, slip):
    """Each slip planted in the oracle makes the library comparison fail."""
    c = _case(mem_lens=(3, 6))
    w = c.layer(0)
    if slip == "no_causal_mask":
        monkeypatch.setattr(dec, "causal_softmax", _unmasked_softmax)
    elif slip == "strict_causal_mask":
        monkeypatch.setattr(dec, "causal_softmax", _strict_causal_softmax)
    elif slip == "no_memory_mask":
        monkeypatch.setattr(dec, "masked_softmax", lambda s, lens: _unmasked_softmax(s))
    elif slip == "no_layernorm":
        monkeypatch.setattr(dec, "layer_norm", lambda z, g, b: z)
    got = dec.decoder_layer(c.x, c.mem, w, c.mem_lens, c.shape.head_num)
    ref = _torch_decoder_layer(c.x, c.mem, w, c.mem_lens, c.shape.head_num)
    assert not np.allclose(got, ref, atol=1e-6)
