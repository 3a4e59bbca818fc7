"""Plain float64 numpy oracle of the BERT-style Transformer encoder forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
HIP path.  Matrix products are numpy's; nothing is fused, blocked or reordered
beyond the definitions below, so each function can be checked against the text
by eye.

Source ("FT article" below): "有钱任性：英伟达训练80亿参数量GPT-2，1475块V100 53分钟训练BERT",
cloud.tencent.com/developer/article/1490359, sections "什么是 Faster Transformer"
(the encoder forward of BERT-BASE-like multi-layer Transformers, parameterised by
head count, size per head, batch size and sentence length) and "Faster Transformer
优化原理" (the per-layer computation as matrix multiplies plus GELU, LayerNorm and
SoftMax; the flow-chart figure of the layer did not survive).

Readings taken where the article is silent (each pinned by the tests in
``tests/test_oracle.py`` against something other than this file):

* layer order: the standard post-LayerNorm BERT encoder layer
  (self-attention -> add & LayerNorm -> feed-forward -> add & LayerNorm);
* attention scores scaled by 1/sqrt(size_per_head);
* padding: keys at positions >= the sequence's valid length get probability 0;
  every query row, padded or not, is computed the same way;
* LayerNorm: biased variance, epsilon 1e-6;
* GELU: the tanh form (the article's TensorFlow timeline shows it built from
  Pow/Add/Tanh ops, and its optimisation list replaces pow(x, 3.0) by x*x*x);
* feed-forward width 4 * hidden;
* weights stored [in][out], y = x W + b; head h owns hidden columns
  h*d .. h*d+d-1 of Q, K and V.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

LN_EPS = 1e-6
_SQRT_2_OVER_PI = np.sqrt(2.0 / np.pi)


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float64:
        raise TypeError("oracle works in float64 only")
    return a


def linear(x, w, b) -> np.ndarray:
    """y = x W + b, W stored [in][out] (one of the FT article's matrix multiplies,
    section "Faster Transformer 优化原理")."""
    return _f64(x) @ _f64(w) + _f64(b)


def split_heads(y, head_num: int) -> np.ndarray:
    """[B, S, H] -> [B, n, S, d]; head h takes columns h*d .. h*d+d-1."""
    B, S, H = y.shape
    d = H // head_num
    if d * head_num != H:
        raise ValueError("hidden not divisible by head_num")
    return y.reshape(B, S, head_num, d).transpose(0, 2, 1, 3)


def merge_heads(c) -> np.ndarray:
    """[B, n, S, d] -> [B, S, n*d], inverse of split_heads."""
    B, n, S, d = c.shape
    return c.transpose(0, 2, 1, 3).reshape(B, S, n * d)


def scaled_scores(q, k) -> np.ndarray:
    """s[b,h,i,j] = <q[b,h,i], k[b,h,j]> / sqrt(d)  ->  [B, n, S, S]."""
    d = q.shape[-1]
    return (_f64(q) @ np.swapaxes(_f64(k), -1, -2)) / np.sqrt(d)


def key_valid(lens, seq_len: int) -> np.ndarray:
    """[B, S] boolean, True where key j < lens[b].  ``lens`` None means no padding."""
    if lens is None:
        return None
    lens = np.asarray(lens)
    if np.any(lens < 1) or np.any(lens > seq_len):
        raise ValueError("valid lengths must lie in [1, seq_len]")
    return np.arange(seq_len)[None, :] < lens[:, None]


def masked_softmax(s, lens) -> np.ndarray:
    """Softmax over the last axis restricted to valid keys (the FT article's SoftMax,
    section "Faster Transformer 优化原理").

    p[b,h,i,j] = exp(s_ij - m_i) / sum_{j' < len_b} exp(s_ij' - m_i) for j < len_b,
    and 0 for j >= len_b, with m_i the maximum over valid keys.
    """
    s = _f64(s)
    valid = key_valid(lens, s.shape[-1])
    if valid is None:
        valid = np.ones((s.shape[0], s.shape[-1]), dtype=bool)
    v = valid[:, None, None, :]
    m = np.where(v, s, -np.inf).max(axis=-1, keepdims=True)
    e = np.where(v, np.exp(np.where(v, s, 0.0) - m), 0.0)
    return e / e.sum(axis=-1, keepdims=True)


def context(p, v) -> np.ndarray:
    """c[b,h,i,:] = sum_j p[b,h,i,j] v[b,h,j,:]."""
    return _f64(p) @ _f64(v)


def layer_norm(z, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis (the FT article's Layer Normalization, section
    "Faster Transformer 优化原理"): gamma * (z - mean) / sqrt(var + eps) + beta, with
    the biased variance."""
    z = _f64(z)
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    return _f64(gamma) * (z - mu) / np.sqrt(var + eps) + _f64(beta)


def gelu_tanh(u) -> np.ndarray:
    """GELU, tanh form: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))) (the FT
    article's GELU built from Pow/Add/Tanh, section "Faster Transformer 优化原理",
    figure 1)."""
    u = _f64(u)
    return 0.5 * u * (1.0 + np.tanh(_SQRT_2_OVER_PI * (u + 0.044715 * u * u * u)))


def layer_steps(x, w: Dict[str, np.ndarray], lens, head_num: int) -> Dict[str, np.ndarray]:
    """One post-LN encoder layer, returning every intermediate.

    Keys: q, k, v ([B,n,S,d], biases added), p ([B,n,S,S]), ctx ([B,S,H], heads
    merged), attn (ctx Wo + bo), y1, u (Y1 W1 + b1), g (gelu(u)), z (G W2 + b2), out.
    """
    x = _f64(x)
    q = split_heads(linear(x, w["w_q"], w["b_q"]), head_num)
    k = split_heads(linear(x, w["w_k"], w["b_k"]), head_num)
    v = split_heads(linear(x, w["w_v"], w["b_v"]), head_num)
    p = masked_softmax(scaled_scores(q, k), lens)
    ctx = merge_heads(context(p, v))
    attn = linear(ctx, w["w_o"], w["b_o"])
    y1 = layer_norm(x + attn, w["ln1_gamma"], w["ln1_beta"])
    u = linear(y1, w["w_ffn1"], w["b_ffn1"])
    g = gelu_tanh(u)
    z = linear(g, w["w_ffn2"], w["b_ffn2"])
    out = layer_norm(y1 + z, w["ln2_gamma"], w["ln2_beta"])
    return dict(q=q, k=k, v=v, p=p, ctx=ctx, attn=attn, y1=y1, u=u, g=g, z=z, out=out)


def encoder_layer(x, w: Dict[str, np.ndarray], lens, head_num: int) -> np.ndarray:
    """One post-LN encoder layer: X' = LN(Y1 + gelu(Y1 W1 + b1) W2 + b2) with
    Y1 = LN(X + Attention(X) Wo + bo)."""
    return layer_steps(x, w, lens, head_num)["out"]


def encoder(x, layers, lens, head_num: int) -> np.ndarray:
    """The L-layer stack; ``layers`` is an iterable of per-layer weight dicts.
    Output at all B x S positions."""
    h = _f64(x)
    for w in layers:
        h = encoder_layer(h, w, lens, head_num)
    return h


def encoder_rows(x, layers, lens, head_num: int, rows) -> np.ndarray:
    """The stack on a subset of sequences (batch entries are independent:
    nothing in a layer mixes sequences).  Returns [len(rows), S, H]."""
    rows = np.asarray(rows)
    sub_lens: Optional[np.ndarray] = None if lens is None else np.asarray(lens)[rows]
    return encoder(np.asarray(x)[rows], layers, sub_lens, head_num)
