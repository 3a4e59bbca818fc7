"""Plain float64 numpy oracle of a Transformer decoder forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and the benchmark's CPU-baseline leg),
never by the library.  It shares no code with the HIP path.  Matrix products are numpy's;
nothing is fused, blocked or reordered beyond the definitions below.

Source: the FT article ("有钱任性：英伟达训练80亿参数量GPT-2，1475块V100 53分钟训练BERT",
cloud.tencent.com/developer/article/1490359), section "什么是 Faster Transformer", which
names decoder support as a later item of the roadmap and says nothing about its
structure.  Readings taken -- each the plainest one that agrees with the encoder layer of
the same section (``fp64_encoder``), and each pinned by ``tests/test_oracle_decoder.py``:

* a decoder layer is the encoder layer with a causal mask on its self-attention and a
  cross-attention sub-layer over the encoder output (the "memory") between the
  self-attention and the feed-forward block; every sub-layer is followed by residual +
  LayerNorm (post-LN, as the encoder):
      Y1  = LN1(X  + SelfAttn_causal(X) Wo + bo)
      Y2  = LN2(Y1 + CrossAttn(Y1, M) Wo2 + bo2)
      out = LN3(Y2 + gelu(Y2 W1 + b1) W2 + b2);
* causal: query i attends to decoder keys j <= i.  There is no key-padding mask on the
  self-attention: a row below a sequence's valid length only sees keys at or before it,
  which are all valid, and every row, padded or not, is computed the same way;
* cross-attention: queries from Y1 (Wq2, bq2), keys and values from the memory (Wk2, bk2,
  Wv2, bv2); memory keys j >= the sequence's memory length get probability 0;
* everything else as the encoder: scores scaled by 1/sqrt(d), LayerNorm with the biased
  variance and epsilon 1e-6, tanh-form GELU, feed-forward width 4H, weights [in][out].
"""
from __future__ import annotations

from typing import Dict, Iterable

import numpy as np

from .fp64_encoder import (_f64, context, gelu_tanh, layer_norm, linear, masked_softmax,
                           merge_heads, scaled_scores, split_heads)

# weight names of one decoder layer, [in][out] matrices and [out] vectors
DECODER_WEIGHT_NAMES = (
    "w_q", "b_q", "w_k", "b_k", "w_v", "b_v", "w_o", "b_o", "ln1_gamma", "ln1_beta",
    "w_q2", "b_q2", "w_k2", "b_k2", "w_v2", "b_v2", "w_o2", "b_o2", "ln2_gamma", "ln2_beta",
    "w_ffn1", "b_ffn1", "w_ffn2", "b_ffn2", "ln3_gamma", "ln3_beta")


def causal_softmax(s) -> np.ndarray:
    """Softmax over the last axis restricted to keys j <= i (query i, key j) of a square
    score block [..., S, S]: p_ij = exp(s_ij - m_i) / sum_{j' <= i} exp(s_ij' - m_i) for
    j <= i and 0 for j > i, with m_i the maximum over j <= i."""
    s = _f64(s)
    S = s.shape[-1]
    if s.shape[-2] != S:
        raise ValueError("causal scores must be square")
    allowed = np.arange(S)[None, :] <= np.arange(S)[:, None]   # [i, j]: j <= i
    m = np.where(allowed, s, -np.inf).max(axis=-1, keepdims=True)
    e = np.where(allowed, np.exp(np.where(allowed, s, 0.0) - m), 0.0)
    return e / e.sum(axis=-1, keepdims=True)


def decoder_layer_steps(x, mem, w: Dict[str, np.ndarray], mem_lens,
                        head_num: int) -> Dict[str, np.ndarray]:
    """One decoder layer (readings above), returning every intermediate.

    x [B, Sd, H] decoder states, mem [B, Se, H] memory, mem_lens [B] (or None: all valid).
    Keys: q, k, v, p (self-attention, p [B,n,Sd,Sd]), ctx, attn, y1; q2, k2, v2, p2
    (cross-attention, p2 [B,n,Sd,Se]), ctx2, cross, y2; u, g, z, out.
    """
    x = _f64(x)
    mem = _f64(mem)
    # causal self-attention + add & LayerNorm
    q = split_heads(linear(x, w["w_q"], w["b_q"]), head_num)
    k = split_heads(linear(x, w["w_k"], w["b_k"]), head_num)
    v = split_heads(linear(x, w["w_v"], w["b_v"]), head_num)
    p = causal_softmax(scaled_scores(q, k))
    ctx = merge_heads(context(p, v))
    attn = linear(ctx, w["w_o"], w["b_o"])
    y1 = layer_norm(x + attn, w["ln1_gamma"], w["ln1_beta"])
    # cross-attention over the memory + add & LayerNorm
    q2 = split_heads(linear(y1, w["w_q2"], w["b_q2"]), head_num)
    k2 = split_heads(linear(mem, w["w_k2"], w["b_k2"]), head_num)
    v2 = split_heads(linear(mem, w["w_v2"], w["b_v2"]), head_num)
    p2 = masked_softmax(scaled_scores(q2, k2), mem_lens)
    ctx2 = merge_heads(context(p2, v2))
    cross = linear(ctx2, w["w_o2"], w["b_o2"])
    y2 = layer_norm(y1 + cross, w["ln2_gamma"], w["ln2_beta"])
    # feed-forward + add & LayerNorm
    u = linear(y2, w["w_ffn1"], w["b_ffn1"])
    g = gelu_tanh(u)
    z = linear(g, w["w_ffn2"], w["b_ffn2"])
    out = layer_norm(y2 + z, w["ln3_gamma"], w["ln3_beta"])
    return dict(q=q, k=k, v=v, p=p, ctx=ctx, attn=attn, y1=y1, q2=q2, k2=k2, v2=v2, p2=p2,
                ctx2=ctx2, cross=cross, y2=y2, u=u, g=g, z=z, out=out)


def decoder_layer(x, mem, w: Dict[str, np.ndarray], mem_lens, head_num: int) -> np.ndarray:
    """One decoder layer's output [B, Sd, H]."""
    return decoder_layer_steps(x, mem, w, mem_lens, head_num)["out"]


def decoder(x, mem, layers: Iterable[Dict[str, np.ndarray]], mem_lens,
            head_num: int) -> np.ndarray:
    """The L-layer stack: every layer attends to the same memory."""
    h = _f64(x)
    for w in layers:
        h = decoder_layer(h, mem, w, mem_lens, head_num)
    return h
