"""Pins of the fp64 oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a dropped bias, a
wrong scale, a transposed operand, a missing mask, the erf GELU, an unbiased
variance, a pre-LN ordering) fails at least one of them; ``test_planted_mistakes``
plants each such slip in the oracle and checks that the pins notice.

Sources pinned against:
* worked examples derived by hand (``tests/golden/*.json``, each with its citation);
* closed forms the definition fixes (one-hot and uniform attention, zero weights);
* independent library routines: torch CPU float64 functional ops and
  ``torch.nn.TransformerEncoderLayer`` (post-LN, tanh GELU, eps 1e-6);
* brute-force scalar loops on tiny shapes;
* invariants: softmax rows sum to 1, masked keys are exactly 0, padded inputs
  do not reach valid outputs, LayerNorm moments, permutation symmetries.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synthetic_inputs import Shape, custom_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tiny_case(B=2, S=4, n=2, d=4, L=2, seed=7, lens=(3, 4), params="random_affine", std=0.5):
    shape = Shape(B, S, n, d, L, "fp32")
    c = custom_case(shape, seed, lens=None if lens is None else np.array(lens), params=params,
                    weight_std=std)
    return c


# ---------------------------------------------------------------- worked examples

def test_softmax_worked_example():
    g = _golden("softmax_worked.json")
    s = np.array(g["scores"], dtype=np.float64).reshape(1, 1, 1, -1)
    p = oracle.masked_softmax(s, np.array([g["len"]]))
    np.testing.assert_allclose(p.ravel(), g["probs"], rtol=0, atol=1e-15)
    assert p.ravel()[-1] == 0.0


def test_layernorm_worked_example():
    g = _golden("layernorm_worked.json")
    out = oracle.layer_norm(np.array(g["z"]), np.array(g["gamma"]), np.array(g["beta"]))
    np.testing.assert_allclose(out, g["out"], rtol=0, atol=1e-14)


def test_scores_worked_example():
    g = _golden("scores_worked.json")
    q = np.array(g["q"]).reshape(1, 1, 1, 4)
    k = np.array(g["k"]).reshape(1, 1, 3, 4)
    s = oracle.scaled_scores(q, k)
    np.testing.assert_allclose(s.ravel(), g["scores"], rtol=0, atol=1e-15)


# ---------------------------------------------------------------- softmax / masking

def test_softmax_rows_sum_to_one_and_masked_zero():
    rng = np.random.default_rng(0)
    s = rng.normal(size=(3, 2, 5, 5)) * 4
    lens = np.array([1, 3, 5])
    p = oracle.masked_softmax(s, lens)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14)
    for b, L in enumerate(lens):
        assert np.all(p[b, :, :, L:] == 0.0)
        assert np.all(p[b, :, :, :L] > 0.0)


def test_softmax_shift_invariance_and_large_scores():
    rng = np.random.default_rng(1)
    s = rng.normal(size=(1, 1, 3, 6))
    p0 = oracle.masked_softmax(s, None)
    p1 = oracle.masked_softmax(s + 700.0, None)   # naive exp would overflow
    np.testing.assert_allclose(p0, p1, atol=1e-14)
    np.testing.assert_allclose(p0, torch.softmax(torch.from_numpy(s), -1).numpy(), atol=1e-15)


def test_len_one_gives_one_hot_context():
    """len_b = 1: every query attends to key 0 only, so the context is V's first row."""
    c = _tiny_case(lens=(1, 1), L=1)
    w = c.layer(0)
    st = oracle.layer_steps(c.x, w, c.lens, c.shape.head_num)
    assert np.all(st["p"][..., 0] == 1.0)
    v0 = st["v"][:, :, 0:1, :]
    np.testing.assert_allclose(st["ctx"], oracle.merge_heads(np.broadcast_to(v0, st["v"].shape)),
                               atol=1e-15)


def test_zero_query_gives_uniform_attention():
    """Wq = 0, bq = 0: all scores 0, P uniform over valid keys, context = mean of valid V rows."""
    c = _tiny_case(lens=(3, 4), L=1)
    w = dict(c.layer(0))
    w["w_q"] = np.zeros_like(w["w_q"])
    w["b_q"] = np.zeros_like(w["b_q"])
    st = oracle.layer_steps(c.x, w, c.lens, c.shape.head_num)
    for b, L in enumerate(c.lens):
        v_tok = c.x[b] @ w["w_v"] + w["b_v"]          # [S, H] token-major V
        mean = v_tok[:L].mean(axis=0)
        np.testing.assert_allclose(st["ctx"][b], np.broadcast_to(mean, (c.shape.seq_len, c.shape.hidden)),
                                   atol=1e-14)


def test_padded_inputs_do_not_reach_valid_rows():
    c = _tiny_case(B=3, S=6, lens=(2, 6, 4), L=2)
    layers = list(c.layers())
    y0 = oracle.encoder(c.x, layers, c.lens, c.shape.head_num)
    x1 = c.x.copy()
    rng = np.random.default_rng(3)
    for b, L in enumerate(c.lens):
        x1[b, L:] = rng.normal(size=x1[b, L:].shape) * 10
    y1 = oracle.encoder(x1, layers, c.lens, c.shape.head_num)
    for b, L in enumerate(c.lens):
        np.testing.assert_allclose(y1[b, :L], y0[b, :L], atol=1e-13)


# ---------------------------------------------------------------- LayerNorm / GELU

def test_layernorm_moments_and_affine():
    rng = np.random.default_rng(4)
    z = rng.normal(size=(5, 64)) * 3 + 1
    ones, zeros = np.ones(64), np.zeros(64)
    y = oracle.layer_norm(z, ones, zeros)
    var = z.var(axis=-1, keepdims=True)
    np.testing.assert_allclose(y.mean(-1), 0.0, atol=1e-14)
    np.testing.assert_allclose(y.var(-1, keepdims=True), var / (var + oracle.LN_EPS), rtol=1e-12)
    gamma, beta = rng.normal(size=64), rng.normal(size=64)
    np.testing.assert_allclose(oracle.layer_norm(z, gamma, beta), gamma * y + beta, atol=1e-13)
    # scale invariance LN(c z) = LN(z) up to the epsilon term
    np.testing.assert_allclose(oracle.layer_norm(7.0 * z, ones, zeros), y, atol=1e-6)
    ref = F.layer_norm(torch.from_numpy(z), (64,), torch.from_numpy(gamma), torch.from_numpy(beta), eps=1e-6)
    np.testing.assert_allclose(oracle.layer_norm(z, gamma, beta), ref.numpy(), atol=1e-13)


def test_gelu_against_library_and_identities():
    x = np.linspace(-12, 12, 2001)
    g = oracle.gelu_tanh(x)
    ref = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(g, ref, atol=1e-15, rtol=1e-14)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(g - oracle.gelu_tanh(-x), x, atol=1e-14)   # gelu(x) - gelu(-x) = x
    big = np.array([30.0, -30.0])
    np.testing.assert_allclose(oracle.gelu_tanh(big), [30.0, 0.0], atol=1e-12)


def test_gelu_is_the_tanh_form_not_erf():
    x = np.array([2.70])
    erf_form = 0.5 * x * (1 + np.vectorize(math.erf)(x / math.sqrt(2)))
    diff = abs(oracle.gelu_tanh(x) - erf_form)[0]
    assert 1e-4 < diff < 6e-4


# ---------------------------------------------------------------- closed forms

def test_zero_weights_reduce_to_layernorm_of_residual():
    c = _tiny_case(lens=(2, 4), L=1, params="bert")
    w = {k: (np.zeros_like(v) if k.startswith(("w_", "b_")) else v) for k, v in c.layer(0).items()}
    out = oracle.encoder_layer(c.x, w, c.lens, c.shape.head_num)
    H = c.shape.hidden
    ln = lambda t: F.layer_norm(t, (H,), eps=1e-6)
    ref = ln(ln(torch.from_numpy(c.x))).numpy()
    np.testing.assert_allclose(out, ref, atol=1e-13)
    # only the two output biases nonzero: Y1 = LN(X + bo), X' = LN(Y1 + b2)
    rng = np.random.default_rng(5)
    w["b_o"] = rng.normal(size=H)
    w["b_ffn2"] = rng.normal(size=H)
    out = oracle.encoder_layer(c.x, w, c.lens, c.shape.head_num)
    y1 = ln(torch.from_numpy(c.x + w["b_o"]))
    ref = ln(y1 + torch.from_numpy(w["b_ffn2"])).numpy()
    np.testing.assert_allclose(out, ref, atol=1e-13)


# ---------------------------------------------------------------- library special case

def _torch_layer_functional(x, w, lens, n):
    """Independent composition of torch CPU float64 routines."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    X = t(x)
    B, S, H = X.shape
    d = H // n
    q = F.linear(X, t(w["w_q"].T), t(w["b_q"])).view(B, S, n, d).transpose(1, 2)
    k = F.linear(X, t(w["w_k"].T), t(w["b_k"])).view(B, S, n, d).transpose(1, 2)
    v = F.linear(X, t(w["w_v"].T), t(w["b_v"])).view(B, S, n, d).transpose(1, 2)
    mask = None
    if lens is not None:
        mask = (torch.arange(S)[None, :] < t(lens.astype(np.int64))[:, None])[:, None, None, :]
    ctx = F.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    ctx = ctx.transpose(1, 2).reshape(B, S, H)
    y1 = F.layer_norm(X + F.linear(ctx, t(w["w_o"].T), t(w["b_o"])), (H,), t(w["ln1_gamma"]),
                      t(w["ln1_beta"]), eps=1e-6)
    u = F.gelu(F.linear(y1, t(w["w_ffn1"].T), t(w["b_ffn1"])), approximate="tanh")
    z = F.linear(u, t(w["w_ffn2"].T), t(w["b_ffn2"]))
    return F.layer_norm(y1 + z, (H,), t(w["ln2_gamma"]), t(w["ln2_beta"]), eps=1e-6).numpy()


def _torch_module_layer(x, w, lens, n):
    """torch.nn.TransformerEncoderLayer (post-LN), loaded with the same weights."""
    H = x.shape[-1]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    layer = torch.nn.TransformerEncoderLayer(
        d_model=H, nhead=n, dim_feedforward=4 * H, dropout=0.0,
        activation=lambda u: F.gelu(u, approximate="tanh"), layer_norm_eps=1e-6,
        batch_first=True, norm_first=False, dtype=torch.float64)
    layer.eval()
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(t(np.concatenate([w["w_q"].T, w["w_k"].T, w["w_v"].T], 0)))
        layer.self_attn.in_proj_bias.copy_(t(np.concatenate([w["b_q"], w["b_k"], w["b_v"]])))
        layer.self_attn.out_proj.weight.copy_(t(w["w_o"].T))
        layer.self_attn.out_proj.bias.copy_(t(w["b_o"]))
        layer.linear1.weight.copy_(t(w["w_ffn1"].T))
        layer.linear1.bias.copy_(t(w["b_ffn1"]))
        layer.linear2.weight.copy_(t(w["w_ffn2"].T))
        layer.linear2.bias.copy_(t(w["b_ffn2"]))
        layer.norm1.weight.copy_(t(w["ln1_gamma"]))
        layer.norm1.bias.copy_(t(w["ln1_beta"]))
        layer.norm2.weight.copy_(t(w["ln2_gamma"]))
        layer.norm2.bias.copy_(t(w["ln2_beta"]))
        pad = None
        if lens is not None:
            pad = torch.arange(x.shape[1])[None, :] >= t(lens.astype(np.int64))[:, None]
        return layer(t(x), src_key_padding_mask=pad).numpy()


@pytest.mark.parametrize("lens", [None, (3, 5, 1)])
def test_oracle_matches_torch_functional(lens):
    c = _tiny_case(B=3, S=5, n=3, d=4, L=1, lens=lens, std=0.3)
    w = c.layer(0)
    out = oracle.encoder_layer(c.x, w, c.lens, c.shape.head_num)
    ref = _torch_layer_functional(c.x, w, c.lens, c.shape.head_num)
    np.testing.assert_allclose(out, ref, atol=1e-12)


@pytest.mark.parametrize("lens", [None, (2, 6)])
def test_oracle_matches_torch_transformer_encoder_layer(lens):
    c = _tiny_case(B=2, S=6, n=2, d=8, L=2, lens=lens, std=0.3)
    ref = c.x
    for w in c.layers():
        ref = _torch_module_layer(ref, w, c.lens, c.shape.head_num)
    out = oracle.encoder(c.x, list(c.layers()), c.lens, c.shape.head_num)
    np.testing.assert_allclose(out, ref, atol=1e-12)


# ---------------------------------------------------------------- brute force

def _brute_layer(x, w, lens, n):
    """Scalar loops, written from the layer definition, for tiny shapes."""
    B, S, H = x.shape
    d = H // n
    F4 = w["w_ffn1"].shape[1]
    out = np.zeros_like(x)

    def lin(row, W, bvec):
        return [sum(row[i] * W[i][j] for i in range(len(row))) + bvec[j] for j in range(len(bvec))]

    def ln(row, g, b):
        mu = sum(row) / len(row)
        var = sum((r - mu) ** 2 for r in row) / len(row)
        return [g[i] * (row[i] - mu) / math.sqrt(var + 1e-6) + b[i] for i in range(len(row))]

    for b in range(B):
        L = S if lens is None else int(lens[b])
        Q = [lin(x[b, s], w["w_q"], w["b_q"]) for s in range(S)]
        K = [lin(x[b, s], w["w_k"], w["b_k"]) for s in range(S)]
        V = [lin(x[b, s], w["w_v"], w["b_v"]) for s in range(S)]
        ctx = [[0.0] * H for _ in range(S)]
        for h in range(n):
            for i in range(S):
                sc = [sum(Q[i][h * d + e] * K[j][h * d + e] for e in range(d)) / math.sqrt(d) for j in range(L)]
                m = max(sc)
                ex = [math.exp(v - m) for v in sc]
                tot = sum(ex)
                for e in range(d):
                    ctx[i][h * d + e] = sum(ex[j] / tot * V[j][h * d + e] for j in range(L))
        for s in range(S):
            a = lin(ctx[s], w["w_o"], w["b_o"])
            y1 = ln([x[b, s, i] + a[i] for i in range(H)], w["ln1_gamma"], w["ln1_beta"])
            u = lin(y1, w["w_ffn1"], w["b_ffn1"])
            g = [0.5 * v * (1 + math.tanh(math.sqrt(2 / math.pi) * (v + 0.044715 * v * v * v))) for v in u]
            assert len(g) == F4
            z = lin(g, w["w_ffn2"], w["b_ffn2"])
            out[b, s] = ln([y1[i] + z[i] for i in range(H)], w["ln2_gamma"], w["ln2_beta"])
    return out


def test_oracle_matches_brute_force_tiny():
    c = _tiny_case(B=2, S=4, n=2, d=4, L=2, lens=(3, 4))
    ref = c.x
    for w in c.layers():
        ref = _brute_layer(ref, w, c.lens, c.shape.head_num)
    out = oracle.encoder(c.x, list(c.layers()), c.lens, c.shape.head_num)
    np.testing.assert_allclose(out, ref, atol=1e-12)


# ---------------------------------------------------------------- symmetries

def test_permutation_equivariance_of_valid_tokens():
    c = _tiny_case(B=1, S=6, n=2, d=4, L=2, lens=(5,))
    layers = list(c.layers())
    y = oracle.encoder(c.x, layers, c.lens, 2)
    perm = np.array([3, 0, 4, 1, 2, 5])         # permutes the 5 valid tokens, keeps the pad
    yp = oracle.encoder(c.x[:, perm], layers, c.lens, 2)
    np.testing.assert_allclose(yp, y[:, perm], atol=1e-12)


def test_head_permutation_invariance():
    c = _tiny_case(B=2, S=4, n=3, d=4, L=1, lens=(4, 2))
    w = c.layer(0)
    perm = [2, 0, 1]
    cols = np.concatenate([np.arange(h * 4, h * 4 + 4) for h in perm])
    wp = dict(w)
    for nm in ("w_q", "w_k", "w_v"):
        wp[nm] = w[nm][:, cols]
    for nm in ("b_q", "b_k", "b_v"):
        wp[nm] = w[nm][cols]
    wp["w_o"] = w["w_o"][cols, :]
    y = oracle.encoder_layer(c.x, w, c.lens, 3)
    yp = oracle.encoder_layer(c.x, wp, c.lens, 3)
    np.testing.assert_allclose(yp, y, atol=1e-12)


def test_batch_independence_and_rows():
    c = _tiny_case(B=4, S=4, n=2, d=4, L=2, lens=(1, 4, 2, 3))
    layers = list(c.layers())
    y = oracle.encoder(c.x, layers, c.lens, 2)
    rows = [2, 0]
    yr = oracle.encoder_rows(c.x, layers, c.lens, 2, rows)
    np.testing.assert_allclose(yr, y[rows], atol=1e-13)


def test_oracle_rejects_zero_length():
    with pytest.raises(ValueError):
        oracle.masked_softmax(np.zeros((1, 1, 2, 2)), np.array([0]))


# ---------------------------------------------------------------- planted mistakes

def _pins_fail(monkeypatch, patch):
    """Apply ``patch`` to the oracle module and report whether the independent
    pins (torch functional, torch module, brute force) catch it."""
    import oracle.fp64_encoder as enc
    patch(monkeypatch, enc)
    caught = 0
    for fn in (test_oracle_matches_brute_force_tiny,
               lambda: test_oracle_matches_torch_functional((3, 5, 1)),
               lambda: test_oracle_matches_torch_transformer_encoder_layer((2, 6))):
        try:
            fn()
        except AssertionError:
            caught += 1
    return caught


_PLANTS = {
    "erf_gelu": lambda mp, e: mp.setattr(e, "gelu_tanh", lambda u: 0.5 * u * (1 + np.vectorize(math.erf)(u / math.sqrt(2)))),
    "no_scale": lambda mp, e: mp.setattr(e, "scaled_scores", lambda q, k: q @ np.swapaxes(k, -1, -2)),
    "scale_by_d": lambda mp, e: mp.setattr(e, "scaled_scores", lambda q, k: q @ np.swapaxes(k, -1, -2) / q.shape[-1]),
    "no_mask": lambda mp, e: mp.setattr(e, "key_valid", lambda lens, S: None),
    "unbiased_var": lambda mp, e: mp.setattr(
        e, "layer_norm", lambda z, g, b, eps=1e-6: g * (z - z.mean(-1, keepdims=True)) / np.sqrt(z.var(-1, ddof=1, keepdims=True) + eps) + b),
    "dropped_bias": lambda mp, e: mp.setattr(e, "linear", lambda x, w, b: x @ w),
    "transposed_scores": lambda mp, e: mp.setattr(
        e, "scaled_scores", lambda q, k: np.swapaxes(q @ np.swapaxes(k, -1, -2), -1, -2) / np.sqrt(q.shape[-1])),
    "heads_interleaved": lambda mp, e: mp.setattr(
        e, "split_heads", lambda y, n: y.reshape(y.shape[0], y.shape[1], y.shape[2] // n, n).transpose(0, 3, 1, 2)),
}


def _pre_ln_steps(x, w, lens, n):
    import oracle.fp64_encoder as e
    a = e.layer_norm(x, w["ln1_gamma"], w["ln1_beta"])
    q = e.split_heads(e.linear(a, w["w_q"], w["b_q"]), n)
    k = e.split_heads(e.linear(a, w["w_k"], w["b_k"]), n)
    v = e.split_heads(e.linear(a, w["w_v"], w["b_v"]), n)
    ctx = e.merge_heads(e.context(e.masked_softmax(e.scaled_scores(q, k), lens), v))
    y1 = x + e.linear(ctx, w["w_o"], w["b_o"])
    b = e.layer_norm(y1, w["ln2_gamma"], w["ln2_beta"])
    out = y1 + e.linear(e.gelu_tanh(e.linear(b, w["w_ffn1"], w["b_ffn1"])), w["w_ffn2"], w["b_ffn2"])
    return dict(out=out)


_PLANTS["pre_ln"] = lambda mp, e: mp.setattr(e, "layer_steps", _pre_ln_steps)


@pytest.mark.parametrize("plant", sorted(_PLANTS))
def test_planted_mistakes(monkeypatch, plant):
    assert _pins_fail(monkeypatch, _PLANTS[plant]) >= 1, f"planted mistake {plant} not caught"
