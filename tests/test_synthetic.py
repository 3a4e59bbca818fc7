"""Seeded input generator: determinism, prefix slicing, rounding (CPU only)."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si


def test_round_to_matches_hardware_conversions():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=20000), rng.normal(size=2000) * 1e-6,
                        rng.normal(size=2000) * 1e4])
    np.testing.assert_array_equal(si.round_to(x, "fp32"), x.astype(np.float32).astype(np.float64))
    # fp16 from the float64 value: numpy's float64->float16 is a direct RNE conversion
    np.testing.assert_array_equal(si.round_to(x, "fp16"), x.astype(np.float16).astype(np.float64))
    # bf16: torch's float32 -> bf16 is RNE; go through float32 only where that is exact
    x32 = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x32).float().to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(si.round_to(x32, "bf16"), ref)


def test_round_to_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1
    assert si.round_to(np.array([1 + 2.0 ** -8]), "bf16")[0] == 1.0
    assert si.round_to(np.array([1 + 3 * 2.0 ** -8]), "bf16")[0] == 1 + 2.0 ** -6
    assert si.round_to(np.array([1 + 2.0 ** -11]), "fp16")[0] == 1.0
    # fp16 subnormal quantum 2^-24
    assert si.round_to(np.array([3 * 2.0 ** -26]), "fp16")[0] == 2.0 ** -24
    with pytest.raises(OverflowError):
        si.round_to(np.array([70000.0]), "fp16")


def test_host_array_bf16_bits_roundtrip():
    x = si.round_to(np.random.default_rng(1).normal(size=1000), "bf16")
    bits = si.host_array(x, "bf16")
    np.testing.assert_array_equal(si.from_bf16_bits(bits), x)


def test_cases_are_deterministic_and_prefix_sliced():
    a = si.make_case("bert_base_fp16_s64_varlen", 1)
    b = si.make_case("bert_base_fp16_s64_varlen", 64)
    np.testing.assert_array_equal(a.x, b.x[:1])
    np.testing.assert_array_equal(a.lens, b.lens[:1])
    np.testing.assert_array_equal(a.layer(3)["w_ffn1"], b.layer(3)["w_ffn1"])
    c = si.make_case("bert_base_fp16_s64_varlen", 64)
    np.testing.assert_array_equal(b.x, c.x)
    assert b.lens.min() >= 16 and b.lens.max() <= 64
    # layer l of a truncated stack is layer l of the full stack
    d = si.make_case("bert_base_fp16_s64_varlen", 1, num_layers=2)
    np.testing.assert_array_equal(d.layer(1)["w_q"], a.layer(1)["w_q"])


def test_workload_distributions():
    c = si.make_case("single_layer_fp32")
    assert c.shape == si.Shape(1, 32, 4, 32, 1, "fp32")
    assert 16 <= int(c.lens[0]) <= 32
    w = c.layer(0)
    assert w["w_q"].shape == (128, 128) and w["w_ffn1"].shape == (128, 512)
    assert np.all(w["b_q"] == 0) and np.all(w["ln1_gamma"] == 1) and np.all(w["ln2_beta"] == 0)
    assert abs(w["w_ffn1"].std() - 0.02) < 0.002
    assert abs(c.x.std() - 1.0) < 0.05
    s5 = si.make_case("bert_large_bf16_s512", num_layers=1)
    assert s5.lens.min() >= 64 and s5.lens.max() <= 512
    assert np.array_equal(si.round_to(s5.x, "bf16"), s5.x)


def test_flop_count():
    s = si.WORKLOADS["bert_base_fp16_s32"].shape(512)
    assert abs(s.flops() - 2.8025e12) / 2.8025e12 < 1e-3


def test_layer_draw_is_stateless():
    c = si.make_case("pruned_fp16_s32", 1)
    a = c.layer(2)["w_o"]
    _ = c.layer(2)
    np.testing.assert_array_equal(c.layer(2)["w_o"], a)
    ss = np.random.SeedSequence(5)
    assert si._child(ss, 1).generate_state(4).tolist() == ss.spawn(2)[1].generate_state(4).tolist()
