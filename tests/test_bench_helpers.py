"""Host logic of bench.py: the step class of each kernel dispatch of a forward, which the
rocprofv3 summaries and the bench's traffic lookup are keyed on."""
from __future__ import annotations

import bench

# kernel symbols of one BERT-base fp16 layer as the library launches them: the Q/K/V
# projection with the attention in its epilogue, the attention-output projection, LN1,
# FFN-in with GELU, FFN-out on the ping-pong K loop, LN2
QKV_ATTN = "_ZN3ftx11gemm_kernelIDF16_Li256ELi192ELi4ELi2ENS_10EpiQKVAttnIDF16_Li32ELi64EEEEEvPKT_S5_iiiiT4_"
LINEAR = "_ZN3ftx11gemm_kernelIDF16_Li256ELi192ELi4ELi2ENS_9EpiLinearIDF16_Lb0EDF16_EEEEvPKT_S5_iiiiT4_"
LINEAR_PP = "_ZN3ftx14gemm_pp_kernelIDF16_Li256ELi192ENS_9EpiLinearIDF16_Lb0EDF16_EEEEvPKT_S5_iiiiT2_"
GELU = "_ZN3ftx11gemm_kernelIDF16_Li256ELi256ELi4ELi2ENS_9EpiLinearIDF16_Lb1EDF16_EEEEvPKT_S5_iiiiT4_"
LN = "_ZN3ftx16layernorm_kernelIDF16_DF16_DF16_Li8ELi32ELi3ELb1EEEvPKT0_PKT1_PKT_S9_S9_PS7_Pfii"
QKV = "_ZN3ftx11gemm_kernelIDF16_Li256ELi192ELi4ELi2ENS_6EpiQKVIDF16_EEEEvPKT_S5_iiiiT4_"
ATTN = "_ZN3ftx16attention_kernelIDF16_Li32ELi64ELi1EEEvPKT_S3_S3_PKiPS1_iiiif"


def test_fused_layer_dispatches():
    layer = [QKV_ATTN, LINEAR, LN, GELU, LINEAR_PP, LN]
    assert bench.classify_dispatches(layer * 2) == [
        "qkv_attention", "attn_out_gemm", "ln1", "ffn1_gemm", "ffn2_gemm", "ln2"] * 2


def test_separate_attention_dispatches():
    layer = [QKV, ATTN, LINEAR, LN, GELU, LINEAR, LN]
    assert bench.classify_dispatches(layer) == [
        "qkv_gemm", "attention", "attn_out_gemm", "ln1", "ffn1_gemm", "ffn2_gemm", "ln2"]


# the same layer with the first LayerNorm folded into FFN-in
RES_STATS = "_ZN3ftx14gemm_pp_kernelIDF16_Li256ELi192ENS_17EpiLinearResStatsIDF16_EEEEvPKT_S5_iiiiiT2_"
NORM_IN = "_ZN3ftx14gemm_pp_kernelIDF16_Li256ELi256ENS_15EpiLinearNormInIDF16_Lb1EEEEEvPKT_S5_iiiiiT2_"
LN_XN = ("_ZN3ftx16layernorm_kernelIDF16_DF16_DF16_Li8ELi32ELi3ELb1ELb1EEEvPKT0_PKT1_PKT_S9_S9_PS7_"
         "PfiiNS_12ResidualNormIS7_EE")


def test_folded_layer_dispatches():
    layer = [QKV_ATTN, RES_STATS, NORM_IN, LINEAR_PP, LN_XN]
    assert bench.classify_dispatches(layer * 2) == [
        "qkv_attention", "attn_out_gemm", "ffn1_gemm", "ffn2_gemm", "ln2"] * 2
    # the FFN block in two row chunks
    chunked = [QKV_ATTN, RES_STATS, NORM_IN, LINEAR_PP, LN_XN, NORM_IN, LINEAR_PP, LN_XN]
    assert bench.classify_dispatches(chunked) == [
        "qkv_attention", "attn_out_gemm", "ffn1_gemm", "ffn2_gemm", "ln2", "ffn1_gemm",
        "ffn2_gemm", "ln2"]
    roles = [next((v for k, v in bench.KERNEL_ROLES if k in n), "") for n in (RES_STATS, NORM_IN, LN_XN, LN)]
    assert "statistics" in roles[0] and "FFN-in" in roles[1] and "rebuilt" in roles[2]
    assert roles[3] == "bias + residual + LayerNorm"


PREFETCH = "_ZN3ftx17prefetch16_kernelEPK15HIP_vector_typeIjLj4EEm"
LINEAR_128 = "_ZN3ftx11gemm_kernelIDF16_Li128ELi128ELi2ELi2ENS_9EpiLinearIDF16_Lb0EDF16_EELi2EEEvPKT_S5_iiiiiT4_"


def test_prefetch_before_ffn_out():
    """The W2 read ahead of the second FFN projection is its own step class, and the plain
    projection after it is still FFN-out; the read moves W2's bytes once."""
    layer = [QKV_ATTN, RES_STATS, NORM_IN, PREFETCH, LINEAR_128, LN_XN]
    assert bench.classify_dispatches(layer * 2) == [
        "qkv_attention", "attn_out_gemm", "ffn1_gemm", "weight_prefetch", "ffn2_gemm", "ln2"] * 2
    role = next((v for k, v in bench.KERNEL_ROLES if k in PREFETCH), "")
    assert "last-level cache" in role
    import synthetic_inputs as si
    sh = si.Shape(256, 32, 12, 64, 12, "fp16")
    assert bench.step_work(sh, "weight_prefetch") == (0.0, sh.hidden * sh.ffn * 2)
    assert bench.launches_per_layer({"qkv_attention": 12, "weight_prefetch": 12}, "weight_prefetch") == 1


def test_unknown_kernels_are_not_classified():
    assert bench.classify_dispatches(["copy_kernel", LN]) == [None, "ln2"]


def test_valid_token_flops():
    """Full lengths give the padded count; the count falls with the valid tokens (projections
    linearly, attention quadratically)."""
    import numpy as np
    import synthetic_inputs as si
    sh = si.Shape(4, 64, 12, 64, 12, "fp16")
    assert sh.valid_flops(np.full(4, 64)) == sh.flops()
    half = sh.valid_flops(np.full(4, 32))
    H, L = 768, 12
    assert half == L * (24.0 * 128 * H * H + 4.0 * 4 * 32 * 32 * H)


def test_profile_commands_run_the_program_directly():
    """Every rocprofv3 command puts python3 right after `--` (no shell or env hop) and keeps
    counter passes apart from the kernel trace."""
    cmds = bench.profile_commands("bert_base_fp16_s32", 512, "x", 64)
    prof = [c for c in cmds if c.startswith("rocprofv3")]
    assert len(prof) == 4
    for c in prof:
        assert " -- python3 bench.py" in c
        assert not ("--pmc" in c and "--kernel-trace" in c)
    assert any("SQ_VALU_MFMA_BUSY_CYCLES" in c for c in prof)
    assert all("--batch 64" in c for c in cmds)


def test_launches_per_layer_and_folded_work():
    """The FFN block in row chunks launches its steps once per chunk: the work of one launch
    is the layer's work over the chunks.  The folded attention-output step also moves the
    residual, Z1 and the statistics; bf16 moves its fp32 tensors at 4 bytes."""
    counts = {"qkv_attention": 48, "attn_out_gemm": 48, "ffn1_gemm": 96, "ffn2_gemm": 96, "ln2": 96}
    assert bench.launches_per_layer(counts, "ffn1_gemm") == 2
    assert bench.launches_per_layer(counts, "ln2") == 2
    assert bench.launches_per_layer(counts, "attn_out_gemm") == 1
    assert bench.launches_per_layer({"ffn1_gemm": 12}, "ffn1_gemm") == 1
    import synthetic_inputs as si
    sh = si.Shape(512, 32, 12, 64, 12, "fp16")
    T, H = sh.tokens, sh.hidden
    fl, plain = bench.step_work(sh, "attn_out_gemm")
    fl2, folded = bench.step_work(sh, "attn_out_gemm", folded=True)
    assert fl == fl2 == 2.0 * T * H * H
    assert folded - plain == T * H * 2 + bench.fold_stats_bytes(sh)  # the residual in, the pairs out
    bf = si.Shape(32, 512, 16, 64, 24, "bf16")
    assert bench.step_work(bf, "ln1")[1] == bf.tokens * bf.hidden * (2 * 2 + 8)
