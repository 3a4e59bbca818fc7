"""ctypes binding of libftx.so, the C ABI declared in include/ftx.h, include/ftx_steps.h and
include/ftx_decoder.h.

Argument marshalling only: every function here checks what a C caller would have to
get right (dtype, device, contiguity, shape), turns tensors into device pointers and
the current torch stream into a hipStream_t, and calls the C function of the same
name.  No step of the encoder or decoder is computed in Python.  If libftx.so is missing the
functions raise: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libftx.so")

FTX_FP32, FTX_FP16, FTX_BF16 = 0, 1, 2
FTX_OK, FTX_ERR_INVALID_ARG, FTX_ERR_UNSUPPORTED, FTX_ERR_OUT_OF_MEMORY, FTX_ERR_DEVICE, \
    FTX_ERR_NOT_READY = range(6)
FTX_OPT_FUSED_EPILOGUES, FTX_OPT_KERNEL_TIMING, FTX_OPT_GRAPH, FTX_OPT_FUSED_ATTENTION = 0, 1, 2, 3
FTX_OPT_FOLD_LAYERNORM = 4
FTX_OPT_PREFETCH_WEIGHTS = 5
STEP_NAMES = ("qkv_gemm", "bias_qkv_split", "attention", "attn_out_gemm", "ln1", "ffn1_gemm",
              "bias_gelu", "ffn2_gemm", "ln2", "qkv_attention", "weight_prefetch")
FTX_NUM_STEPS = len(STEP_NAMES)

WEIGHT_FIELDS = ("w_q", "b_q", "w_k", "b_k", "w_v", "b_v", "w_o", "b_o", "ln1_gamma", "ln1_beta",
                 "w_ffn1", "b_ffn1", "w_ffn2", "b_ffn2", "ln2_gamma", "ln2_beta")

DECODER_WEIGHT_FIELDS = ("w_q", "b_q", "w_k", "b_k", "w_v", "b_v", "w_o", "b_o", "ln1_gamma",
                         "ln1_beta", "w_q2", "b_q2", "w_k2", "b_k2", "w_v2", "b_v2", "w_o2", "b_o2",
                         "ln2_gamma", "ln2_beta", "w_ffn1", "b_ffn1", "w_ffn2", "b_ffn2",
                         "ln3_gamma", "ln3_beta")


EXPORTED = ("ftx_encoder_create", "ftx_set_weights", "ftx_forward", "ftx_forward_static_workspace",
            "ftx_destroy",
            "ftx_status_string", "ftx_last_error", "ftx_set_option", "ftx_kernel_times",
            "ftx_step_linear", "ftx_step_qkv_projection", "ftx_step_qkv_attention",
            "ftx_step_bias_qkv_split",
            "ftx_step_attention", "ftx_step_masked_attention", "ftx_step_bias_residual_layernorm",
            "ftx_step_bias_gelu", "ftx_step_transpose", "ftx_plan_linear",
            "ftx_decoder_create", "ftx_decoder_set_weights", "ftx_decoder_forward",
            "ftx_decoder_set_option", "ftx_decoder_kernel_times", "ftx_decoder_destroy")
DEC_STEP_NAMES = ("self_qkv_gemm", "self_attention", "self_out_gemm", "ln1", "cross_q_gemm",
                  "cross_kv_gemm", "cross_attention", "cross_out_gemm", "ln2", "ffn1_gemm",
                  "ffn2_gemm", "ln3", "self_qkv_attention")

_DTYPES = {torch.float32: FTX_FP32, torch.float16: FTX_FP16, torch.bfloat16: FTX_BF16}
_NAMES = {"fp32": FTX_FP32, "fp16": FTX_FP16, "bf16": FTX_BF16}
TORCH_DTYPE = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


class FtxError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})" + (f": {detail}" if detail else ""))


class ftx_layer_weights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in WEIGHT_FIELDS]


class ftx_decoder_layer_weights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in DECODER_WEIGHT_FIELDS]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libftx.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it first (python -m transformer_encoder_bert_amd.build)")
    lib = ctypes.CDLL(path)
    i, p, v = ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    sig = {
        "ftx_encoder_create": (i, [i, i, i, i, i, i, ctypes.POINTER(p)]),
        "ftx_set_weights": (i, [p, i, ctypes.POINTER(ftx_layer_weights), v]),
        "ftx_forward": (i, [p, p, p, p, v]),
        "ftx_forward_static_workspace": (i, [p, p, p, p, v]),
        "ftx_destroy": (i, [p]),
        "ftx_status_string": (ctypes.c_char_p, [i]),
        "ftx_last_error": (ctypes.c_char_p, []),
        "ftx_set_option": (i, [p, i, i]),
        "ftx_kernel_times": (i, [p, p, p]),
        "ftx_step_linear": (i, [i, i, i, i, p, p, p, i, p, v]),
        "ftx_step_qkv_projection": (i, [i, i, i, i, i, p, p, p, p, p, p, v]),
        "ftx_step_qkv_attention": (i, [i, i, i, i, i, p, p, p, p, i, p, v]),
        "ftx_step_bias_qkv_split": (i, [i, i, i, i, i, p, p, p, p, p, v]),
        "ftx_step_attention": (i, [i, i, i, i, i, p, p, p, p, p, v]),
        "ftx_step_masked_attention": (i, [i, i, i, i, i, i, p, p, p, p, i, p, v]),
        "ftx_decoder_create": (i, [i, i, i, i, i, i, i, ctypes.POINTER(p)]),
        "ftx_decoder_set_weights": (i, [p, i, ctypes.POINTER(ftx_decoder_layer_weights), v]),
        "ftx_decoder_forward": (i, [p, p, p, p, p, v]),
        "ftx_decoder_destroy": (i, [p]),
        "ftx_decoder_set_option": (i, [p, i, i]),
        "ftx_decoder_kernel_times": (i, [p, p, p]),
        "ftx_step_bias_residual_layernorm": (i, [i, i, i, p, p, p, p, p, p, v]),
        "ftx_step_bias_gelu": (i, [i, i, i, p, p, p, v]),
        "ftx_step_transpose": (i, [i, i, i, p, p, v]),
        "ftx_plan_linear": (i, [i, i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i),
                                ctypes.POINTER(i)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().ftx_status_string(status).decode()
    except ImportError:
        return "?"


def _check(status: int, where: str) -> None:
    if status != FTX_OK:
        raise FtxError(status, where, load_library().ftx_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dt(x) -> int:
    if isinstance(x, str):
        return _NAMES[x]
    if isinstance(x, torch.dtype):
        return _DTYPES[x]
    return int(x)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, numel: Optional[int] = None) -> None:
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


# ------------------------------------------------------------------------ the four calls

def ftx_encoder_create(batch_size: int, seq_len: int, head_num: int, size_per_head: int,
                       num_layers: int, dtype) -> ctypes.c_void_p:
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.ftx_encoder_create(batch_size, seq_len, head_num, size_per_head, num_layers,
                                  _dt(dtype), ctypes.byref(h)), "ftx_encoder_create")
    return h


def ftx_set_weights(enc, layer: int, weights: Dict[str, torch.Tensor], stream=None) -> None:
    w = ftx_layer_weights(**{k: _ptr(weights[k]) for k in WEIGHT_FIELDS})
    _check(load_library().ftx_set_weights(enc, layer, ctypes.byref(w), _stream(stream)),
           "ftx_set_weights")


def ftx_forward(enc, x: torch.Tensor, seq_lens: Optional[torch.Tensor], out: torch.Tensor,
                stream=None) -> None:
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32)
    _check(load_library().ftx_forward(enc, _ptr(x), _ptr(seq_lens), _ptr(out), _stream(stream)),
           "ftx_forward")


def ftx_forward_static_workspace(enc, x: torch.Tensor, seq_lens: Optional[torch.Tensor],
                                 out: torch.Tensor, stream=None) -> None:
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32)
    _check(load_library().ftx_forward_static_workspace(enc, _ptr(x), _ptr(seq_lens), _ptr(out),
                                                       _stream(stream)),
           "ftx_forward_static_workspace")


def ftx_destroy(enc) -> None:
    _check(load_library().ftx_destroy(enc), "ftx_destroy")


def ftx_set_option(enc, option: int, value: int) -> None:
    _check(load_library().ftx_set_option(enc, option, value), "ftx_set_option")


def ftx_kernel_times(enc):
    ms = (ctypes.c_double * FTX_NUM_STEPS)()
    counts = (ctypes.c_int64 * FTX_NUM_STEPS)()
    _check(load_library().ftx_kernel_times(enc, ms, counts), "ftx_kernel_times")
    return {STEP_NAMES[i]: (ms[i], counts[i]) for i in range(FTX_NUM_STEPS)}


class Encoder:
    """Owns one handle.  ``forward`` allocates the output tensor and calls ftx_forward."""

    def __init__(self, batch_size: int, seq_len: int, head_num: int, size_per_head: int,
                 num_layers: int, dtype: str):
        self.shape = (batch_size, seq_len, head_num * size_per_head)
        self.num_layers = num_layers
        self.dtype = TORCH_DTYPE[dtype]
        self.handle = ftx_encoder_create(batch_size, seq_len, head_num, size_per_head,
                                         num_layers, dtype)

    def set_weights(self, layer: int, weights: Dict[str, torch.Tensor], stream=None) -> None:
        for k in WEIGHT_FIELDS:
            _need(weights[k], k, self.dtype)
        ftx_set_weights(self.handle, layer, weights, stream)

    def forward(self, x: torch.Tensor, seq_lens: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        # the kernels read seq_lens[b] for every sequence b of the batch
        if seq_lens is not None:
            _need(seq_lens, "seq_lens", torch.int32, self.shape[0])
        _need(x, "input", self.dtype, self.shape[0] * self.shape[1] * self.shape[2])
        if seq_lens is not None and seq_lens.device != x.device:
            raise ValueError(f"seq_lens is on {seq_lens.device}, input on {x.device}")
        if out is None:
            out = torch.empty(self.shape, dtype=self.dtype, device=x.device)
        _need(out, "output", self.dtype, x.numel())
        ftx_forward(self.handle, x, seq_lens, out, stream)
        return out

    def forward_static_workspace(self, x: torch.Tensor, seq_lens: Optional[torch.Tensor],
                                 out: torch.Tensor, stream=None) -> torch.Tensor:
        """ftx_forward_static_workspace: the forward with the library's static scratch as
        workspace; ``out`` is the caller's (nothing is allocated)."""
        if seq_lens is not None:
            _need(seq_lens, "seq_lens", torch.int32, self.shape[0])
        _need(x, "input", self.dtype, self.shape[0] * self.shape[1] * self.shape[2])
        _need(out, "output", self.dtype, x.numel())
        ftx_forward_static_workspace(self.handle, x, seq_lens, out, stream)
        return out

    def set_option(self, option: int, value: int) -> None:
        ftx_set_option(self.handle, option, value)

    def kernel_times(self):
        return ftx_kernel_times(self.handle)

    def close(self) -> None:
        if self.handle is not None:
            ftx_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------------ decoder

def ftx_decoder_create(batch_size: int, tgt_len: int, mem_len: int, head_num: int,
                       size_per_head: int, num_layers: int, dtype) -> ctypes.c_void_p:
    lib = load_library()
    h = ctypes.c_void_p()
    _check(lib.ftx_decoder_create(batch_size, tgt_len, mem_len, head_num, size_per_head,
                                  num_layers, _dt(dtype), ctypes.byref(h)), "ftx_decoder_create")
    return h


def ftx_decoder_set_weights(dec, layer: int, weights: Dict[str, torch.Tensor], stream=None) -> None:
    w = ftx_decoder_layer_weights(**{k: _ptr(weights[k]) for k in DECODER_WEIGHT_FIELDS})
    _check(load_library().ftx_decoder_set_weights(dec, layer, ctypes.byref(w), _stream(stream)),
           "ftx_decoder_set_weights")


def ftx_decoder_forward(dec, x: torch.Tensor, memory: torch.Tensor,
                        mem_lens: Optional[torch.Tensor], out: torch.Tensor, stream=None) -> None:
    if mem_lens is not None:
        _need(mem_lens, "mem_lens", torch.int32)
    _check(load_library().ftx_decoder_forward(dec, _ptr(x), _ptr(memory), _ptr(mem_lens), _ptr(out),
                                              _stream(stream)), "ftx_decoder_forward")


def ftx_decoder_destroy(dec) -> None:
    _check(load_library().ftx_decoder_destroy(dec), "ftx_decoder_destroy")


def ftx_decoder_set_option(dec, option: int, value: int) -> None:
    _check(load_library().ftx_decoder_set_option(dec, option, value), "ftx_decoder_set_option")


def ftx_decoder_kernel_times(dec):
    n = len(DEC_STEP_NAMES)
    ms = (ctypes.c_double * n)()
    counts = (ctypes.c_int64 * n)()
    _check(load_library().ftx_decoder_kernel_times(dec, ms, counts), "ftx_decoder_kernel_times")
    return {DEC_STEP_NAMES[i]: (ms[i], counts[i]) for i in range(n)}


class Decoder:
    """Owns one decoder handle.  ``forward(x, memory, mem_lens)`` allocates the output and
    calls ftx_decoder_forward."""

    def __init__(self, batch_size: int, tgt_len: int, mem_len: int, head_num: int,
                 size_per_head: int, num_layers: int, dtype: str):
        H = head_num * size_per_head
        self.shape = (batch_size, tgt_len, H)
        self.mem_shape = (batch_size, mem_len, H)
        self.num_layers = num_layers
        self.dtype = TORCH_DTYPE[dtype]
        self.handle = ftx_decoder_create(batch_size, tgt_len, mem_len, head_num, size_per_head,
                                         num_layers, dtype)

    def set_weights(self, layer: int, weights: Dict[str, torch.Tensor], stream=None) -> None:
        for k in DECODER_WEIGHT_FIELDS:
            _need(weights[k], k, self.dtype)
        ftx_decoder_set_weights(self.handle, layer, weights, stream)

    def forward(self, x: torch.Tensor, memory: torch.Tensor, mem_lens: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        _need(x, "input", self.dtype, self.shape[0] * self.shape[1] * self.shape[2])
        _need(memory, "memory", self.dtype, self.mem_shape[0] * self.mem_shape[1] * self.mem_shape[2])
        if mem_lens is not None:
            _need(mem_lens, "mem_lens", torch.int32, self.shape[0])
        if out is None:
            out = torch.empty(self.shape, dtype=self.dtype, device=x.device)
        _need(out, "output", self.dtype, x.numel())
        ftx_decoder_forward(self.handle, x, memory, mem_lens, out, stream)
        return out

    def set_option(self, option: int, value: int) -> None:
        ftx_decoder_set_option(self.handle, option, value)

    def kernel_times(self):
        return ftx_decoder_kernel_times(self.handle)

    def close(self) -> None:
        if self.handle is not None:
            ftx_decoder_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------------ step entry points

def ftx_step_linear(a: torch.Tensor, w_t: torch.Tensor, bias: Optional[torch.Tensor], gelu: bool,
                    c: torch.Tensor, stream=None) -> None:
    M, K = a.shape
    N = w_t.shape[0]
    for t, nm in ((a, "a"), (w_t, "w_t"), (c, "c")):
        _need(t, nm, a.dtype)
    if w_t.shape[1] != K or tuple(c.shape) != (M, N):
        raise ValueError("shape mismatch")
    if bias is not None:
        _need(bias, "bias", a.dtype, N)
    _check(load_library().ftx_step_linear(_dt(a.dtype), M, N, K, _ptr(a), _ptr(w_t), _ptr(bias),
                                          int(bool(gelu)), _ptr(c), _stream(stream)), "ftx_step_linear")


def ftx_step_qkv_projection(B, S, n, d, x, w_qkv_t, b_qkv, q, k, v_t, stream=None) -> None:
    H = n * d
    _need(x, "x", x.dtype, B * S * H)
    _need(w_qkv_t, "w_qkv_t", x.dtype, 3 * H * H)
    _need(b_qkv, "b_qkv", x.dtype, 3 * H)
    for t, nm in ((q, "q"), (k, "k"), (v_t, "v_t")):
        _need(t, nm, x.dtype, B * S * H)
    _check(load_library().ftx_step_qkv_projection(_dt(x.dtype), B, S, n, d, _ptr(x), _ptr(w_qkv_t),
                                                  _ptr(b_qkv), _ptr(q), _ptr(k), _ptr(v_t),
                                                  _stream(stream)), "ftx_step_qkv_projection")


def ftx_step_qkv_attention(B, S, n, d, x, w_qkv_t, b_qkv, seq_lens, ctx, causal=False,
                           stream=None) -> None:
    """w_qkv_t / b_qkv rows ordered per head: [Q_h | K_h | V_h] for h = 0 .. n-1."""
    H = n * d
    _need(x, "x", x.dtype, B * S * H)
    _need(w_qkv_t, "w_qkv_t", x.dtype, 3 * H * H)
    _need(b_qkv, "b_qkv", x.dtype, 3 * H)
    _need(ctx, "ctx", x.dtype, B * S * H)
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32, B)
    _check(load_library().ftx_step_qkv_attention(_dt(x.dtype), B, S, n, d, _ptr(x), _ptr(w_qkv_t),
                                                 _ptr(b_qkv), _ptr(seq_lens), int(bool(causal)),
                                                 _ptr(ctx), _stream(stream)), "ftx_step_qkv_attention")


def ftx_step_bias_qkv_split(B, S, n, d, qkv, b_qkv, q, k, v_t, stream=None) -> None:
    H = n * d
    _need(qkv, "qkv", qkv.dtype, B * S * 3 * H)
    _need(b_qkv, "b_qkv", qkv.dtype, 3 * H)
    for t, nm in ((q, "q"), (k, "k"), (v_t, "v_t")):
        _need(t, nm, qkv.dtype, B * S * H)
    _check(load_library().ftx_step_bias_qkv_split(_dt(qkv.dtype), B, S, n, d, _ptr(qkv), _ptr(b_qkv),
                                                  _ptr(q), _ptr(k), _ptr(v_t), _stream(stream)),
           "ftx_step_bias_qkv_split")


def ftx_step_attention(B, S, n, d, q, k, v_t, seq_lens, ctx, stream=None) -> None:
    H = n * d
    for t, nm in ((q, "q"), (k, "k"), (v_t, "v_t"), (ctx, "ctx")):
        _need(t, nm, q.dtype, B * S * H)
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32, B)
    _check(load_library().ftx_step_attention(_dt(q.dtype), B, S, n, d, _ptr(q), _ptr(k), _ptr(v_t),
                                             _ptr(seq_lens), _ptr(ctx), _stream(stream)),
           "ftx_step_attention")


def ftx_step_masked_attention(B, Sq, Sk, n, d, q, k, v_t, key_lens, causal, ctx, stream=None) -> None:
    H = n * d
    _need(q, "q", q.dtype, B * Sq * H)
    _need(k, "k", q.dtype, B * Sk * H)
    _need(v_t, "v_t", q.dtype, B * Sk * H)
    _need(ctx, "ctx", q.dtype, B * Sq * H)
    if key_lens is not None:
        _need(key_lens, "key_lens", torch.int32, B)
    _check(load_library().ftx_step_masked_attention(_dt(q.dtype), B, Sq, Sk, n, d, _ptr(q), _ptr(k),
                                                    _ptr(v_t), _ptr(key_lens), int(bool(causal)),
                                                    _ptr(ctx), _stream(stream)),
           "ftx_step_masked_attention")


def ftx_step_bias_residual_layernorm(x, a, bias, gamma, beta, y, stream=None) -> None:
    rows, cols = x.shape
    for t, nm in ((x, "x"), (a, "a"), (y, "y")):
        _need(t, nm, x.dtype, rows * cols)
    for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        _need(t, nm, x.dtype, cols)
    _check(load_library().ftx_step_bias_residual_layernorm(
        _dt(x.dtype), rows, cols, _ptr(x), _ptr(a), _ptr(bias), _ptr(gamma), _ptr(beta), _ptr(y),
        _stream(stream)), "ftx_step_bias_residual_layernorm")


def ftx_step_bias_gelu(u, bias, g, stream=None) -> None:
    rows, cols = u.shape
    _need(u, "u", u.dtype)
    _need(g, "g", u.dtype, rows * cols)
    _need(bias, "bias", u.dtype, cols)
    _check(load_library().ftx_step_bias_gelu(_dt(u.dtype), rows, cols, _ptr(u), _ptr(bias), _ptr(g),
                                             _stream(stream)), "ftx_step_bias_gelu")


def ftx_step_transpose(inp, out, stream=None) -> None:
    rows, cols = inp.shape
    _need(inp, "in", inp.dtype)
    _need(out, "out", inp.dtype, rows * cols)
    _check(load_library().ftx_step_transpose(_dt(inp.dtype), rows, cols, _ptr(inp), _ptr(out),
                                             _stream(stream)), "ftx_step_transpose")


def ftx_plan_linear(dtype, M: int, N: int, K: int, cus: int, sums_partials: bool = False):
    """(tile_m, tile_n, splits) of an M x N x K projection on a device with `cus` CUs.
    Host arithmetic in the library; needs no GPU."""
    tm, tn, sp = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(load_library().ftx_plan_linear(_dt(dtype), M, N, K, cus, int(bool(sums_partials)),
                                          ctypes.byref(tm), ctypes.byref(tn), ctypes.byref(sp)),
           "ftx_plan_linear")
    return tm.value, tn.value, sp.value
