"""Seeded synthetic inputs for the BERT-style encoder forward.

This module draws random numbers and nothing else of the method: it holds no
projection, attention, normalisation or activation arithmetic.  Both sides of a
parity check (the fp64 oracle and the HIP library) consume what it returns.

Workload shapes follow the Faster Transformer article ("有钱任性：英伟达训练80亿参数量
GPT-2，1475块V100 53分钟训练BERT", cloud.tencent.com/developer/article/1490359):
section "什么是 Faster Transformer" names the four runtime parameters (head count,
size per head, batch size, maximum sentence length 32/64/128) and the FP16/FP32
modes; section "Faster Transformer 性能怎么样" benchmarks a 12-layer encoder at
sequence length 32 over a batch sweep for the 12x64 model and a pruned 4x32 model.
The sequence-length-512 and bf16 shapes extend that family (BERT-large).

Conventions
-----------
* Every value is drawn in float64 from numpy's PCG64, then rounded to the run's
  storage format with round-to-nearest-even, ONCE.  The arrays handed out are
  float64 arrays whose every element is exactly representable in that format,
  so the oracle (which upcasts nothing further) and the GPU (which stores the
  format) see identical numbers.
* Streams: ``SeedSequence(seed)`` -> optional variant spawn -> three children
  (weights, input, lengths); the weights child spawns one stream per layer and
  each layer stream one per tensor.  A layer's weights can therefore be drawn
  on demand, in any order, with the same result.
* Batch sweeps draw the input and lengths at the largest batch of the sweep and
  take a prefix, so a smaller batch is a prefix of a larger one.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Iterator, Optional, Tuple

import numpy as np

# (significand bits including the implicit one, smallest normal exponent)
_FORMATS = {"fp32": (24, -126), "fp16": (11, -14), "bf16": (8, -126)}
_MAX_FINITE = {"fp32": float(np.finfo(np.float32).max), "fp16": 65504.0,
               "bf16": float.fromhex("0x1.fep127")}

DTYPES = tuple(_FORMATS)

# Field names of one layer's weights, in the order of the C struct.
WEIGHT_NAMES = ("w_q", "b_q", "w_k", "b_k", "w_v", "b_v", "w_o", "b_o",
                "ln1_gamma", "ln1_beta", "w_ffn1", "b_ffn1", "w_ffn2", "b_ffn2",
                "ln2_gamma", "ln2_beta")


def round_to(x, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` (round-to-nearest-even), returned as float64.

    Works from the float64 value directly (no intermediate float32 step, so no
    double rounding).  Subnormals of the target format are handled; values that
    would overflow the format raise.
    """
    p, emin = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value")
    if np.any(np.abs(x) > _MAX_FINITE[dtype]):
        raise OverflowError(f"value outside {dtype} range")
    _, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    qexp = np.maximum(e - p, emin - p + 1)  # exponent of one unit in the last place
    scale = np.ldexp(1.0, qexp)
    out = np.rint(x / scale) * scale        # exact scaling; rint is half-to-even
    if np.any(np.abs(out) > _MAX_FINITE[dtype]):
        raise OverflowError(f"value rounds outside {dtype} range")
    return out


@dataclass(frozen=True)
class Shape:
    """The four runtime parameters plus layer count and storage dtype."""
    batch: int
    seq_len: int
    head_num: int
    size_per_head: int
    num_layers: int
    dtype: str

    @property
    def hidden(self) -> int:
        return self.head_num * self.size_per_head

    @property
    def ffn(self) -> int:
        return 4 * self.hidden

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def flops(self) -> float:
        """Algorithmic dense-contraction flops of one forward at the padded length.

        Per layer: the four projections 2*T*(3H*H + H*H + H*4H + 4H*H) = 24*T*H^2,
        plus scores and context 2 * 2*T*S*H.
        """
        T, S, H = self.tokens, self.seq_len, self.hidden
        return float(self.num_layers) * (24.0 * T * H * H + 4.0 * T * S * H)

    def valid_flops(self, lens) -> float:
        """The same count on the valid tokens only: the projections on sum(len_b) rows, scores
        and context over len_b queries and len_b keys per sequence."""
        ln = np.asarray(lens, dtype=np.float64)
        H = self.hidden
        return float(self.num_layers) * (24.0 * ln.sum() * H * H + 4.0 * (ln * ln).sum() * H)


@dataclass(frozen=True)
class Workload:
    """One synthetic configuration: a shape family, its distributions and its seed."""
    name: str
    description: str
    seq_len: int
    head_num: int
    size_per_head: int
    num_layers: int
    dtype: str
    batches: Tuple[int, ...]
    seed: int
    variant: Optional[int] = None          # spawn index for families with two seq lengths
    lens: Optional[Tuple[str, int, int]] = None   # ("one"|"each", lo, hi) or None = no padding
    weight_std: float = 0.02

    def shape(self, batch: Optional[int] = None, num_layers: Optional[int] = None) -> Shape:
        b = max(self.batches) if batch is None else batch
        nl = self.num_layers if num_layers is None else num_layers
        return Shape(b, self.seq_len, self.head_num, self.size_per_head, nl, self.dtype)


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("single_layer_fp32",
             "single encoder layer fp32, batch 1, seq 32, 4x32 (hidden 128), one seeded valid length in [16,32]",
             seq_len=32, head_num=4, size_per_head=32, num_layers=1, dtype="fp32",
             batches=(1,), seed=101, lens=("one", 16, 32)),
    Workload("bert_base_fp16_s32",
             "BERT-base 12 layers 12x64 fp16, seq 32, no padding",
             seq_len=32, head_num=12, size_per_head=64, num_layers=12, dtype="fp16",
             batches=(1, 8, 64, 128, 256, 512), seed=102),
    Workload("pruned_fp16_s32",
             "pruned 12 layers 4x32 fp16, seq 32, no padding",
             seq_len=32, head_num=4, size_per_head=32, num_layers=12, dtype="fp16",
             batches=(1, 64, 512), seed=103),
    Workload("bert_base_fp16_s64_varlen",
             "BERT-base 12 layers 12x64 fp16, seq 64, lengths uniform in [16,64]",
             seq_len=64, head_num=12, size_per_head=64, num_layers=12, dtype="fp16",
             batches=(1, 64), seed=104, variant=0, lens=("each", 16, 64)),
    Workload("bert_base_fp16_s128_varlen",
             "BERT-base 12 layers 12x64 fp16, seq 128, lengths uniform in [32,128]",
             seq_len=128, head_num=12, size_per_head=64, num_layers=12, dtype="fp16",
             batches=(1, 64), seed=104, variant=1, lens=("each", 32, 128)),
    Workload("bert_large_bf16_s128",
             "BERT-large 24 layers 16x64 bf16, seq 128, batch 256, lengths uniform in [64,128]",
             seq_len=128, head_num=16, size_per_head=64, num_layers=24, dtype="bf16",
             batches=(256,), seed=105, variant=0, lens=("each", 64, 128)),
    Workload("bert_large_bf16_s512",
             "BERT-large 24 layers 16x64 bf16, seq 512, batch 32, lengths uniform in [64,512]",
             seq_len=512, head_num=16, size_per_head=64, num_layers=24, dtype="bf16",
             batches=(32,), seed=105, variant=1, lens=("each", 64, 512)),
]}


def _child(ss: np.random.SeedSequence, i: int) -> np.random.SeedSequence:
    """The i-th child of ``ss``, as ``ss.spawn`` would make it, but without the
    spawn counter's state: the same call always gives the same stream."""
    return np.random.SeedSequence(entropy=ss.entropy, spawn_key=tuple(ss.spawn_key) + (i,),
                                  pool_size=ss.pool_size)


def _root(w: Workload) -> Tuple[np.random.SeedSequence, np.random.SeedSequence, np.random.SeedSequence]:
    ss = np.random.SeedSequence(w.seed)
    if w.variant is not None:
        ss = _child(ss, w.variant)
    return _child(ss, 0), _child(ss, 1), _child(ss, 2)


@dataclass
class Case:
    """A fully drawn synthetic case (weights drawn lazily, per layer)."""
    workload: Workload
    shape: Shape
    x: np.ndarray                     # [B, S, H] float64, exactly representable in dtype
    lens: Optional[np.ndarray]        # [B] int32 in [1, S], or None (no padding)
    params: str = "bert"              # "bert" | "random_affine"
    _layer_seqs: list = field(default_factory=list, repr=False)

    def layer(self, l: int) -> Dict[str, np.ndarray]:
        return _draw_layer(self._layer_seqs[l], self.shape, self.workload.weight_std,
                           self.params)

    def layers(self) -> Iterator[Dict[str, np.ndarray]]:
        for l in range(self.shape.num_layers):
            yield self.layer(l)

    def lens_or_full(self) -> np.ndarray:
        if self.lens is None:
            return np.full(self.shape.batch, self.shape.seq_len, dtype=np.int32)
        return self.lens


def _draw_layer(seq: np.random.SeedSequence, shape: Shape, std: float, params: str) -> Dict[str, np.ndarray]:
    H, F, dt = shape.hidden, shape.ffn, shape.dtype
    seqs = {name: _child(seq, i) for i, name in enumerate(WEIGHT_NAMES)}
    dims = {"w_q": (H, H), "w_k": (H, H), "w_v": (H, H), "w_o": (H, H),
            "w_ffn1": (H, F), "w_ffn2": (F, H)}
    vec = {"b_q": H, "b_k": H, "b_v": H, "b_o": H, "ln1_gamma": H, "ln1_beta": H,
           "b_ffn1": F, "b_ffn2": H, "ln2_gamma": H, "ln2_beta": H}
    out: Dict[str, np.ndarray] = {}
    for name in WEIGHT_NAMES:
        rng = np.random.Generator(np.random.PCG64(seqs[name]))
        if name in dims:
            out[name] = round_to(rng.normal(0.0, std, size=dims[name]), dt)
            continue
        n = vec[name]
        if params == "bert":
            val = np.ones(n) if name.endswith("gamma") else np.zeros(n)
        elif params == "random_affine":
            if name.endswith("gamma"):
                val = 1.0 + rng.normal(0.0, 0.2, size=n)
            else:
                val = rng.normal(0.0, 0.2, size=n)
        else:
            raise ValueError(params)
        out[name] = round_to(val, dt)
    return out


def make_case(workload: str | Workload, batch: Optional[int] = None, *,
              num_layers: Optional[int] = None, params: str = "bert",
              draw_batch: Optional[int] = None) -> Case:
    """Draw a case of ``workload`` at ``batch`` (default: the largest of its sweep).

    ``num_layers`` truncates the stack (layer l of a truncated case equals layer l
    of the full one).  ``draw_batch`` overrides the batch the input and lengths
    are drawn at before the prefix is taken (default: the sweep's largest, or
    ``batch`` when that is larger).
    """
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    shape = w.shape(batch, num_layers)
    wseq, xseq, lseq = _root(w)
    nb = draw_batch if draw_batch is not None else max(max(w.batches), shape.batch)
    if nb < shape.batch:
        raise ValueError("draw_batch smaller than batch")
    xr = np.random.Generator(np.random.PCG64(xseq))
    x = round_to(xr.standard_normal(size=(nb, shape.seq_len, shape.hidden)), shape.dtype)
    x = x[:shape.batch]
    lens = None
    if w.lens is not None:
        kind, lo, hi = w.lens
        lr = np.random.Generator(np.random.PCG64(lseq))
        if kind == "one":
            lens = np.full(nb, lr.integers(lo, hi, endpoint=True), dtype=np.int32)
        else:
            lens = lr.integers(lo, hi, size=nb, endpoint=True).astype(np.int32)
        lens = lens[:shape.batch].copy()
    layer_seqs = [_child(wseq, l) for l in range(w.num_layers)]
    return Case(w, shape, np.ascontiguousarray(x), lens, params, layer_seqs)


def custom_case(shape: Shape, seed: int, *, lens: Optional[np.ndarray] = None,
                params: str = "bert", weight_std: float = 0.02,
                lens_range: Optional[Tuple[int, int]] = None) -> Case:
    """A case of arbitrary shape (edge cases: ragged batches, odd head counts...)."""
    w = Workload("custom", "custom", shape.seq_len, shape.head_num, shape.size_per_head,
                 shape.num_layers, shape.dtype, (shape.batch,), seed,
                 lens=None if lens_range is None else ("each",) + tuple(lens_range),
                 weight_std=weight_std)
    c = make_case(w, shape.batch, params=params)
    if lens is not None:
        c.lens = np.asarray(lens, dtype=np.int32).copy()
    return c


# ----------------------------------------------------------------------------- decoder
# Draws for the decoder forward (the article's roadmap item): the same conventions as the
# encoder's -- float64 PCG64 draws rounded once to the storage format, one stream per tensor.

# Field names of one decoder layer's weights, in the order of the C struct: causal
# self-attention, cross-attention over the memory, feed-forward, each with its LayerNorm.
DECODER_WEIGHT_NAMES = ("w_q", "b_q", "w_k", "b_k", "w_v", "b_v", "w_o", "b_o",
                        "ln1_gamma", "ln1_beta",
                        "w_q2", "b_q2", "w_k2", "b_k2", "w_v2", "b_v2", "w_o2", "b_o2",
                        "ln2_gamma", "ln2_beta",
                        "w_ffn1", "b_ffn1", "w_ffn2", "b_ffn2", "ln3_gamma", "ln3_beta")


@dataclass(frozen=True)
class DecoderShape:
    batch: int
    tgt_len: int      # decoder positions per sequence
    mem_len: int      # memory (encoder output) positions per sequence
    head_num: int
    size_per_head: int
    num_layers: int
    dtype: str

    @property
    def hidden(self) -> int:
        return self.head_num * self.size_per_head

    @property
    def ffn(self) -> int:
        return 4 * self.hidden

    def flops(self) -> float:
        """Algorithmic dense-contraction flops of one forward at the padded lengths.

        Per layer, T = B*tgt_len decoder rows and Tm = B*mem_len memory rows: self-attention
        projections 8*T*H^2 (Q, K, V, O), cross-attention Q and O 4*T*H^2, its K and V on the
        memory 4*Tm*H^2, feed-forward 16*T*H^2, and scores plus context 4*T*tgt_len*H
        (self) and 4*T*mem_len*H (cross), all at the full padded extent.
        """
        T, Tm, H = self.batch * self.tgt_len, self.batch * self.mem_len, self.hidden
        per = 28.0 * T * H * H + 4.0 * Tm * H * H + 4.0 * T * (self.tgt_len + self.mem_len) * H
        return float(self.num_layers) * per


@dataclass
class DecoderCase:
    shape: DecoderShape
    x: np.ndarray                  # [B, tgt_len, H]
    mem: np.ndarray                # [B, mem_len, H]
    mem_lens: Optional[np.ndarray]  # [B] int32 in [1, mem_len], or None
    params: str
    weight_std: float
    _layer_seqs: list = field(default_factory=list, repr=False)

    def layer(self, l: int) -> Dict[str, np.ndarray]:
        sh, dt = self.shape, self.shape.dtype
        H, F = sh.hidden, sh.ffn
        seqs = {name: _child(self._layer_seqs[l], i) for i, name in enumerate(DECODER_WEIGHT_NAMES)}
        out: Dict[str, np.ndarray] = {}
        for name in DECODER_WEIGHT_NAMES:
            rng = np.random.Generator(np.random.PCG64(seqs[name]))
            if name.startswith("w_"):
                dims = (H, F) if name == "w_ffn1" else (F, H) if name == "w_ffn2" else (H, H)
                out[name] = round_to(rng.normal(0.0, self.weight_std, size=dims), dt)
                continue
            n = F if name == "b_ffn1" else H
            if self.params == "bert":
                val = np.ones(n) if name.endswith("gamma") else np.zeros(n)
            elif self.params == "random_affine":
                val = (1.0 if name.endswith("gamma") else 0.0) + rng.normal(0.0, 0.2, size=n)
            else:
                raise ValueError(self.params)
            out[name] = round_to(val, dt)
        return out

    def layers(self) -> Iterator[Dict[str, np.ndarray]]:
        for l in range(self.shape.num_layers):
            yield self.layer(l)


def make_decoder_case(shape: DecoderShape, seed: int, *, params: str = "bert",
                      weight_std: float = 0.02,
                      mem_lens_range: Optional[Tuple[int, int]] = None,
                      mem_lens: Optional[np.ndarray] = None) -> DecoderCase:
    """Decoder input x ~ N(0, 1), memory ~ N(0, 1) (standing in for an encoder output),
    memory lengths uniform in ``mem_lens_range`` (or given, or None = no padding).
    Streams: SeedSequence(seed) -> weights (one per layer, one per tensor), x, memory,
    lengths."""
    ss = np.random.SeedSequence(seed)
    wseq, xseq, mseq, lseq = (_child(ss, i) for i in range(4))
    B, H, dt = shape.batch, shape.hidden, shape.dtype
    x = round_to(np.random.Generator(np.random.PCG64(xseq)).standard_normal((B, shape.tgt_len, H)), dt)
    mem = round_to(np.random.Generator(np.random.PCG64(mseq)).standard_normal((B, shape.mem_len, H)), dt)
    lens = None
    if mem_lens is not None:
        lens = np.asarray(mem_lens, dtype=np.int32).copy()
    elif mem_lens_range is not None:
        lo, hi = mem_lens_range
        lens = np.random.Generator(np.random.PCG64(lseq)).integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    return DecoderCase(shape, np.ascontiguousarray(x), np.ascontiguousarray(mem), lens, params,
                       weight_std, [_child(wseq, l) for l in range(shape.num_layers)])


# The decoder benchmark shape: BERT-base sized (12 layers, 12x64 heads), 32 decoder
# positions attending to a 32-position memory with lengths uniform in [16, 32].
DECODER_WORKLOAD = dict(name="decoder_base_fp16_s32",
                        description="decoder 12 layers 12x64 fp16, 32 positions, memory 32 "
                                    "(lengths uniform in [16,32])",
                        tgt_len=32, mem_len=32, head_num=12, size_per_head=64, num_layers=12,
                        dtype="fp16", batches=(1, 64, 512), seed=106, mem_lens_range=(16, 32))


def host_array(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage-format numpy array of an exactly representable float64 array.

    fp32 -> float32, fp16 -> float16, bf16 -> uint16 bit patterns (the upper half
    of the float32 encoding, exact because the value is representable)."""
    if dtype == "fp32":
        return a.astype(np.float32)
    if dtype == "fp16":
        return a.astype(np.float16)
    if dtype == "bf16":
        return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    raise ValueError(dtype)


def from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """float64 values of bf16 bit patterns (uint16)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
