"""Seeded synthetic workloads for the Blockwise Parallel Transformer layer.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It holds only layer shapes and seeded random numbers: none of the
layer's arithmetic lives here.

Shapes follow the five single-layer workloads the layer is measured on:

* ``gpt-tiny-fp32``   s=256, h=64, 2 heads x 32, ReLU FFN 64->256->64, biases,
                      pre-LayerNorm, causal, query/KV blocks 64 (fp32).
* ``gpt1b-s8k``       GPT-1B-shaped layer (h=2048, 16 heads x 128, GeLU FFN 4h),
                      s=8192, query block 1024, KV block 2048 (bf16 storage).
* ``gpt1b-s128k``     the same layer at s=131072, query block 2048, KV block 4096.
* ``llama8b-s64k``    Llama3-8B-shaped layer: h=4096, 32 query / 8 KV heads x 128
                      (GQA), RoPE base 500000, RMSNorm, SwiGLU 4096->14336->4096,
                      no biases, s=65536, 8 query heads per head chunk.
* ``llama70b-s8k``    70B-shaped layer: h=8192, 64 query / 8 KV heads x 128,
                      RMSNorm, SwiGLU 8192->28672->8192, no biases, s=8192.

Value recipe (the pages' workloads are OpenWebText and long synthetic
sequences; neither corpus is used, only shapes matter):

* x ~ N(0, 1); every weight matrix ~ N(0, 1/fan_in) (variance 1/fan_in, fan_in
  the matrix's input width); biases 0; norm scales 1 and shifts 0; the output
  cotangent dy ~ N(0, 1).
* Each tensor has its own seed, ``1000 * workload_id + tensor_id``, drawn with
  NumPy's PCG64 ``standard_normal(dtype=float32)`` and scaled in float32.
* In bf16 mode every tensor is rounded to bf16 by round-to-nearest-even of its
  float32 bits; the same bf16 values (converted exactly to float64) feed the
  oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

TENSOR_IDS = {
    "x": 0, "w_qkv": 1, "w_o": 2, "w_1": 3, "w_2": 4, "w_3": 5,
    "b_qkv": 6, "b_o": 7, "b_1": 8, "dy": 9, "b_2": 10,
    "n1_g": 11, "n1_b": 12, "n2_g": 13, "n2_b": 14,
}


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    wid: int                 # seed family
    dtype: str               # "f32" or "bf16"
    batch: int
    seq_len: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    norm: str                # "layernorm" | "rmsnorm"
    ffn: str                 # "relu" | "gelu" | "swiglu"
    has_bias: bool
    causal: bool
    rope_base: Optional[float]
    q_block: int
    kv_block: int
    head_chunk: int
    norm_eps: float = 1e-5
    window: int = 0          # causal sliding window (0: none)
    dropout_p: float = 0.0   # attention-probability dropout (0: none)
    seed: int = 0            # dropout seed

    def replace(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)

    @property
    def qkv_cols(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


WORKLOADS: Dict[str, LayerShape] = {
    "gpt-tiny-fp32": LayerShape("gpt-tiny-fp32", 1, "f32", 1, 256, 64, 2, 2, 32, 256,
                                "layernorm", "relu", True, True, None, 64, 64, 2),
    "gpt1b-s8k": LayerShape("gpt1b-s8k", 2, "bf16", 1, 8192, 2048, 16, 16, 128, 8192,
                            "layernorm", "gelu", True, True, None, 1024, 2048, 16),
    "gpt1b-s128k": LayerShape("gpt1b-s128k", 3, "bf16", 1, 131072, 2048, 16, 16, 128, 8192,
                              "layernorm", "gelu", True, True, None, 2048, 4096, 16),
    "llama8b-s64k": LayerShape("llama8b-s64k", 4, "bf16", 1, 65536, 4096, 32, 8, 128, 14336,
                               "rmsnorm", "swiglu", False, True, 500000.0, 1024, 2048, 8),
    "llama70b-s8k": LayerShape("llama70b-s8k", 5, "bf16", 1, 8192, 8192, 64, 8, 128, 28672,
                               "rmsnorm", "swiglu", False, True, None, 1024, 2048, 64),
}

# The small-hidden shape of the pages' reinforcement-learning experiment: an
# Agentic-Transformer-style GPT of 3 layers, embedding 128, one attention head,
# over 32 trajectories x 1000 steps x 4 tokens = 128000 positions (one
# trajectory per query block). Run as a stack of 3 layers.
RL_SMALL_H = LayerShape("rl-small-h-s128k", 6, "bf16", 1, 128000, 128, 1, 1, 128, 512,
                        "layernorm", "gelu", True, True, None, 4000, 4000, 1)
RL_SMALL_H_LAYERS = 3

# Reduced shapes that keep each workload's structure (dtype, norm, FFN kind,
# GQA grouping, RoPE, head chunking) at sizes the float64 oracle finishes in
# seconds; sequence lengths are chosen so the last attention and GEMM tiles are
# partial (ragged).
SMALL: Dict[str, LayerShape] = {
    "gpt-tiny-fp32": WORKLOADS["gpt-tiny-fp32"],
    "gpt-small-fp32-ragged": WORKLOADS["gpt-tiny-fp32"].replace(
        name="gpt-small-fp32-ragged", seq_len=208, q_block=104, kv_block=52),
    "gpt1b-small": WORKLOADS["gpt1b-s8k"].replace(
        name="gpt1b-small", seq_len=784, hidden=256, n_heads=2, n_kv_heads=2, ffn_dim=1024,
        q_block=392, kv_block=196, head_chunk=2),
    "gpt1b-small-chunked": WORKLOADS["gpt1b-s8k"].replace(
        name="gpt1b-small-chunked", seq_len=512, hidden=512, n_heads=4, n_kv_heads=4,
        ffn_dim=2048, q_block=128, kv_block=256, head_chunk=2),
    "llama8b-small": WORKLOADS["llama8b-s64k"].replace(
        name="llama8b-small", seq_len=656, hidden=512, n_heads=4, n_kv_heads=2, ffn_dim=1536,
        q_block=328, kv_block=164, head_chunk=2),
    "llama70b-small": WORKLOADS["llama70b-s8k"].replace(
        name="llama70b-small", seq_len=400, hidden=1024, n_heads=8, n_kv_heads=2,
        ffn_dim=2816, q_block=200, kv_block=400, head_chunk=8),
    # Code paths the five workloads do not reach: head_dim 64 and 32 in bf16,
    # attention without the causal mask, fp32 with GQA and RoPE. (ReLU is run
    # in fp32 only: in bf16 the pre-activation is recomputed from bf16-stored
    # values, and where it lies within rounding of 0 the ReLU derivative flips,
    # an O(1) difference per such element that no tolerance on rounding covers.)
    # Five query blocks (one FFN group here; the parity test at s = 20480
    # covers FFN groups of 2, 2 and 1 blocks).
    "gpt1b-small-5blocks": WORKLOADS["gpt1b-s8k"].replace(
        name="gpt1b-small-5blocks", seq_len=640, hidden=256, n_heads=2, n_kv_heads=2,
        ffn_dim=512, q_block=128, kv_block=320, head_chunk=2),
    # Hidden 4096: the norm backward shares each row among a workgroup's waves.
    "bf16-wide-rows": WORKLOADS["llama8b-s64k"].replace(
        name="bf16-wide-rows", seq_len=144, hidden=4096, n_heads=32, n_kv_heads=8,
        ffn_dim=512, q_block=48, kv_block=144, head_chunk=32),
    "bf16-d64-noncausal": WORKLOADS["gpt1b-s8k"].replace(
        name="bf16-d64-noncausal", seq_len=336, hidden=256, n_heads=4, n_kv_heads=4,
        head_dim=64, ffn_dim=512, causal=False, q_block=112, kv_block=168, head_chunk=4),
    "bf16-d64-gqa-rope": WORKLOADS["llama8b-s64k"].replace(
        name="bf16-d64-gqa-rope", seq_len=400, hidden=256, n_heads=4, n_kv_heads=2,
        head_dim=64, ffn_dim=768, q_block=200, kv_block=400, head_chunk=2),
    "bf16-d32": WORKLOADS["gpt1b-s8k"].replace(
        name="bf16-d32", seq_len=272, hidden=128, n_heads=4, n_kv_heads=4, head_dim=32,
        ffn_dim=512, q_block=136, kv_block=272, head_chunk=2),
    # Causal sliding windows (not multiples of the 64-key tiles): the DMA
    # kernels at head_dim 128 and at 64 with GQA (the query-head-split dK/dV
    # pass), the register kernels in bf16 (head_dim 32) and fp32.
    "bf16-d128-window": WORKLOADS["gpt1b-s8k"].replace(
        name="bf16-d128-window", seq_len=1040, hidden=256, n_heads=2, n_kv_heads=2,
        head_dim=128, ffn_dim=512, q_block=520, kv_block=1040, head_chunk=2, window=200),
    "bf16-d64-gqa-rope-window": WORKLOADS["llama8b-s64k"].replace(
        name="bf16-d64-gqa-rope-window", seq_len=1040, hidden=256, n_heads=4, n_kv_heads=2,
        head_dim=64, ffn_dim=768, q_block=520, kv_block=1040, head_chunk=2, window=100),
    "bf16-d32-window": WORKLOADS["gpt1b-s8k"].replace(
        name="bf16-d32-window", seq_len=528, hidden=128, n_heads=4, n_kv_heads=4, head_dim=32,
        ffn_dim=512, q_block=264, kv_block=528, head_chunk=2, window=33),
    "f32-d64-window": WORKLOADS["gpt-tiny-fp32"].replace(
        name="f32-d64-window", seq_len=400, hidden=128, n_heads=2, n_kv_heads=2, head_dim=64,
        ffn_dim=256, q_block=200, kv_block=400, head_chunk=2, window=77),
    # Attention dropout (masks regenerated in the backward): DMA kernels at
    # head_dim 128, and at 64 with GQA, RoPE, a window and the split dK/dV
    # pass; register kernels in bf16 (head_dim 32) and fp32.
    "bf16-d128-dropout": WORKLOADS["gpt1b-s8k"].replace(
        name="bf16-d128-dropout", seq_len=1040, hidden=256, n_heads=2, n_kv_heads=2,
        head_dim=128, ffn_dim=512, q_block=520, kv_block=1040, head_chunk=2, dropout_p=0.1,
        seed=7),
    "bf16-d64-gqa-rope-window-dropout": WORKLOADS["llama8b-s64k"].replace(
        name="bf16-d64-gqa-rope-window-dropout", seq_len=1040, hidden=256, n_heads=4,
        n_kv_heads=2, head_dim=64, ffn_dim=768, q_block=520, kv_block=1040, head_chunk=2,
        window=300, dropout_p=0.2, seed=(1 << 40) + 11),
    "bf16-d32-dropout": WORKLOADS["gpt1b-s8k"].replace(
        name="bf16-d32-dropout", seq_len=528, hidden=128, n_heads=4, n_kv_heads=4, head_dim=32,
        ffn_dim=512, q_block=264, kv_block=528, head_chunk=2, dropout_p=0.25, seed=3),
    "f32-d64-dropout": WORKLOADS["gpt-tiny-fp32"].replace(
        name="f32-d64-dropout", seq_len=400, hidden=128, n_heads=2, n_kv_heads=2, head_dim=64,
        ffn_dim=256, q_block=200, kv_block=400, head_chunk=2, dropout_p=0.3, seed=5),
    "f32-d64-gqa-rope-noncausal": WORKLOADS["gpt-tiny-fp32"].replace(
        name="f32-d64-gqa-rope-noncausal", seq_len=240, hidden=256, n_heads=4, n_kv_heads=2,
        head_dim=64, ffn_dim=512, norm="rmsnorm", ffn="gelu", causal=False,
        rope_base=10000.0, q_block=120, kv_block=80, head_chunk=2),
    # Hidden, FFN and Q/K/V widths that are not multiples of the GEMM column
    # tile (320, 1344 and 960 / 448 columns): a partial column tile in every
    # projection, with the GeLU and the SwiGLU epilogues.
    "bf16-ragged-cols": WORKLOADS["gpt1b-s8k"].replace(
        name="bf16-ragged-cols", seq_len=400, hidden=320, n_heads=5, n_kv_heads=5,
        head_dim=64, ffn_dim=1344, q_block=200, kv_block=400, head_chunk=5),
    "bf16-ragged-cols-swiglu": WORKLOADS["llama8b-s64k"].replace(
        name="bf16-ragged-cols-swiglu", seq_len=400, hidden=320, n_heads=5, n_kv_heads=1,
        head_dim=64, ffn_dim=1344, q_block=200, kv_block=400, head_chunk=5),
}


def _normal(seed: int, shape, std: float) -> np.ndarray:
    rng = np.random.default_rng(seed)
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


class Tensor:
    """A generated tensor: float32 values already rounded to the storage dtype,
    plus the raw storage (bf16 bits or float32) to copy to a device."""

    def __init__(self, values_f32: np.ndarray, storage: np.ndarray, dtype: str):
        self.f32 = values_f32
        self.storage = storage
        self.dtype = dtype

    @property
    def shape(self):
        return self.f32.shape

    def f64(self) -> np.ndarray:
        return self.f32.astype(np.float64)


def _make(values: np.ndarray, dtype: str) -> Tensor:
    if dtype == "bf16":
        bits = round_to_bf16_bits(values)
        return Tensor(bf16_bits_to_f32(bits), bits, dtype)
    v = np.ascontiguousarray(values, dtype=np.float32)
    return Tensor(v, v, dtype)


def weight_shapes(sh: LayerShape) -> Dict[str, tuple]:
    h, f, hd = sh.hidden, sh.ffn_dim, sh.n_heads * sh.head_dim
    shapes = {"w_qkv": (h, sh.qkv_cols), "w_o": (hd, h), "w_1": (h, f), "w_2": (f, h),
              "n1_g": (h,), "n2_g": (h,)}
    if sh.ffn == "swiglu":
        shapes["w_3"] = (h, f)
    if sh.norm == "layernorm":
        shapes["n1_b"] = (h,)
        shapes["n2_b"] = (h,)
    if sh.has_bias:
        shapes.update({"b_qkv": (sh.qkv_cols,), "b_o": (h,), "b_1": (f,), "b_2": (h,)})
    return shapes


def fan_in(name: str, sh: LayerShape) -> int:
    return {"w_qkv": sh.hidden, "w_o": sh.n_heads * sh.head_dim, "w_1": sh.hidden,
            "w_3": sh.hidden, "w_2": sh.ffn_dim}[name]


def make_weights(sh: LayerShape, bias_std: float = 0.0, norm_std: float = 0.0) -> Dict[str, Tensor]:
    """Weights per the recipe. ``bias_std``/``norm_std`` > 0 perturb biases and
    norm parameters away from 0/1 (used by tests so every term is exercised)."""
    out = {}
    for name, shape in weight_shapes(sh).items():
        seed = 1000 * sh.wid + TENSOR_IDS[name]
        if name.startswith("w_"):
            vals = _normal(seed, shape, float(fan_in(name, sh)) ** -0.5)
        elif name in ("n1_g", "n2_g"):
            vals = np.ones(shape, np.float32)
            if norm_std:
                vals = vals + _normal(seed, shape, norm_std)
        else:
            vals = np.zeros(shape, np.float32)
            if bias_std:
                vals = _normal(seed, shape, bias_std)
        out[name] = _make(vals, sh.dtype)
    return out


def make_x(sh: LayerShape) -> Tensor:
    return _make(_normal(1000 * sh.wid + TENSOR_IDS["x"],
                         (sh.batch, sh.seq_len, sh.hidden), 1.0), sh.dtype)


def make_dy(sh: LayerShape, rows: Optional[np.ndarray] = None) -> Tensor:
    """Output cotangent ~ N(0,1). With ``rows`` given, only those sequence
    positions (of every batch element) are non-zero."""
    vals = _normal(1000 * sh.wid + TENSOR_IDS["dy"], (sh.batch, sh.seq_len, sh.hidden), 1.0)
    if rows is not None:
        mask = np.zeros(sh.seq_len, bool)
        mask[np.asarray(rows)] = True
        vals[:, ~mask, :] = 0.0
    return _make(vals, sh.dtype)


def sample_rows(sh: LayerShape, n_head: int = 8, n_tail: int = 8, n_mid: int = 8,
                seed: int = 7) -> np.ndarray:
    """Sequence positions sampled for full-size checks: the first rows, rows
    just before the end (longest causal key range; the very last row is left
    out so a causal layer's last position must receive exactly zero gradient)
    and random rows in between."""
    s = sh.seq_len
    rng = np.random.default_rng(1000 * sh.wid + seed)
    tail0 = max(n_head, s - 1 - n_tail)
    mid = rng.choice(np.arange(n_head, tail0), size=min(n_mid, max(0, tail0 - n_head)),
                     replace=False)
    rows = np.concatenate([np.arange(min(n_head, s)), mid, np.arange(tail0, s - 1)])
    return np.unique(rows)


def scaled(t: Tensor, factor: float, cols=slice(None)) -> Tensor:
    """A copy of ``t`` with the columns ``cols`` of its last axis multiplied by
    ``factor`` before rounding to the storage dtype (exact for a power of two).
    Used to build stress inputs, e.g. peaked attention scores from larger
    query projections."""
    vals = t.f32.copy()
    vals[..., cols] *= np.float32(factor)
    return _make(vals, t.dtype)



# ----------------------------------------------------------------- LM head with cross-entropy
@dataclasses.dataclass(frozen=True)
class LmHeadShape:
    """The output layer with cross-entropy over rows = batch x sequence
    positions. The vocabulary is padded to a multiple of 64 (the pages' worked
    example has V = 50257; 50304 = 64 x 786)."""
    name: str
    wid: int
    dtype: str
    rows: int
    hidden: int
    vocab: int
    chunk_rows: int
    ignore_every: int = 0      # every n-th row's target is -1 (ignored); 0: none

    def replace(self, **kw) -> "LmHeadShape":
        return dataclasses.replace(self, **kw)


LM_TENSOR_IDS = {"z": 20, "w_head": 21, "targets": 22, "dloss": 23}

LM_HEADS: Dict[str, LmHeadShape] = {
    # the GPT-1B-shaped model's head over the benchmarked s = 131072 tokens
    "lmhead-gpt1b-s128k": LmHeadShape("lmhead-gpt1b-s128k", 30, "bf16", 131072, 2048, 50304,
                                      8192),
    # reduced shapes: three chunks, the last one ragged, some ignored rows
    "lmhead-small-bf16": LmHeadShape("lmhead-small-bf16", 31, "bf16", 1000, 256, 1024, 384,
                                     ignore_every=7),
    "lmhead-small-f32": LmHeadShape("lmhead-small-f32", 32, "f32", 1000, 256, 1024, 384,
                                    ignore_every=7),
}


def make_z(sh: LmHeadShape) -> Tensor:
    """Final hidden states ~ N(0, 1) (the normalised input of the head)."""
    return _make(_normal(1000 * sh.wid + LM_TENSOR_IDS["z"], (sh.rows, sh.hidden), 1.0), sh.dtype)


def make_w_head(sh: LmHeadShape) -> Tensor:
    """[hidden, vocab] ~ N(0, 1/hidden)."""
    return _make(_normal(1000 * sh.wid + LM_TENSOR_IDS["w_head"], (sh.hidden, sh.vocab),
                         sh.hidden ** -0.5), sh.dtype)


def make_targets(sh: LmHeadShape) -> np.ndarray:
    """int32 targets uniform in [0, vocab); every ignore_every-th row -1."""
    rng = np.random.default_rng(1000 * sh.wid + LM_TENSOR_IDS["targets"])
    t = rng.integers(0, sh.vocab, size=sh.rows).astype(np.int32)
    if sh.ignore_every:
        t[::sh.ignore_every] = -1
    return t


def make_dloss(sh: LmHeadShape, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 cotangent of the per-row losses ~ N(0, 1); with ``rows`` only
    those rows are non-zero."""
    g = _normal(1000 * sh.wid + LM_TENSOR_IDS["dloss"], (sh.rows,), 1.0)
    if rows is not None:
        mask = np.zeros(sh.rows, bool)
        mask[np.asarray(rows)] = True
        g[~mask] = 0.0
    return g


def make_stack_weights(sh: LayerShape, n_layers: int, bias_std: float = 0.0,
                       norm_std: float = 0.0):
    """One weight set per layer of a stack; layer l draws from seed family
    wid + 1000 (l + 1)."""
    return [make_weights(sh.replace(wid=sh.wid + 1000 * (li + 1)), bias_std, norm_std)
            for li in range(n_layers)]
