"""Seeded synthetic workloads shared by the oracle checks, the GPU tests and the benchmark.

This module draws random inputs and names shapes; it holds none of the attention
arithmetic.  Every tensor is ``numpy.random.default_rng(seed).standard_normal``
in float32, drawn in the order Q, K, V, dO with shape ``[B, H, N, d]`` (C order),
then rounded on the CPU to the working dtype by torch (round to nearest even).
The GPU receives exactly those rounded bytes and the oracle upcasts the same
rounded values to float64, so both sides see identical inputs.

Shapes follow the pages' own examples: the SDPA example shape (B=2, H=8, N=1024,
d=64) of "Flash Attention 3.7 核心原理与实战" §3.2, the memory example
(B=32, H=16, N=2048, d=64) of "告别OOM和训练慢…（含A100环境配置）" §1, and the
long-sequence / causal training settings those pages discuss.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str               # "f16" | "bf16" | "f32" (f32: source values, cast per test)
    causal: bool
    window: tuple            # (left, right); -1 means unbounded
    seed: int
    backward: bool = False
    scale: float = field(default=float("nan"))
    padded: bool = False     # a padded batch: per-sample lengths from draw_seqlens
    packed: bool = False     # (with padded) the same sequences packed: [H, total, d], offsets

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d) if math.isnan(self.scale) else self.scale

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


# The five workloads.  Seeds are fixed once and never tuned after seeing results.
TINY = Workload("tiny_b1h2n128d64", 1, 2, 128, 64, "f32", False, (-1, -1), seed=1)
BERT = Workload("sdpa_b2h8n1024d64_f16", 2, 8, 1024, 64, "f16", False, (-1, -1), seed=2)
CAUSAL = Workload("causal_b32h16n2048d64_bf16", 32, 16, 2048, 64, "bf16", True, (-1, -1), seed=3)
LONG_4K = Workload("window_b2h8n4096d128_bf16", 2, 8, 4096, 128, "bf16", True, (1024, 0), seed=41)
LONG_8K = Workload("window_b2h8n8192d128_bf16", 2, 8, 8192, 128, "bf16", True, (1024, 0), seed=42)
TRAIN = Workload("train_b8h16n4096d64_bf16", 8, 16, 4096, 64, "bf16", True, (-1, -1), seed=5,
                 backward=True)

ALL = (TINY, BERT, CAUSAL, LONG_4K, LONG_8K, TRAIN)

# Plain causal forward at head dim 128 and N >= 4096 (the long-sequence head dim without the
# window): the training heads at N = 4096, and half the batch at N = 8192.
CAUSAL_128_4K = Workload("causal_b8h16n4096d128_bf16", 8, 16, 4096, 128, "bf16", True, (-1, -1),
                         seed=43)
CAUSAL_128_8K = Workload("causal_b4h16n8192d128_bf16", 4, 16, 8192, 128, "bf16", True, (-1, -1),
                         seed=44)
LONG_128 = (CAUSAL_128_4K, CAUSAL_128_8K)


@dataclass(frozen=True)
class DecodeWorkload:
    """A decode step: n_q new queries per (batch, head) over a KV cache of n_k keys (the
    queries are the last n_q positions), causal."""
    name: str
    B: int
    H: int
    n_q: int
    n_k: int
    d: int
    dtype: str
    seed: int

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The training workload's head shape (B=8, H=16, d=64) and the long-sequence head dim
# (d=128), one new query over a 16384-key cache.
DECODE_64 = DecodeWorkload("decode_b8h16q1k16384d64_bf16", 8, 16, 1, 16384, 64, "bf16", seed=7)
DECODE_128 = DecodeWorkload("decode_b8h16q1k16384d128_bf16", 8, 16, 1, 16384, 128, "bf16", seed=8)
DECODES = (DECODE_64, DECODE_128)


@dataclass(frozen=True)
class BlockWorkload:
    """A training step of a block of n_q new queries over n_k keys (the block being the last
    n_q positions: a cache of n_k - n_q keys plus the block itself), causal, forward and
    backward through fa_fwd_kv / fa_bwd_kv."""
    name: str
    B: int
    H: int
    n_q: int
    n_k: int
    d: int
    dtype: str
    seed: int

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass(frozen=True)
class Fp8Workload:
    """A forward over FP8 E4M3 queries, keys and values: codes of N(0, 1) * 16 with descale
    1/16 per tensor (``fp8_attention_case``), output in ``out_dtype``."""
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    window: tuple
    seed: int
    out_dtype: str = "bf16"

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)


# the causal forward shapes at head dims 64 and 128, with FP8 operands
FP8_64 = Fp8Workload("fp8_causal_b8h16n4096d64", 8, 16, 4096, 64, True, (-1, -1), seed=51)
FP8_128 = Fp8Workload("fp8_causal_b8h16n4096d128", 8, 16, 4096, 128, True, (-1, -1), seed=52)
FP8S = (FP8_64, FP8_128)


# the training workload's heads, a 1024-query block over 4096 keys
BLOCK = BlockWorkload("block_b8h16q1024k4096d64_bf16", 8, 16, 1024, 4096, 64, "bf16", seed=9)
# The training step over a padded batch: sample lengths drawn by draw_seqlens (the pages fix
# no length mix; uniform over [N/4, N] is a plain stand-in for a batch of mixed lengths).
VARLEN = Workload("varlen_b8h16n4096d64_bf16", 8, 16, 4096, 64, "bf16", True, (-1, -1), seed=6,
                  backward=True, padded=True)
# The same training step over the same sequences packed per head ([H, total, d], offsets).
PACKED = Workload("packed_b8h16n4096d64_bf16", 8, 16, 4096, 64, "bf16", True, (-1, -1), seed=6,
                  backward=True, padded=True, packed=True)
BY_NAME = {w.name: w for w in ALL + LONG_128 + (VARLEN, PACKED) + DECODES + (BLOCK,) + FP8S}


def draw_f32(shape, seed: int, count: int):
    """``count`` standard-normal float32 arrays of ``shape`` from one seeded stream."""
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape, dtype=np.float32) for _ in range(count)]


def round_to(x_f32: np.ndarray, dtype: str):
    """Round float32 values to ``dtype`` on the CPU with torch (RNE).

    Returns ``(torch_cpu_tensor_in_dtype, float64_numpy_of_the_rounded_values)``.
    """
    import torch

    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    t = torch.from_numpy(np.ascontiguousarray(x_f32)).to(tdt)
    return t, t.to(torch.float64).numpy()


def make_inputs(w: Workload, dtype: str | None = None, shape=None, seed=None, with_grad=None):
    """Seeded inputs for workload ``w``.

    Returns a dict with torch CPU tensors ``q, k, v`` (and ``do`` when the workload
    has a backward pass) in the working dtype, and their float64 numpy copies
    ``q64, k64, v64 (, do64)`` holding exactly the rounded values.
    """
    dtype = dtype or w.dtype
    shape = tuple(shape or w.shape)
    seed = w.seed if seed is None else seed
    with_grad = w.backward if with_grad is None else with_grad
    names = ["q", "k", "v"] + (["do"] if with_grad else [])
    out = {}
    for name, arr in zip(names, draw_f32(shape, seed, len(names))):
        t, a64 = round_to(arr, dtype)
        out[name] = t
        out[name + "64"] = a64
    return out


def draw_seqlens(B: int, N: int, seed: int):
    """B sample lengths, uniform integers in [N/4, N], from their own seeded stream (the
    seed's Q, K, V, dO stream is untouched): ``int32`` numpy array."""
    rng = np.random.default_rng([seed, 1])
    return rng.integers(N // 4, N, size=B, endpoint=True).astype(np.int32)


def cross_case(B: int, H: int, n_q: int, n_k: int, d: int, dtype: str, seed: int):
    """Seeded N(0, 1) inputs with N_q query rows and N_k key rows: q [B, H, n_q, d], then k and
    v [B, H, n_k, d], drawn in that order from one stream and rounded like ``make_inputs``."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, rows in (("q", n_q), ("k", n_k), ("v", n_k)):
        t, a64 = round_to(rng.standard_normal((B, H, rows, d), dtype=np.float32), dtype)
        out[name] = t
        out[name + "64"] = a64
    return out


def key_padding_case(B: int, n_k: int, seed: int, density: float = 0.3, runs=()) -> np.ndarray:
    """A seeded key padding mask, bool [B, n_k] (True = padding key): each key padded with
    probability ``density`` (holes anywhere), plus the key ranges ``runs`` [(b, start, stop)]
    padded whole (whole key tiles, a whole batch entry)."""
    m = np.random.default_rng(seed).random((B, n_k)) < density
    for b, start, stop in runs:
        m[b, start:stop] = True
    return m


def fp8_cache_case(B: int, H: int, n_q: int, n_k: int, d: int, dtype: str, seed: int,
                   amax: float = 16.0):
    """Seeded decode inputs over an FP8 cache: q [B, H, n_q, d] N(0, 1) rounded like
    ``make_inputs``; k and v [B, H, n_k, d] as E4M3 codes (uint8) of N(0, 1) * amax, rounded to
    nearest by torch's float8_e4m3fn conversion, with descale 1 / amax (so the decoded keys and
    values are about N(0, 1)).  Any codes but the NaN ones are valid input; the rounding only
    picks them."""
    import torch
    rng = np.random.default_rng(seed)
    q, q64 = round_to(rng.standard_normal((B, H, n_q, d), dtype=np.float32), dtype)
    out = {"q": q, "q64": q64, "k_descale": 1.0 / amax, "v_descale": 1.0 / amax}
    for name in ("k", "v"):
        x = torch.from_numpy(rng.standard_normal((B, H, n_k, d), dtype=np.float32) * amax)
        out[name + "8"] = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out


def draw_blocks(H: int, n_q: int, n_k: int, density: float, seed: int):
    """A seeded block-sparse mask [H, ceil(n_q / 64), ceil(n_k / 64)] (bool) selecting each
    64 x 64 block with probability ``density``, from its own stream."""
    rng = np.random.default_rng([seed, 2])
    return rng.random((H, -(-n_q // 64), -(-n_k // 64))) < density


def random_case(shape, dtype: str, seed: int, with_grad: bool = False, scale_inputs: float = 1.0):
    """Seeded N(0, scale_inputs^2) inputs of an arbitrary shape (edge-case tests)."""
    names = ["q", "k", "v"] + (["do"] if with_grad else [])
    out = {}
    for name, arr in zip(names, draw_f32(tuple(shape), seed, len(names))):
        t, a64 = round_to(arr * np.float32(scale_inputs), dtype)
        out[name] = t
        out[name + "64"] = a64
    return out


def fp8_attention_case(shape, seed: int, amax: float = 16.0):
    """Seeded FP8 forward inputs: q, k, v [B, H, N, d] as E4M3 codes (uint8 numpy) of
    N(0, 1) * amax drawn in that order from one stream and rounded to nearest by torch's
    float8_e4m3fn conversion, with descale 1 / amax each (so the values are about N(0, 1))."""
    import torch
    rng = np.random.default_rng(seed)
    out = {"q_descale": 1.0 / amax, "k_descale": 1.0 / amax, "v_descale": 1.0 / amax}
    for name in ("q", "k", "v"):
        x = torch.from_numpy(rng.standard_normal(tuple(shape), dtype=np.float32) * np.float32(amax))
        out[name + "8"] = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out
