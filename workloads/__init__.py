"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws random tensors and nothing else: it holds none of the
method's arithmetic (no matmul, no activation, no slicing into shards).
Both the fp64 oracle and the HIP path receive exactly the tensors made here,
so the two sides never exchange values with each other.

Recipe (the same for every workload):
  * a ``torch.Generator('cpu')`` seeded per workload and per tensor;
  * ``torch.randn`` in float32, scaled by the stated standard deviation;
  * for bf16 workloads, rounded to bfloat16 by torch (round-to-nearest-even).
The oracle upcasts the *rounded* values to float64, so the comparison
measures only the GPU's arithmetic, not the input rounding.

Distributions follow the workloads the pages describe: activations ~N(0, 1),
weights ~N(0, 0.02^2) (std 0.02, the usual initialisation scale).  Weights are
stored (in, out) row-major, as the feed-forward description writes W1 of
shape (d, 4d) and W2 of shape (4d, d).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import torch

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class MlpWorkload:
    """A per-rank MLP shard workload (one rank's columns of W1/W_up, rows of W2)."""
    name: str
    T: int            # tokens in the micro-batch
    d: int            # hidden size
    ff: int           # unsharded intermediate size
    p: int            # tensor-parallel width
    act: str          # "relu" | "gelu" | "swiglu"
    dtype: str        # "bf16" | "f32"
    seed: int

    @property
    def ff_i(self) -> int:
        return self.ff // self.p


@dataclasses.dataclass(frozen=True)
class GqaWorkload:
    """Per-rank grouped-query-attention projections (fused local QKV, o_proj)."""
    name: str
    T: int
    h: int
    n_q: int
    n_kv: int
    head_dim: int
    p: int
    seed: int


# The five workloads.  Sizes: tiny fp32 check; 70B-class SwiGLU MLP shard at
# decode (T=64) and prefill (T=4096) for p=8; GQA projections of a 70B-class
# model (h=8192, 64 Q heads, 8 KV heads, head_dim 128, p=8); SwiGLU backward
# with d=4096, d_ff=14336, p=8, T=2048.
TINY = MlpWorkload("tiny_fp32_relu_p4", T=4, d=64, ff=256, p=4, act="relu", dtype="f32", seed=0)
DECODE = MlpWorkload("swiglu_mlp_decode_T64", T=64, d=8192, ff=28672, p=8, act="swiglu",
                     dtype="bf16", seed=1)
PREFILL = MlpWorkload("swiglu_mlp_prefill_T4096", T=4096, d=8192, ff=28672, p=8,
                      act="swiglu", dtype="bf16", seed=2)
GQA_PREFILL = GqaWorkload("gqa_proj_T4096", T=4096, h=8192, n_q=64, n_kv=8, head_dim=128, p=8, seed=3)
GQA_DECODE = GqaWorkload("gqa_proj_T64", T=64, h=8192, n_q=64, n_kv=8, head_dim=128, p=8, seed=3)
GQA_ATTN = GqaWorkload("gqa_attention_T4096", T=4096, h=8192, n_q=64, n_kv=8, head_dim=128, p=8, seed=6)
GQA_BWD = GqaWorkload("gqa_proj_bwd_T4096", T=4096, h=8192, n_q=64, n_kv=8, head_dim=128, p=8, seed=5)
BACKWARD = MlpWorkload("swiglu_mlp_bwd_T2048", T=2048, d=4096, ff=14336, p=8, act="swiglu",
                       dtype="bf16", seed=4)

ALL = {w.name: w for w in (TINY, DECODE, PREFILL, GQA_PREFILL, GQA_DECODE, GQA_ATTN, GQA_BWD, BACKWARD)}


def _gen(seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    # one independent stream per (workload seed, tensor id)
    g.manual_seed(seed * 1_000_003 + stream)
    return g


def normal(shape, std: float, seed: int, stream: int, dtype: str = "bf16") -> torch.Tensor:
    """fp32 N(0, std^2) draw, rounded to bf16 (RNE) unless dtype == 'f32'."""
    t = torch.randn(*shape, generator=_gen(seed, stream), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(f"unknown dtype {dtype}")


# Tensor stream ids (fixed so every consumer draws the same values).
S_X, S_W1, S_WUP, S_W2, S_DY = 1, 2, 3, 4, 5
S_WQ, S_WK, S_WV, S_WO, S_ATTN = 11, 12, 13, 14, 15
S_DQ, S_DK, S_DV = 16, 17, 18
S_QKV = 19


def mlp_unsharded(w: MlpWorkload, with_dy: bool = False, T: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Unsharded x, W1 (d, ff), [W_up (d, ff)], W2 (ff, d) and optionally dy (T, d)."""
    T = w.T if T is None else T
    out = {
        "x": normal((T, w.d), 1.0, w.seed, S_X, w.dtype),
        "w1": normal((w.d, w.ff), WEIGHT_STD, w.seed, S_W1, w.dtype),
        "w2": normal((w.ff, w.d), WEIGHT_STD, w.seed, S_W2, w.dtype),
    }
    if w.act == "swiglu":
        out["w_up"] = normal((w.d, w.ff), WEIGHT_STD, w.seed, S_WUP, w.dtype)
    if with_dy:
        out["dy"] = normal((T, w.d), 1.0, w.seed, S_DY, w.dtype)
    return out


def mlp_rank_weights(w: MlpWorkload, rank: int, weight_seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """One rank's weights drawn directly at shard shape.

    For the 70B-class shards the unsharded matrices would be 8192 x 28672; the
    entries are i.i.d., so drawing rank ``rank``'s block directly has the same
    distribution as slicing it out of an unsharded draw.  Decode and prefill
    share these weights (``weight_seed`` defaults to the decode seed)."""
    s = (DECODE.seed if weight_seed is None else weight_seed) * 64 + rank
    out = {
        "w1": normal((w.d, w.ff_i), WEIGHT_STD, s, S_W1, w.dtype),
        "w2": normal((w.ff_i, w.d), WEIGHT_STD, s, S_W2, w.dtype),
    }
    if w.act == "swiglu":
        out["w_up"] = normal((w.d, w.ff_i), WEIGHT_STD, s, S_WUP, w.dtype)
    return out


def mlp_input(w: MlpWorkload, T: Optional[int] = None) -> torch.Tensor:
    T = w.T if T is None else T
    return normal((T, w.d), 1.0, w.seed, S_X, w.dtype)


def gqa_unsharded(w: GqaWorkload) -> Dict[str, torch.Tensor]:
    """Unsharded Wq (h, n_q*hd), Wk, Wv (h, n_kv*hd), Wo (n_q*hd, h), x (T, h) and
    the p ranks' attention outputs attn (T, n_q*hd) (rank i owns a 1024-wide slice)."""
    qw = w.n_q * w.head_dim
    kvw = w.n_kv * w.head_dim
    return {
        "x": normal((w.T, w.h), 1.0, w.seed + w.T, S_X),
        "wq": normal((w.h, qw), WEIGHT_STD, w.seed, S_WQ),
        "wk": normal((w.h, kvw), WEIGHT_STD, w.seed, S_WK),
        "wv": normal((w.h, kvw), WEIGHT_STD, w.seed, S_WV),
        "wo": normal((qw, w.h), WEIGHT_STD, w.seed, S_WO),
        "attn": normal((w.T, qw), 1.0, w.seed + w.T, S_ATTN),
    }


def gqa_grads(w: GqaWorkload, T: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Gradients arriving at the projections' outputs: unsharded dQ (T, n_q*hd),
    dK, dV (T, n_kv*hd) and the o_proj output gradient dy (T, h)."""
    T = w.T if T is None else T
    qw = w.n_q * w.head_dim
    kvw = w.n_kv * w.head_dim
    return {
        "dq": normal((T, qw), 1.0, w.seed, S_DQ),
        "dk": normal((T, kvw), 1.0, w.seed, S_DK),
        "dv": normal((T, kvw), 1.0, w.seed, S_DV),
        "dy": normal((T, w.h), 1.0, w.seed, S_DY),
    }


def attention_qkv(w: GqaWorkload, T: Optional[int] = None) -> torch.Tensor:
    """One rank's fused projection output (T, (n_q/p + 2 n_kv/p) * head_dim):
    rows [Q heads | K heads | V heads].  Drawn directly with the spread a
    projection of N(0, 1) activations through N(0, 0.02^2) weights has
    (std 0.02 * sqrt(h)), so the scaled scores have a realistic spread."""
    T = w.T if T is None else T
    width = (w.n_q // w.p + 2 * (w.n_kv // w.p)) * w.head_dim
    return normal((T, width), WEIGHT_STD * w.h ** 0.5, w.seed, S_QKV)


def e4m3_codes(shape, seed: int, stream: int) -> torch.Tensor:
    """fp8 weight codes (uint8, OCP E4M3): an N(0, 64^2) fp32 draw rounded to
    the nearest e4m3 value by torch (saturating at +-448), so the codes span
    normal and subnormal values of both signs."""
    t = torch.randn(*shape, generator=_gen(seed, stream), dtype=torch.float32).mul_(64.0)
    return t.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def column_scales(n: int, seed: int, stream: int) -> torch.Tensor:
    """Per-column fp32 weight scales, uniform in [0.5, 1.5) * 0.02 / 64, so the
    scaled weights have about the spread of the bf16 workloads' weights."""
    u = torch.rand(n, generator=_gen(seed, stream), dtype=torch.float32)
    return (0.5 + u) * (WEIGHT_STD / 64.0)


@dataclasses.dataclass(frozen=True)
class MoeWorkload:
    """One rank's slice of an MoE block with experts sharded in place."""
    name: str
    T: int
    d: int
    ff: int        # one expert's intermediate size (unsharded)
    E: int
    k: int
    p: int
    seed: int

    @property
    def ff_i(self) -> int:
        return self.ff // self.p


# A Qwen3-MoE-class layer (hidden 2048, 128 routed experts, top-8, expert
# intermediate 768) on p = 8 ranks, at prefill length.
MOE_PREFILL = MoeWorkload("moe_qwen3_class_T4096", T=4096, d=2048, ff=768, E=128, k=8, p=8, seed=8)
S_ROUTER, S_MW1, S_MWUP, S_MW2 = 30, 31, 32, 33


def moe_rank_inputs(w: MoeWorkload, T: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """x (T, d), router logits (T, E) fp32 drawn directly (N(0, 1): the spread of
    a router projection), and rank weights w1, w_up (E, d, ff_i), w2 (E, ff_i, d)."""
    T = w.T if T is None else T
    return {
        "x": normal((T, w.d), 1.0, w.seed, S_X),
        "logits": normal((T, w.E), 1.0, w.seed, S_ROUTER, "f32"),
        "w1": normal((w.E, w.d, w.ff_i), WEIGHT_STD, w.seed, S_MW1),
        "w_up": normal((w.E, w.d, w.ff_i), WEIGHT_STD, w.seed, S_MWUP),
        "w2": normal((w.E, w.ff_i, w.d), WEIGHT_STD, w.seed, S_MW2),
    }


def row_subset(T: int, n: int, seed: int) -> List[int]:
    """Seeded, sorted subset of ``n`` distinct rows out of ``T`` (all rows if T <= n)."""
    if T <= n:
        return list(range(T))
    g = _gen(seed, 99)
    return sorted(torch.randperm(T, generator=g)[:n].tolist())
