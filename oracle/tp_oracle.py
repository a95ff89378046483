"""Plain, slow, obviously-correct float64 oracle for one rank's tensor-parallel shard.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU product
path never calls it, imports nothing from it and shares no code with it.

Everything here is numpy float64 (``numpy.matmul`` is the only library
primitive used for the contraction).  Inputs that arrive as bf16/fp32 tensors
are upcast to float64 *after* the shared generator has rounded them, so the
oracle sees exactly the values the GPU sees.

Sources (the web pages this method is described on):
  [MLX]  "Tensor-parallel all-reduce count per transformer layer in MLX
         shard_linear" - Facts list (ShardedToAllLinear adds its bias once,
         after the sum).
  [KL]   "Tensor Parallelism" (inference-engineering notes) - first paragraph
         (column / row parallelism algebra), second paragraph (GQA per-rank
         bookkeeping), fifth paragraph (KV heads bound the TP width).
  [KS]   "Why Tensor Parallelism has to stay inside the scale-up domain" -
         "What is Tensor Parallel" (h=2, d_ff=3 worked example),
         "Where the 320 comes from" (sequence parallelism: reduce-scatter
         + all-gather in place of each all-reduce),
         "What happens if TP leaves the node" (6 x params x tokens).
  [FFN]  "How does tensor parallelism split a transformer feed-forward block's
         two matmuls across devices?" - "The shape of the block",
         "Column split, then row split" (First matmul, column-parallel /
         The nonlinearity is free / Second matmul, row-parallel /
         One collective), "The backward pass", "Common failure".

Readings where the pages are silent (also listed with the design notes):
  * SwiGLU is silu(x W_gate) * (x W_up) with gate and up over the SAME owned
    column range ([FFN] "The nonlinearity is free" allows "a gated variant
    computed from the same slice"); silu(g) = g * sigmoid(g).
  * GELU is the exact erf form 0.5 x (1 + erf(x / sqrt 2)); no tanh variant.
  * ReLU'(0) = 0.
  * Equal contiguous chunks only; an intermediate size not divisible by p is
    rejected ([FFN] partitions 4d into N chunks of size 4d/N).
  * Column-parallel bias: each shard adds its own slice; row-parallel bias:
    added once after the sum ([MLX]).
  * The backward of the attention projections is the backward of two
    linear shards: QKV column-parallel (partial dx), o_proj row-parallel
    (replicated dy, local dx); no bias gradients.
  * MoE routing: softmax over the router logits, top-k (ties to the lower
    index), the k probabilities renormalised; experts sharded in place.
  * Local attention is scaled dot-product softmax attention, optionally
    causal, with query head j reading KV head j // (n_q / n_kv).
  * The "quantized equivalent" of a sharded linear is read as fp8 weights:
    OCP E4M3 codes with one fp32 scale per output column, bf16 activations.
  * The normalization after the block's sum is RMSNorm with a learned scale
    and a caller-given epsilon, taken over the fp32/float64 sum.

Every function below has a pin in ``tests/test_oracle_pins.py`` that checks it
against something other than itself (the pages' worked example, exact rational
brute force, algebraic invariants, finite differences, library special values).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64
ACTS = ("none", "relu", "gelu", "swiglu")


def to64(a) -> np.ndarray:
    """Upcast a torch tensor (any float dtype) or array to a float64 ndarray."""
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").float().numpy()
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------------------
# Shard ownership.  [FFN] "Column split, then row split": the intermediate
# dimension is cut into N equal chunks; device i owns columns i*n/N .. (i+1)*n/N
# of the first matrix and exactly the matching rows of the second.
# ---------------------------------------------------------------------------
def shard_range(n_total: int, p: int, i: int) -> Tuple[int, int]:
    """(begin, length) of shard ``i`` when ``n_total`` is cut into ``p`` equal chunks."""
    if p <= 0 or not (0 <= i < p) or n_total < 0:
        raise ValueError("bad shard request")
    if n_total % p != 0:
        raise ValueError(f"{n_total} is not divisible by p={p}")
    length = n_total // p
    return i * length, length


def gqa_shard(n_q: int, n_kv: int, head_dim: int, p: int, i: int) -> Tuple[int, int, int, int]:
    """Column ranges of rank ``i``'s query heads and KV heads.

    [KL] second paragraph: with 64 Q heads, 8 KV heads, head dim 128 and p=8,
    each rank owns 8 Q heads and 1 KV head, i.e. a 1024-wide Q slice and a
    128-wide K and V slice.  [FFN] attention paragraph: heads are never split,
    so both head counts must divide by p ([KL] fifth paragraph: 8 KV heads map
    cleanly only for p <= 8).  Heads are taken contiguously, so Q head j groups
    with KV head floor(j / (n_q / n_kv)) and both land on the same rank.
    Returns (q_begin, q_len, kv_begin, kv_len) in columns."""
    if n_q % p != 0 or n_kv % p != 0:
        raise ValueError("head counts must be divisible by p (a head is never split)")
    qh_b, qh_n = shard_range(n_q, p, i)
    kh_b, kh_n = shard_range(n_kv, p, i)
    return qh_b * head_dim, qh_n * head_dim, kh_b * head_dim, kh_n * head_dim


def slice_cols(w: np.ndarray, begin: int, length: int) -> np.ndarray:
    return np.ascontiguousarray(w[:, begin:begin + length])


def slice_rows(w: np.ndarray, begin: int, length: int) -> np.ndarray:
    return np.ascontiguousarray(w[begin:begin + length, :])


# ---------------------------------------------------------------------------
# Activations.  [FFN] "The nonlinearity is free": GELU, ReLU or a gated
# variant, applied elementwise to the owned columns.
# ---------------------------------------------------------------------------
def sigmoid(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=F64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def relu(a: np.ndarray) -> np.ndarray:
    return np.where(a > 0, a, 0.0)


def relu_grad(a: np.ndarray) -> np.ndarray:
    return np.where(a > 0, 1.0, 0.0)


_erf = np.vectorize(math.erf, otypes=[F64])


def gelu(a: np.ndarray) -> np.ndarray:
    """Exact GELU: a * Phi(a) with Phi the standard normal CDF, via erf."""
    a = np.asarray(a, dtype=F64)
    return 0.5 * a * (1.0 + _erf(a / math.sqrt(2.0)))


def gelu_grad(a: np.ndarray) -> np.ndarray:
    """d/da [a Phi(a)] = Phi(a) + a phi(a)."""
    a = np.asarray(a, dtype=F64)
    cdf = 0.5 * (1.0 + _erf(a / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * a * a) / math.sqrt(2.0 * math.pi)
    return cdf + a * pdf


def silu(g: np.ndarray) -> np.ndarray:
    return np.asarray(g, dtype=F64) * sigmoid(g)


def silu_grad(g: np.ndarray) -> np.ndarray:
    """d/dg [g s(g)] = s(g) + g s(g) (1 - s(g))."""
    s = sigmoid(g)
    return s + np.asarray(g, dtype=F64) * s * (1.0 - s)


def act_apply(a: np.ndarray, act: str, up: Optional[np.ndarray] = None) -> np.ndarray:
    if act == "none":
        return np.asarray(a, dtype=F64)
    if act == "relu":
        return relu(a)
    if act == "gelu":
        return gelu(a)
    if act == "swiglu":
        if up is None:
            raise ValueError("swiglu needs the up projection")
        return silu(a) * up
    raise ValueError(f"unknown act {act}")


# ---------------------------------------------------------------------------
# Linear layers.  [KL] first paragraph: Y = XW; column parallelism splits W
# along its output dimension so device i computes Y_i = X W_i; row
# parallelism splits W along its input dimension and X to match, so device i
# computes the full-shape partial Z_i = X_i W_i and Y = sum_i Z_i.
# ---------------------------------------------------------------------------
def matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.matmul(to64(a), to64(b))


def col_linear(x, w, w_up=None, bias=None, act: str = "none") -> np.ndarray:
    """act(x W_i [+ b_i]); for swiglu: silu(x W_i) * (x W_up_i) (no bias).

    [KL] first paragraph (Y_i = X W_i) and [FFN] "First matmul,
    column-parallel" / "The nonlinearity is free" (act on owned columns)."""
    a = matmul(x, w)
    if act == "swiglu":
        if bias is not None:
            raise ValueError("bias is not defined for the gated variant")
        return act_apply(a, act, matmul(x, w_up))
    if bias is not None:
        a = a + to64(bias)[None, :]
    return act_apply(a, act)


def row_linear_partial(x_i, w_i) -> np.ndarray:
    """Z_i = X_i W_i: the full output shape, but only a partial sum.

    [KL] first paragraph (row parallelism) and [FFN] "Second matmul,
    row-parallel"; no bias here ([MLX]: the bias is added after the sum)."""
    return matmul(x_i, w_i)


def e4m3_decode(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (the "quantized" weights): bit 7 sign,
    bits 6-3 exponent e with bias 7, bits 2-0 mantissa m.
        e = 0:       (-1)^s * m/8 * 2^(1-7)       (subnormal, m = 0 is zero)
        0 < e < 15:  (-1)^s * (1 + m/8) * 2^(e-7)
        e = 15:      as above, except m = 7 is NaN (no infinities; max 448)
    Written out from the format's definition (the pages only mention a
    "quantized equivalent" of the sharded linear)."""
    c = np.asarray(codes.cpu().numpy() if hasattr(codes, "cpu") else codes).astype(np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(F64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e.astype(F64) - 7.0))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


def dequant_e4m3(codes, scale) -> np.ndarray:
    """W[k, n] = e4m3(codes[k, n]) * scale[n] (one scale per output column)."""
    return e4m3_decode(codes) * to64(scale)[None, :]


def col_linear_fp8(x, wq, scale, wq_up=None, scale_up=None, bias=None, act: str = "none") -> np.ndarray:
    """The column-parallel linear of col_linear with fp8 weights."""
    w = dequant_e4m3(wq, scale)
    w_up = dequant_e4m3(wq_up, scale_up) if wq_up is not None else None
    return col_linear(x, w, w_up, bias, act)


def row_linear_partial_fp8(x_i, wq_i, scale_i) -> np.ndarray:
    """The row-parallel partial of row_linear_partial with fp8 weights."""
    return row_linear_partial(x_i, dequant_e4m3(wq_i, scale_i))


def partial_sum(zs: Sequence[np.ndarray], bias=None) -> np.ndarray:
    """Y = sum_i Z_i, then + bias once.

    [KL] first paragraph (Y = sum_i Z_i, done by an all-reduce);
    [FFN] "One collective"; [MLX] (ShardedToAllLinear adds the bias once,
    after the sum)."""
    y = np.zeros_like(to64(zs[0]))
    for z in zs:
        y = y + to64(z)
    if bias is not None:
        y = y + to64(bias)[None, :]
    return y


def rs_residual_rmsnorm(zs: Sequence[np.ndarray], rank: int, residual, norm_w, eps: float, bias=None):
    """One rank's share of the sequence-parallel block boundary.

    [KS] "Where the 320 comes from", sequence-parallel paragraph (with
    sequence parallelism every all-reduce is split into a reduce-scatter and
    an all-gather: after the reduce-scatter rank `rank` holds the sum over
    its T/p contiguous rows only) and [FFN] "One
    collective" (the summed output goes to the residual add and the
    following normalization).  The normalization is read as RMSNorm with a
    learned scale (the pages name a Llama-style block but not the norm):
    y = s / sqrt(mean(s^2) + eps) * norm_w, over the summed row s.
    Returns (s, y) for the rank's rows; the partials are summed in order,
    then the bias (once), then the residual is added."""
    p = len(zs)
    T = zs[0].shape[0]
    if T % p != 0:
        raise ValueError(f"{T} rows do not split into {p} equal shares")
    rows = T // p
    r0 = rank * rows
    part = [to64(z)[r0:r0 + rows] for z in zs]
    s = partial_sum(part, bias) + to64(residual)
    y = s / np.sqrt(np.mean(s * s, axis=1, keepdims=True) + eps) * to64(norm_w)[None, :]
    return s, y


# ---------------------------------------------------------------------------
# The feed-forward block.  [FFN] "The shape of the block": h = act(x W1),
# y = h W2; "Column split, then row split": h_i = act(x W1_i),
# y_i = h_i W2_i, y = sum_i y_i.
# ---------------------------------------------------------------------------
def mlp_full(x, w1, w_up, w2, act: str) -> np.ndarray:
    """Unsharded block: act(x W1 [, x W_up]) W2."""
    return matmul(col_linear(x, w1, w_up, None, act), w2)


def mlp_shard_fwd(x, w1_i, w_up_i, w2_i, act: str) -> Tuple[np.ndarray, Dict[str, np.ndarray]]:
    """One rank's forward: y_i = act(x W1_i [, x W_up_i]) W2_i.

    Returns (y_i, saved) with the pre-activations the backward needs:
    saved = {"g": x W1_i, "u": x W_up_i} for swiglu, {"a": x W1_i} otherwise."""
    a = matmul(x, w1_i)
    if act == "swiglu":
        u = matmul(x, w_up_i)
        h = silu(a) * u
        saved = {"g": a, "u": u}
    else:
        h = act_apply(a, act)
        saved = {"a": a}
    return matmul(h, w2_i), saved


def mlp_shard_bwd(x, w1_i, w_up_i, w2_i, dy, act: str,
                  saved: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """One rank's backward.

    [FFN] "The backward pass": the gradient arriving at y is identical on
    every device (the exit is an all-reduce forward, identity backward); each
    device forms the gradients of its own W1/W2 slices with no exchange and a
    partial gradient of x from its own column slice; those partials are summed
    before leaving the block.  Chain rule for h_i = act(x W1_i) and
    y_i = h_i W2_i:
        dW2_i = h_i^T dy,   dh_i = dy W2_i^T,
        dA = dh_i * act'(A)                        (relu / gelu)
        dG = dh_i * U * silu'(G), dU = dh_i * silu(G)   (swiglu)
        dW1_i = x^T dA (or x^T dG), dW_up_i = x^T dU,
        dx_i = dA W1_i^T  (or dG W1_i^T + dU W_up_i^T).
    The pre-activations are recomputed from x here unless given."""
    x = to64(x)
    dy = to64(dy)
    if saved is None:
        _, saved = mlp_shard_fwd(x, w1_i, w_up_i, w2_i, act)
    out: Dict[str, np.ndarray] = {}
    if act == "swiglu":
        g, u = saved["g"], saved["u"]
        h = silu(g) * u
        dh = matmul(dy, to64(w2_i).T)
        dg = dh * u * silu_grad(g)
        du = dh * silu(g)
        out["dw2"] = matmul(h.T, dy)
        out["dw1"] = matmul(x.T, dg)
        out["dw_up"] = matmul(x.T, du)
        out["dx"] = matmul(dg, to64(w1_i).T) + matmul(du, to64(w_up_i).T)
    else:
        a = saved["a"]
        h = act_apply(a, act)
        dh = matmul(dy, to64(w2_i).T)
        if act == "relu":
            da = dh * relu_grad(a)
        elif act == "gelu":
            da = dh * gelu_grad(a)
        elif act == "none":
            da = dh
        else:
            raise ValueError(act)
        out["dw2"] = matmul(h.T, dy)
        out["dw1"] = matmul(x.T, da)
        out["dx"] = matmul(da, to64(w1_i).T)
    return out


def mlp_full_bwd(x, w1, w_up, w2, dy, act: str) -> Dict[str, np.ndarray]:
    """Unsharded backward (the same chain rule with p = 1)."""
    return mlp_shard_bwd(x, w1, w_up, w2, dy, act)


def shard_mlp_weights(w1, w_up, w2, p: int, i: int):
    """Rank i's (W1_i, W_up_i, W2_i): columns of W1/W_up and the matching rows of W2."""
    w1 = to64(w1)
    w2 = to64(w2)
    b, n = shard_range(w1.shape[1], p, i)
    w1_i = slice_cols(w1, b, n)
    w_up_i = slice_cols(to64(w_up), b, n) if w_up is not None else None
    w2_i = slice_rows(w2, b, n)
    return w1_i, w_up_i, w2_i


# ---------------------------------------------------------------------------
# GQA projections.  [KL] second paragraph: rank i's fused QKV projection is
# the column slices [Q_i | K_i | V_i] of the unsharded projections; its
# o_proj consumes the rank's 1024-wide attention output and contributes a
# partial 8192-wide residual update that is then summed over ranks.
# ---------------------------------------------------------------------------
def gqa_local_qkv_weight(wq, wk, wv, n_q: int, n_kv: int, head_dim: int, p: int, i: int) -> np.ndarray:
    qb, ql, kb, kl = gqa_shard(n_q, n_kv, head_dim, p, i)
    return np.concatenate([slice_cols(to64(wq), qb, ql), slice_cols(to64(wk), kb, kl),
                           slice_cols(to64(wv), kb, kl)], axis=1)


def gqa_qkv_full(x, wq, wk, wv) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    return matmul(x, wq), matmul(x, wk), matmul(x, wv)


def linear_shard_bwd(x, w, dy) -> Dict[str, np.ndarray]:
    """Backward of one rank's shard of a linear layer y = x W.

    Chain rule for y = x W: dW = x^T dy, dx = dy W^T.  What the two outputs
    mean depends on how the layer is sharded ([FFN] "The backward pass";
    [KL] second paragraph for the attention projections):
      * column-parallel (the fused QKV projection): x is the replicated input,
        W = W_i its column slice and dy the rank's own output gradient; dW_i
        needs no exchange, dx_i is a partial that the group sums;
      * row-parallel (o_proj): x = X_i is the rank's own input slice and dy is
        identical on every rank (all-reduce forward, identity backward); dW_i
        and dX_i are both final, with no exchange."""
    x = to64(x)
    w = to64(w)
    dy = to64(dy)
    return {"dw": matmul(x.T, dy), "dx": matmul(dy, w.T)}


# ---------------------------------------------------------------------------
# Mixture-of-experts block with experts sharded in place.  [MLX] Facts: the
# MoE layers of DeepSeek V3 and Qwen3-MoE shard their routed experts in place
# (each rank keeps a slice of every expert), leave the router replicated and
# sum the block's output once.  The routing rule is not on the pages; it is
# read as softmax over the router logits, the top-k experts per token (ties to
# the lower index), with the k probabilities renormalised to sum to 1.
# ---------------------------------------------------------------------------
def moe_route(logits, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """(idx (T, k) int, gate (T, k)) from router logits (T, E): the k largest
    softmax probabilities per row in descending order (equal logits: lower
    expert index first), renormalised over the chosen k.  A NaN logit ranks
    as -inf (a NaN has no place in the order; treating it as the least
    likely expert keeps the ranking total), so it ties with -inf logits and
    those ties also go to the lower index."""
    lg = to64(logits)
    lg = np.where(np.isnan(lg), -np.inf, lg)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in 1..E")
    idx = np.zeros((T, k), dtype=np.int64)
    gate = np.zeros((T, k), dtype=F64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
        w = np.exp(lg[t, order] - lg[t, order[0]])
        idx[t] = order
        gate[t] = w / w.sum()
    return idx, gate


def moe_shard_fwd(x, idx, gate, w1, w_up, w2, act: str = "swiglu") -> np.ndarray:
    """One rank's partial of the MoE block: for each token t,
        y_i[t] = sum_j gate[t, j] * mlp_shard(x[t]; expert idx[t, j]'s slices)
    with w1, w_up (E, d, ff_i) and w2 (E, ff_i, d) the rank's slices of every
    expert (in-place sharding).  Summing y_i over ranks gives the block."""
    x = to64(x)
    idx = np.asarray(idx)
    gate = to64(gate)
    T, d = x.shape
    y = np.zeros((T, d), dtype=F64)
    for j in range(idx.shape[1]):
        for e in np.unique(idx[:, j]):
            rows = np.nonzero(idx[:, j] == e)[0]
            h = col_linear(x[rows], w1[e], None if w_up is None else w_up[e], None, act)
            y[rows] += gate[rows, j][:, None] * matmul(h, to64(w2[e]))
    return y


def gqa_attention(qkv, n_q: int, n_kv: int, head_dim: int, causal: bool, scale: float,
                  rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Attention over one rank's local heads, between the fused QKV projection
    and o_proj.

    [KL] second paragraph: with grouped-query attention each rank owns n_q
    query heads and n_kv KV heads and computes attention locally over them;
    [FFN] attention paragraph: heads are independent, so this needs no
    communication.  The pages do not write the attention itself; it is read
    as scaled dot-product softmax attention (the tiling of "QK softmax V" that
    [KL]'s FlashAttention paragraph refers to): for query head j, served by KV
    head j // (n_q / n_kv),
        S = scale * Q_j K^T,  S[t, u] = -inf for u > t when causal,
        P = softmax over u (each row), O_j = P V.
    qkv is (T, (n_q + 2 n_kv) * head_dim) with each row [Q heads | K heads |
    V heads]; the result is (T, n_q * head_dim), heads side by side (the
    layout o_proj consumes).  ``rows`` restricts the queries (each output row
    depends only on its own query), giving (len(rows), n_q * head_dim)."""
    a = to64(qkv)
    T = a.shape[0]
    if n_q % n_kv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    if a.shape[1] != (n_q + 2 * n_kv) * head_dim:
        raise ValueError("qkv width does not match the head counts")
    group = n_q // n_kv
    qrows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(qrows), n_q * head_dim), dtype=F64)
    k0 = n_q * head_dim
    v0 = k0 + n_kv * head_dim
    for j in range(n_q):
        g = j // group
        q = a[qrows, j * head_dim:(j + 1) * head_dim]
        k = a[:, k0 + g * head_dim:k0 + (g + 1) * head_dim]
        v = a[:, v0 + g * head_dim:v0 + (g + 1) * head_dim]
        s = scale * matmul(q, k.T)
        if causal:
            s = np.where(np.arange(T)[None, :] <= qrows[:, None], s, -np.inf)
        if T:
            s = s - np.max(s, axis=1, keepdims=True)
        e = np.exp(s)
        pm = e / np.sum(e, axis=1, keepdims=True)
        out[:, j * head_dim:(j + 1) * head_dim] = matmul(pm, v)
    return out


def attention_flops(T: int, n_q: int, head_dim: int, causal: bool) -> int:
    """Multiply-adds x 2 of Q K^T and P V over the (unmasked) score matrix."""
    pairs = T * (T + 1) // 2 if causal else T * T
    return 4 * pairs * head_dim * n_q


# ---------------------------------------------------------------------------
# Work accounting.  [KS] "What happens if TP leaves the node": training costs
# about 6 x params x tokens; the forward matmuls are 2 x params x tokens.
# ---------------------------------------------------------------------------
def mlp_shard_params(d: int, ff_i: int, act: str) -> int:
    return (3 if act == "swiglu" else 2) * d * ff_i


def mlp_fwd_flops(T: int, d: int, ff_i: int, act: str) -> int:
    return 2 * mlp_shard_params(d, ff_i, act) * T


def mlp_bwd_flops(T: int, d: int, ff_i: int, act: str) -> int:
    return 4 * mlp_shard_params(d, ff_i, act) * T


# ---------------------------------------------------------------------------
# Comparison metric (relative Frobenius error and max-abs error relative to
# the reference's largest magnitude).
# ---------------------------------------------------------------------------
def compare(got, ref) -> Tuple[float, float]:
    g = to64(got)
    r = to64(ref)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    if r.size == 0:
        return 0.0, 0.0
    diff = g - r
    nr = float(np.linalg.norm(r))
    mr = float(np.max(np.abs(r)))
    rel_frob = float(np.linalg.norm(diff)) / nr if nr > 0 else float(np.linalg.norm(diff))
    rel_max = float(np.max(np.abs(diff))) / mr if mr > 0 else float(np.max(np.abs(diff)))
    return rel_frob, rel_max


BF16_TOL = (5e-3, 1e-2)   # rel Frobenius, max-abs / max|ref|
F32_TOL = (1e-5, 1e-5)


def within(got, ref, tol=BF16_TOL) -> Tuple[bool, float, float]:
    rf, rm = compare(got, ref)
    return (rf <= tol[0] and rm <= tol[1]), rf, rm


__all__: List[str] = [n for n in dir() if not n.startswith("_")]
