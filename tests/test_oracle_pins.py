"""Pins for the fp64 oracle: each check ties the oracle to something other than itself.

Sources cited by page title and section:
  "Why Tensor Parallelism has to stay inside the scale-up domain" -
      "What is Tensor Parallel" (worked example), "What happens if TP leaves
      the node" (6 x params x tokens).
  "Tensor Parallelism" (inference-engineering notes) - paragraph 1 (column /
      row algebra), paragraph 2 (GQA bookkeeping), paragraph 5 (KV heads bound p).
  "How does tensor parallelism split a transformer feed-forward block's two
      matmuls across devices?" - "Column split, then row split",
      "The backward pass", "Common failure".
  "Tensor-parallel all-reduce count per transformer layer in MLX
      shard_linear" - Facts (bias added once after the sum).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            rows = [[float(t) for t in r.split()] for r in v.split(";")]
            out[k.strip()] = np.array(rows if len(rows) > 1 else rows[0], dtype=np.float64)
    return out


# --------------------------------------------------------------------------
# The pages' worked example (h=2, d_ff=3, TP=3), exact.
# --------------------------------------------------------------------------
def test_worked_example_unsharded_exact():
    g = load_golden("worked_example.txt")
    x = g["x"][None, :]
    for act in ("none", "relu"):
        y = O.col_linear(x, g["A"], act=act)
        assert np.array_equal(y[0], g["y"])
        assert np.array_equal(O.mlp_full(x, g["A"], None, g["B"], act)[0], g["z"])


def test_worked_example_tp3_shards_exact():
    g = load_golden("worked_example.txt")
    x = g["x"][None, :]
    p = int(g["tp"][0])
    partials = []
    for i in range(p):
        w1_i, _, w2_i = O.shard_mlp_weights(g["A"], None, g["B"], p, i)
        assert w1_i.shape == (2, 1) and w2_i.shape == (1, 2)   # one column of A, one row of B
        y_i, _ = O.mlp_shard_fwd(x, w1_i, None, w2_i, "relu")
        # each shard's intermediate is exactly the page's y[i]
        assert O.col_linear(x, w1_i, act="relu")[0, 0] == g["y"][i]
        partials.append(y_i)
    assert np.array_equal(O.partial_sum(partials)[0], g["z"])


# --------------------------------------------------------------------------
# Exact rational brute force on tiny integer inputs.
# --------------------------------------------------------------------------
def _brute_mlp_relu(x, w1, w2):
    T, d = len(x), len(x[0])
    ff = len(w1[0])
    h = [[max(Fraction(0), sum((x[t][k] * w1[k][j] for k in range(d)), Fraction(0))) for j in range(ff)]
         for t in range(T)]
    return [[sum((h[t][j] * w2[j][c] for j in range(ff)), Fraction(0)) for c in range(d)] for t in range(T)]


@pytest.mark.parametrize("p", [1, 2, 3, 6])
def test_bruteforce_fraction_relu(p):
    rng = np.random.default_rng(100 + p)
    T, d, ff = 3, 4, 6
    x = rng.integers(-3, 4, size=(T, d))
    w1 = rng.integers(-3, 4, size=(d, ff))
    w2 = rng.integers(-3, 4, size=(ff, d))
    exact = _brute_mlp_relu([[Fraction(int(v)) for v in r] for r in x],
                            [[Fraction(int(v)) for v in r] for r in w1],
                            [[Fraction(int(v)) for v in r] for r in w2])
    exact = np.array([[float(v) for v in r] for r in exact])
    assert np.array_equal(O.mlp_full(x, w1, None, w2, "relu"), exact)
    parts = []
    for i in range(p):
        a, _, c = O.shard_mlp_weights(w1, None, w2, p, i)
        parts.append(O.mlp_shard_fwd(x, a, None, c, "relu")[0])
    assert np.array_equal(O.partial_sum(parts), exact)


def test_bruteforce_matmul_triple_loop():
    rng = np.random.default_rng(7)
    a = rng.standard_normal((5, 7))
    b = rng.standard_normal((7, 3))
    ref = np.zeros((5, 3))
    for i in range(5):
        for j in range(3):
            s = 0.0
            for k in range(7):
                s += a[i, k] * b[k, j]
            ref[i, j] = s
    np.testing.assert_allclose(O.matmul(a, b), ref, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Sharding invariants (column concatenation, sum of row partials).
# --------------------------------------------------------------------------
@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu", "none"])
@pytest.mark.parametrize("p", [1, 2, 3, 4, 8])
def test_sum_of_partials_equals_unsharded(act, p):
    rng = np.random.default_rng(p * 10 + len(act))
    T, d, ff = 5, 16, 48
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((d, ff)) * 0.3
    wup = rng.standard_normal((d, ff)) * 0.3 if act == "swiglu" else None
    w2 = rng.standard_normal((ff, d)) * 0.3
    full = O.mlp_full(x, w1, wup, w2, act)
    parts, hs = [], []
    for i in range(p):
        a, u, c = O.shard_mlp_weights(w1, wup, w2, p, i)
        parts.append(O.mlp_shard_fwd(x, a, u, c, act)[0])
        hs.append(O.col_linear(x, a, u, None, act))
    rf, rm = O.compare(O.partial_sum(parts), full)
    assert rf < 1e-12 and rm < 1e-12
    # the concatenation of the column shards is the unsharded intermediate
    h_full = O.col_linear(x, w1, wup, None, act)
    np.testing.assert_allclose(np.concatenate(hs, axis=1), h_full, rtol=0, atol=1e-12)


def test_row_parallel_bias_added_once():
    """A row-parallel linear with bias: sum of partials + bias once equals the
    unsharded biased linear layer x W + b (the bias is not multiplied by p)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 12))
    w = rng.standard_normal((12, 5))
    b = rng.standard_normal(5)
    p = 4
    zs = []
    for i in range(p):
        s, n = O.shard_range(12, p, i)
        zs.append(O.row_linear_partial(x[:, s:s + n], w[s:s + n, :]))
    direct = np.array([[sum(x[t, k] * w[k, j] for k in range(12)) + b[j] for j in range(5)] for t in range(4)])
    np.testing.assert_allclose(O.partial_sum(zs, b), direct, rtol=1e-12, atol=1e-12)


def test_column_bias_slices():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 8))
    w = rng.standard_normal((8, 12))
    b = rng.standard_normal(12)
    full = O.col_linear(x, w, bias=b, act="gelu")
    for i in range(3):
        s, n = O.shard_range(12, 3, i)
        np.testing.assert_allclose(O.col_linear(x, w[:, s:s + n], bias=b[s:s + n], act="gelu"),
                                   full[:, s:s + n], rtol=1e-13, atol=1e-13)


# Hand values for the column-parallel bias (each shard adds its own slice of
# the bias BEFORE the activation, so h_i stays a genuine slice of h):
# x = [1, 2] through the worked example's A gives x A = [1, 2, 3]; with
# b = [-2, -1, -4] the pre-activations are [-1, 1, -1].  Adding the bias after
# the activation would give relu(x A) + b = [-1, 1, -1] instead of [0, 1, 0].
# Phi(-1) = 0.158655253931457051 (standard normal CDF), so gelu(-1) = -Phi(-1)
# and gelu(1) = 1 - Phi(-1).
_PHI_M1 = 0.158655253931457051
_BIAS_HAND = {"relu": [0.0, 1.0, 0.0],
              "gelu": [-_PHI_M1, 1.0 - _PHI_M1, -_PHI_M1],
              "none": [-1.0, 1.0, -1.0]}


def _column_bias_pin_error():
    """Largest deviation of the oracle's column-parallel linear (bf16-style and
    fp8 weights) from the hand values above, shard by shard (TP = 3, one column
    and one bias entry per shard)."""
    tpo = O.tp_oracle
    x = np.array([[1.0, 2.0]])
    a = np.array([[1.0, 0.0, 1.0], [0.0, 1.0, 1.0]])
    b = np.array([-2.0, -1.0, -4.0])
    # fp8 weights: code 0x40 is 2.0; with a column scale of 0.5 it is 1.0 again
    q = np.where(a > 0, 0x40, 0x00)
    sc = np.full(3, 0.5)
    err = 0.0
    for act, want in _BIAS_HAND.items():
        for i in range(3):
            s, n = O.shard_range(3, 3, i)
            got = tpo.col_linear(x, a[:, s:s + n], bias=b[s:s + n], act=act)
            got8 = tpo.col_linear_fp8(x, q[:, s:s + n], sc[s:s + n], bias=b[s:s + n], act=act)
            err = max(err, float(np.max(np.abs(got - want[i]))), float(np.max(np.abs(got8 - want[i]))))
    return err


def test_column_bias_hand_values():
    assert _column_bias_pin_error() <= 1e-15


def test_planted_bias_after_activation_is_caught(monkeypatch):
    """Adding the column bias after the activation must fail the hand values."""
    tpo = O.tp_oracle

    def wrong(x, w, w_up=None, bias=None, act="none"):
        h = tpo.act_apply(tpo.matmul(x, w), act)
        return h + O.to64(bias)[None, :] if bias is not None else h

    monkeypatch.setattr(tpo, "col_linear", wrong)
    assert _column_bias_pin_error() > 0.5


def test_planted_fp8_scale_after_bias_is_caught(monkeypatch):
    """Scaling the fp8 column sums after the bias is added must fail too."""
    tpo = O.tp_oracle

    def wrong(x, wq, scale, wq_up=None, scale_up=None, bias=None, act="none"):
        a = tpo.matmul(x, tpo.e4m3_decode(wq))
        if bias is not None:
            a = a + O.to64(bias)[None, :]
        return tpo.act_apply(a * O.to64(scale)[None, :], act)

    monkeypatch.setattr(tpo, "col_linear_fp8", wrong)
    assert _column_bias_pin_error() > 0.1


def test_row_then_column_needs_a_reduction_first():
    """Common failure: splitting the first matmul by rows yields partial sums,
    and the nonlinearity does not commute with the sum."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 8))
    w1 = rng.standard_normal((8, 10))
    parts = []
    for i in range(2):
        s, n = O.shard_range(8, 2, i)
        parts.append(O.relu(O.row_linear_partial(x[:, s:s + n], w1[s:s + n, :])))
    wrong = parts[0] + parts[1]
    right = O.relu(O.matmul(x, w1))
    assert np.max(np.abs(wrong - right)) > 1e-3


# --------------------------------------------------------------------------
# Activations: special values and library routines.
# --------------------------------------------------------------------------
def test_activation_special_values():
    assert O.relu(np.array([-1.0]))[0] == 0.0 and O.relu(np.array([2.5]))[0] == 2.5
    assert O.gelu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([0.0]))[0] == 0.0
    # Phi(1) and sigmoid(1) to double precision
    assert abs(O.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    assert abs(O.silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-15
    big = np.array([40.0, -40.0])
    np.testing.assert_allclose(O.gelu(big), [40.0, 0.0], atol=1e-300)
    np.testing.assert_allclose(O.silu(big), [40.0, -40.0 * math.exp(-40.0)], rtol=1e-12)


def test_activations_match_library_routines():
    xs = np.linspace(-8, 8, 1001)
    np.testing.assert_allclose(O.gelu(xs), xs * scipy.stats.norm.cdf(xs), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.silu(xs), xs * scipy.special.expit(xs), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.sigmoid(xs), scipy.special.expit(xs), rtol=1e-14, atol=0)


@pytest.mark.parametrize("name", ["relu", "gelu", "silu"])
def test_activation_derivatives_finite_difference(name):
    f = getattr(O, name)
    fp = getattr(O, name + "_grad")
    xs = np.linspace(-5, 5, 401)
    xs = xs[np.abs(xs) > 1e-3]            # ReLU is not differentiable at 0
    eps = 1e-6
    fd = (f(xs + eps) - f(xs - eps)) / (2 * eps)
    np.testing.assert_allclose(fp(xs), fd, rtol=1e-7, atol=1e-8)


# --------------------------------------------------------------------------
# Backward: central finite differences of L = sum(y * dy) on tiny shapes.
# --------------------------------------------------------------------------
def _fd_check(act, oracle_mod=O, seed=0):
    rng = np.random.default_rng(seed)
    T, d, ff = 3, 4, 6
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((d, ff)) * 0.7
    wup = rng.standard_normal((d, ff)) * 0.7 if act == "swiglu" else None
    w2 = rng.standard_normal((ff, d)) * 0.7
    dy = rng.standard_normal((T, d))

    def loss(x_, w1_, wup_, w2_):
        y, _ = O.mlp_shard_fwd(x_, w1_, wup_, w2_, act)
        return float(np.sum(y * dy))

    g = oracle_mod.mlp_shard_bwd(x, w1, wup, w2, dy, act)
    eps = 1e-6
    worst = 0.0
    params = {"dx": x, "dw1": w1, "dw2": w2}
    if wup is not None:
        params["dw_up"] = wup
    for key, arr in params.items():
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss(x, w1, wup, w2)
            arr[idx] = old - eps
            lm = loss(x, w1, wup, w2)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        worst = max(worst, float(np.max(np.abs(num - g[key])) / (np.max(np.abs(num)) + 1e-30)))
    return worst


@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu", "none"])
def test_backward_finite_difference(act):
    assert _fd_check(act) < 1e-6


def test_planted_mistake_in_backward_is_caught(monkeypatch):
    """A dropped term in silu' (s instead of s + g s (1 - s)) must fail the FD pin."""
    monkeypatch.setattr(O.tp_oracle, "silu_grad", lambda g: O.sigmoid(g))
    assert _fd_check("swiglu") > 1e-3


def test_planted_sign_error_in_gelu_grad_is_caught(monkeypatch):
    real = O.tp_oracle.gelu_grad
    monkeypatch.setattr(O.tp_oracle, "gelu_grad", lambda a: real(a) - 2 * a * np.exp(-0.5 * a * a) / math.sqrt(2 * math.pi))
    assert _fd_check("gelu") > 1e-3


@pytest.mark.parametrize("act", ["swiglu", "relu"])
def test_weight_gradients_are_shard_local_and_dx_partials_sum(act):
    """The backward pass: weight gradients need no exchange (each shard's
    gradient is the slice of the unsharded one), and the partial input
    gradients sum to the unsharded input gradient."""
    rng = np.random.default_rng(21)
    T, d, ff, p = 6, 8, 24, 4
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((d, ff)) * 0.4
    wup = rng.standard_normal((d, ff)) * 0.4 if act == "swiglu" else None
    w2 = rng.standard_normal((ff, d)) * 0.4
    dy = rng.standard_normal((T, d))
    full = O.mlp_full_bwd(x, w1, wup, w2, dy, act)
    dxs = []
    for i in range(p):
        s, n = O.shard_range(ff, p, i)
        a, u, c = O.shard_mlp_weights(w1, wup, w2, p, i)
        gi = O.mlp_shard_bwd(x, a, u, c, dy, act)
        np.testing.assert_allclose(gi["dw1"], full["dw1"][:, s:s + n], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(gi["dw2"], full["dw2"][s:s + n, :], rtol=1e-12, atol=1e-12)
        if act == "swiglu":
            np.testing.assert_allclose(gi["dw_up"], full["dw_up"][:, s:s + n], rtol=1e-12, atol=1e-12)
        dxs.append(gi["dx"])
    np.testing.assert_allclose(O.partial_sum(dxs), full["dx"], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Shard ranges and GQA bookkeeping.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n,p", [(256, 4), (28672, 8), (3, 3), (14336, 8), (0, 2)])
def test_shard_ranges_partition(n, p):
    covered = []
    for i in range(p):
        b, ln = O.shard_range(n, p, i)
        assert ln == n // p
        covered.extend(range(b, b + ln))
    assert covered == list(range(n))


def test_shard_range_rejects_uneven():
    with pytest.raises(ValueError):
        O.shard_range(10, 4, 0)


def test_gqa_shard_matches_the_page_numbers():
    """h=8192, 64 Q heads, 8 KV heads, head dim 128, p=8: each rank owns 8 Q
    heads and 1 KV head; local Q is 8192 x 1024, local K and V 8192 x 128,
    o_proj takes a 1024-wide input."""
    for i in range(8):
        qb, ql, kb, kl = O.gqa_shard(64, 8, 128, 8, i)
        assert (qb, ql, kb, kl) == (1024 * i, 1024, 128 * i, 128)
        # the rank's Q heads all group with its own KV head (contiguous grouping)
        for qh in range(qb // 128, (qb + ql) // 128):
            assert qh // (64 // 8) == kb // 128
    rng = np.random.default_rng(0)
    wq = rng.standard_normal((8192, 8192)).astype(np.float32)
    wk = rng.standard_normal((8192, 1024)).astype(np.float32)
    wv = rng.standard_normal((8192, 1024)).astype(np.float32)
    assert O.gqa_local_qkv_weight(wq, wk, wv, 64, 8, 128, 8, 3).shape == (8192, 1024 + 128 + 128)
    with pytest.raises(ValueError):          # 8 KV heads cannot map onto p = 16
        O.gqa_shard(64, 8, 128, 16, 0)


def test_gqa_local_qkv_is_slice_of_unsharded():
    rng = np.random.default_rng(5)
    h, nq, nkv, hd, p = 16, 8, 4, 2, 4
    x = rng.standard_normal((3, h))
    wq, wk, wv = (rng.standard_normal((h, n * hd)) for n in (nq, nkv, nkv))
    q, k, v = O.gqa_qkv_full(x, wq, wk, wv)
    for i in range(p):
        qb, ql, kb, kl = O.gqa_shard(nq, nkv, hd, p, i)
        loc = O.matmul(x, O.gqa_local_qkv_weight(wq, wk, wv, nq, nkv, hd, p, i))
        np.testing.assert_allclose(loc, np.concatenate([q[:, qb:qb + ql], k[:, kb:kb + kl], v[:, kb:kb + kl]], 1),
                                   rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Backward of the attention projections: a column-parallel QKV shard and a
# row-parallel o_proj shard ("The backward pass"; "Tensor Parallelism"
# paragraph 2).
# --------------------------------------------------------------------------
def _linear_fd_check(fn, T=3, K=4, N=4, seed=31):
    """Worst relative error of fn's (dW, dx) against central differences of
    L(x, W) = sum((x W) * dy), whose gradients are the backward's outputs."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, K))
    w = rng.standard_normal((K, N))
    dy = rng.standard_normal((T, N))
    g = fn(x, w, dy)

    def loss(x_, w_):
        return float(np.sum((x_ @ w_) * dy))

    worst = 0.0
    for key, arr in (("dx", x), ("dw", w)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + 1e-3
            lp = loss(x, w)
            arr[idx] = old - 1e-3
            lm = loss(x, w)
            arr[idx] = old
            num[idx] = (lp - lm) / 2e-3
        worst = max(worst, float(np.max(np.abs(num - g[key])) / np.max(np.abs(num))))
    return worst


def test_linear_backward_finite_difference():
    assert _linear_fd_check(O.linear_shard_bwd) < 1e-9
    assert _linear_fd_check(O.linear_shard_bwd, T=5, K=2, N=7) < 1e-9


def test_linear_backward_planted_transpose_is_caught():
    """dx = dy W instead of dy W^T (shapes agree when W is square) must fail."""
    wrong = lambda x, w, dy: {"dw": O.matmul(x.T, dy), "dx": O.matmul(dy, w)}
    assert _linear_fd_check(wrong) > 1e-2


def test_attention_projection_backward_shards():
    """QKV column-parallel: each rank's dW_qkv_i is its [Q_i | K_i | V_i]
    column slice of the unsharded weight gradient and the dx_i partials sum
    to the unsharded dx.  o_proj row-parallel: with dy replicated, dW_o_i is
    the rank's row slice of the unsharded gradient and dX_i the rank's
    column slice of the unsharded input gradient."""
    rng = np.random.default_rng(41)
    T, h, nq, nkv, hd, p = 5, 16, 8, 4, 2, 4
    x = rng.standard_normal((T, h))
    wq, wk, wv = (rng.standard_normal((h, n * hd)) for n in (nq, nkv, nkv))
    dq, dk, dv = (rng.standard_normal((T, n * hd)) for n in (nq, nkv, nkv))
    full = {n: O.linear_shard_bwd(x, w_, g_) for n, w_, g_ in (("q", wq, dq), ("k", wk, dk), ("v", wv, dv))}
    dx_full = full["q"]["dx"] + full["k"]["dx"] + full["v"]["dx"]
    attn = rng.standard_normal((T, nq * hd))
    wo = rng.standard_normal((nq * hd, h))
    dy = rng.standard_normal((T, h))
    ofull = O.linear_shard_bwd(attn, wo, dy)
    dxs = []
    for i in range(p):
        qb, ql, kb, kl = O.gqa_shard(nq, nkv, hd, p, i)
        w_i = O.gqa_local_qkv_weight(wq, wk, wv, nq, nkv, hd, p, i)
        d_i = np.concatenate([dq[:, qb:qb + ql], dk[:, kb:kb + kl], dv[:, kb:kb + kl]], 1)
        gi = O.linear_shard_bwd(x, w_i, d_i)
        np.testing.assert_allclose(gi["dw"], np.concatenate([full["q"]["dw"][:, qb:qb + ql],
                                                             full["k"]["dw"][:, kb:kb + kl],
                                                             full["v"]["dw"][:, kb:kb + kl]], 1),
                                   rtol=1e-12, atol=1e-12)
        dxs.append(gi["dx"])
        go = O.linear_shard_bwd(attn[:, qb:qb + ql], O.slice_rows(wo, qb, ql), dy)
        np.testing.assert_allclose(go["dw"], ofull["dw"][qb:qb + ql], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(go["dx"], ofull["dx"][:, qb:qb + ql], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.partial_sum(dxs), dx_full, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Local attention over the rank's heads ("Tensor Parallelism" paragraph 2;
# "How does tensor parallelism split..." attention paragraph).
# --------------------------------------------------------------------------
def _qkv(q, k, v):
    return np.concatenate([q, k, v], axis=1)


def test_attention_hand_values():
    """One head of width 1: q = [1, 2], k = [0, ln 3], v = [4, 8].  Row 0
    weighs the keys 1/4 and 3/4 (non-causal) and sees only key 0 (causal);
    row 1 has logits 0 and 2 ln 3, weights 1/10 and 9/10."""
    q = np.array([[1.0], [2.0]])
    k = np.array([[0.0], [math.log(3.0)]])
    v = np.array([[4.0], [8.0]])
    full = O.gqa_attention(_qkv(q, k, v), 1, 1, 1, False, 1.0)
    np.testing.assert_allclose(full[:, 0], [0.25 * 4 + 0.75 * 8, 0.1 * 4 + 0.9 * 8], rtol=1e-14)
    causal = O.gqa_attention(_qkv(q, k, v), 1, 1, 1, True, 1.0)
    np.testing.assert_allclose(causal[:, 0], [4.0, 0.1 * 4 + 0.9 * 8], rtol=1e-14)


def test_attention_uniform_keys_give_prefix_means():
    """Equal keys make every weight equal: the output is the mean of the
    visible values (all of them, or the prefix 0..t when causal)."""
    rng = np.random.default_rng(51)
    T, hd = 9, 4
    q = rng.standard_normal((T, hd))
    k = np.tile(rng.standard_normal((1, hd)), (T, 1))
    v = rng.standard_normal((T, hd))
    full = O.gqa_attention(_qkv(q, k, v), 1, 1, hd, False, 0.7)
    np.testing.assert_allclose(full, np.tile(v.mean(0), (T, 1)), rtol=1e-12, atol=1e-12)
    causal = O.gqa_attention(_qkv(q, k, v), 1, 1, hd, True, 0.7)
    prefix = np.cumsum(v, 0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(causal, prefix, rtol=1e-12, atol=1e-12)


def test_attention_invariances():
    """Permuting keys with their values leaves non-causal attention unchanged;
    adding one vector to every key shifts each row's logits by a constant and
    changes nothing, causal or not; a very large scale selects the value of
    the highest-scoring key."""
    rng = np.random.default_rng(52)
    T, hd = 7, 3
    q, k, v = (rng.standard_normal((T, hd)) for _ in range(3))
    base = O.gqa_attention(_qkv(q, k, v), 1, 1, hd, False, 0.5)
    perm = rng.permutation(T)
    np.testing.assert_allclose(O.gqa_attention(_qkv(q, k[perm], v[perm]), 1, 1, hd, False, 0.5), base,
                               rtol=1e-12, atol=1e-12)
    c = rng.standard_normal((1, hd))
    for causal in (False, True):
        ref = O.gqa_attention(_qkv(q, k, v), 1, 1, hd, causal, 0.5)
        np.testing.assert_allclose(O.gqa_attention(_qkv(q, k + c, v), 1, 1, hd, causal, 0.5), ref,
                                   rtol=1e-12, atol=1e-12)
    hard = O.gqa_attention(_qkv(q, k, v), 1, 1, hd, False, 1e4)
    np.testing.assert_allclose(hard, v[np.argmax(q @ k.T, axis=1)], rtol=1e-9, atol=1e-9)


def test_attention_matches_library_softmax():
    rng = np.random.default_rng(53)
    T, hd = 6, 5
    q, k, v = (rng.standard_normal((T, hd)) for _ in range(3))
    w = scipy.special.softmax(0.3 * (q @ k.T) + np.triu(np.full((T, T), -np.inf), 1), axis=1)
    np.testing.assert_allclose(O.gqa_attention(_qkv(q, k, v), 1, 1, hd, True, 0.3), w @ v, rtol=1e-12, atol=1e-12)


def test_gqa_attention_equals_mha_with_shared_kv():
    """Grouped-query attention with 4 query heads over 2 KV heads equals
    multi-head attention with each KV head repeated for its group of query
    heads (query heads 0, 1 read KV head 0; heads 2, 3 read KV head 1)."""
    rng = np.random.default_rng(54)
    T, hd = 5, 2
    q = rng.standard_normal((T, 4 * hd))
    k = rng.standard_normal((T, 2 * hd))
    v = rng.standard_normal((T, 2 * hd))
    rep = lambda a: np.concatenate([a[:, :hd], a[:, :hd], a[:, hd:], a[:, hd:]], 1)
    got = O.gqa_attention(_qkv(q, k, v), 4, 2, hd, True, 0.8)
    mha = O.gqa_attention(_qkv(q, rep(k), rep(v)), 4, 4, hd, True, 0.8)
    np.testing.assert_allclose(got, mha, rtol=1e-13, atol=1e-13)
    for j in range(4):       # and each head on its own
        one = O.gqa_attention(_qkv(q[:, j * hd:(j + 1) * hd], k[:, (j // 2) * hd:(j // 2 + 1) * hd],
                                   v[:, (j // 2) * hd:(j // 2 + 1) * hd]), 1, 1, hd, True, 0.8)
        np.testing.assert_allclose(got[:, j * hd:(j + 1) * hd], one, rtol=1e-13, atol=1e-13)


def test_attention_row_subset_equals_full():
    rng = np.random.default_rng(55)
    T, hd = 11, 3
    qkv = rng.standard_normal((T, (2 + 2) * hd))
    rows = [0, 4, 10]
    for causal in (False, True):
        full = O.gqa_attention(qkv, 2, 1, hd, causal, 0.6)
        np.testing.assert_allclose(O.gqa_attention(qkv, 2, 1, hd, causal, 0.6, rows=rows), full[rows],
                                   rtol=1e-13, atol=1e-13)


def test_attention_flops():
    assert O.attention_flops(4096, 8, 128, False) == 4 * 4096 * 4096 * 128 * 8
    assert O.attention_flops(3, 1, 1, True) == 4 * 6


# --------------------------------------------------------------------------
# fp8 (OCP E4M3) weights of the quantized sharded linear.
# --------------------------------------------------------------------------
def test_e4m3_hand_values():
    got = O.e4m3_decode(np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0x80, 0xB8, 0x40, 0x3C, 0x7F, 0xFF]))
    want = [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, 7 * 2.0 ** -9, -0.0, -1.0, 2.0, 1.5]
    np.testing.assert_array_equal(got[:9], want)
    assert np.signbit(got[5]) and np.isnan(got[9]) and np.isnan(got[10])


def test_e4m3_matches_library_for_every_code():
    """Every code against torch's float8_e4m3fn conversion (a library routine
    the oracle does not use)."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = O.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_fp8_linear_column_scales():
    """A per-column scale multiplies that output column (linear case), and the
    fp8 linear with unit scales is the plain linear of the decoded weights
    summed term by term (exact on small integers)."""
    rng = np.random.default_rng(61)
    x = rng.integers(-3, 4, size=(3, 5)).astype(np.float64)
    q = rng.integers(0, 256, size=(5, 4))
    q[q == 0x7F] = 0x38
    q[q == 0xFF] = 0xB8
    ones = np.ones(4)
    s = np.array([0.5, 2.0, 0.25, 8.0])
    base = O.row_linear_partial_fp8(x, q, ones)
    np.testing.assert_allclose(O.row_linear_partial_fp8(x, q, s), base * s[None, :], rtol=1e-15)
    vals = O.e4m3_decode(q)
    brute = np.array([[sum(x[t, k] * vals[k, n] for k in range(5)) for n in range(4)] for t in range(3)])
    np.testing.assert_allclose(base, brute, rtol=1e-13, atol=1e-13)
    y = O.col_linear_fp8(x, q, s, q, s, None, "swiglu")
    np.testing.assert_allclose(y, O.silu(base * s) * (base * s), rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Mixture of experts, experts sharded in place (MLX page, Facts).
# --------------------------------------------------------------------------
def test_moe_route_hand_values():
    idx, gate = O.moe_route(np.array([[0.0, 1.0, 1.0, -1.0], [2.0, 0.0, 0.0, 0.0]]), 2)
    np.testing.assert_array_equal(idx, [[1, 2], [0, 1]])            # equal logits: lower index first
    np.testing.assert_allclose(gate, [[0.5, 0.5], [math.e ** 2 / (math.e ** 2 + 1), 1 / (math.e ** 2 + 1)]],
                               rtol=1e-14)


def test_moe_route_nan_and_infinite_logits():
    """A NaN logit ranks as -inf: below every finite logit, tied with -inf
    (lower index first), and an expert picked at -inf gets gate exp(-inf) = 0."""
    nan, inf = float("nan"), float("inf")
    idx, gate = O.moe_route(np.array([[nan, 0.0, -inf, 1.0, nan],
                                      [-inf, nan, 2.0, -inf, 2.0]]), 4)
    np.testing.assert_array_equal(idx, [[3, 1, 0, 2], [2, 4, 0, 1]])
    e = math.e
    np.testing.assert_allclose(gate, [[e / (e + 1), 1 / (e + 1), 0.0, 0.0], [0.5, 0.5, 0.0, 0.0]], rtol=1e-14)


def test_moe_route_all_experts_is_the_softmax():
    rng = np.random.default_rng(71)
    lg = rng.standard_normal((5, 6))
    idx, gate = O.moe_route(lg, 6)
    sm = scipy.special.softmax(lg, axis=1)
    np.testing.assert_array_equal(idx, np.argsort(-lg, axis=1, kind="stable"))
    np.testing.assert_allclose(gate, np.take_along_axis(sm, idx, 1), rtol=1e-13)


def _moe_weights(rng, E, d, ff):
    return (rng.standard_normal((E, d, ff)) * 0.3, rng.standard_normal((E, d, ff)) * 0.3,
            rng.standard_normal((E, ff, d)) * 0.3)


def test_moe_identical_experts_reduce_to_the_dense_block():
    """With every expert equal and gates summing to 1 the block is the plain
    SwiGLU shard."""
    rng = np.random.default_rng(72)
    T, d, ff, E, k = 6, 8, 12, 5, 3
    x = rng.standard_normal((T, d))
    w1, wu, w2 = (np.repeat(a[:1], E, axis=0) for a in _moe_weights(rng, 1, d, ff))
    idx, gate = O.moe_route(rng.standard_normal((T, E)), k)
    dense, _ = O.mlp_shard_fwd(x, w1[0], wu[0], w2[0], "swiglu")
    np.testing.assert_allclose(O.moe_shard_fwd(x, idx, gate, w1, wu, w2), dense, rtol=1e-12, atol=1e-12)


def test_moe_in_place_shards_sum_to_the_block_and_match_a_token_loop():
    rng = np.random.default_rng(73)
    T, d, ff, E, k, p = 7, 8, 12, 4, 2, 3
    x = rng.standard_normal((T, d))
    w1, wu, w2 = _moe_weights(rng, E, d, ff)
    idx, gate = O.moe_route(rng.standard_normal((T, E)), k)
    full = O.moe_shard_fwd(x, idx, gate, w1, wu, w2)
    loop = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            g = x[t] @ w1[e]
            loop[t] += gate[t, j] * ((g / (1 + np.exp(-g)) * (x[t] @ wu[e])) @ w2[e])
    np.testing.assert_allclose(full, loop, rtol=1e-12, atol=1e-12)
    parts = []
    for i in range(p):
        b, n = O.shard_range(ff, p, i)
        parts.append(O.moe_shard_fwd(x, idx, gate, w1[:, :, b:b + n], wu[:, :, b:b + n], w2[:, b:b + n, :]))
    np.testing.assert_allclose(O.partial_sum(parts), full, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Work accounting: training ~ 6 x params x tokens.
# --------------------------------------------------------------------------
def test_flop_accounting():
    T, d, ff_i = 4096, 8192, 3584
    n = O.mlp_shard_params(d, ff_i, "swiglu")
    assert O.mlp_fwd_flops(T, d, ff_i, "swiglu") + O.mlp_bwd_flops(T, d, ff_i, "swiglu") == 6 * n * T
    assert O.mlp_fwd_flops(T, d, ff_i, "swiglu") == 721_554_505_728
    assert O.mlp_bwd_flops(2048, 4096, 1792, "swiglu") == 180_388_626_432
    # the page's training example: 6 x 70e9 x 4096 over 8 GPUs at 400 TFLOP/s ~ 0.5 s
    assert abs(6 * 70e9 * 4096 / 8 / 400e12 - 0.5) < 0.05


def test_compare_metric():
    r = np.array([[3.0, -4.0]])
    assert O.compare(r, r) == (0.0, 0.0)
    rf, rm = O.compare(r * 1.01, r)
    assert abs(rf - 0.01) < 1e-12 and abs(rm - 0.04 / 4.0) < 1e-12


# ---------------------------------------------------------------------------
# Sequence-parallel boundary: the rank's rows of sum + residual, then RMSNorm.
# ---------------------------------------------------------------------------
def test_rs_norm_hand_values():
    # one rank owns row 1 of 2; s = [2, -2] -> mean(s^2) = 4; eps = 5 -> sqrt(9) = 3
    z0 = np.array([[9.0, 9.0], [1.5, -0.5]])
    z1 = np.array([[9.0, 9.0], [0.5, -1.5]])
    res = np.array([[0.0, 0.0]])
    w = np.array([3.0, 0.75])
    s, y = O.rs_residual_rmsnorm([z0, z1], 1, res, w, 5.0)
    assert s.tolist() == [[2.0, -2.0]]
    assert np.allclose(y, [[2.0 / 3.0 * 3.0, -2.0 / 3.0 * 0.75]], rtol=0, atol=1e-15)
    # bias once after the partials, then the residual
    s, _ = O.rs_residual_rmsnorm([z0, z1], 0, np.array([[1.0, 2.0]]), w, 0.0, bias=np.array([0.25, 0.5]))
    assert s.tolist() == [[19.25, 20.5]]


def test_rs_norm_constant_rows_and_scale_invariance():
    rng = np.random.default_rng(5)
    T, N, p = 12, 7, 3
    c = rng.normal(size=(T, 1))
    zs = [np.repeat(c / p, N, axis=1) for _ in range(p)]
    w = rng.normal(size=N)
    for rank in range(p):
        res = np.zeros((T // p, N))
        s, y = O.rs_residual_rmsnorm(zs, rank, res, w, 0.0)
        # a constant row normalizes to its sign
        assert np.allclose(y, np.sign(c[rank * 4:(rank + 1) * 4]) * w[None, :], rtol=1e-12, atol=1e-12)
    # eps = 0: positive scaling of everything leaves y unchanged; y / w has unit RMS
    zs = [rng.normal(size=(T, N)) for _ in range(p)]
    res = rng.normal(size=(T // p, N))
    _, y1 = O.rs_residual_rmsnorm(zs, 2, res, w, 0.0)
    _, y2 = O.rs_residual_rmsnorm([3.5 * z for z in zs], 2, 3.5 * res, w, 0.0)
    assert np.allclose(y1, y2, rtol=1e-12, atol=1e-12)
    assert np.allclose(np.mean((y1 / w[None, :]) ** 2, axis=1), 1.0, rtol=1e-12)


def test_rs_norm_shares_tile_the_unsharded_sum():
    # element by element with plain loops: the p ranks' shares, stacked, are the
    # full residual add (reduce-scatter of the all-reduce's result)
    rng = np.random.default_rng(6)
    T, N, p = 6, 5, 3
    zs = [rng.normal(size=(T, N)) for _ in range(p)]
    res = rng.normal(size=(T, N))
    w = np.ones(N)
    got = np.vstack([O.rs_residual_rmsnorm(zs, r, res[r * 2:(r + 1) * 2], w, 1e-6)[0] for r in range(p)])
    for t in range(T):
        for n in range(N):
            want = res[t, n]
            for z in zs:
                want += z[t, n]
            assert abs(got[t, n] - want) < 1e-12
    with pytest.raises(ValueError):  # 5 rows do not split into 3 equal shares
        O.rs_residual_rmsnorm([z[:5] for z in zs], 0, res[:1], w, 0.0)
