"""GPU parity: every entry point of the C ABI against the fp64 oracle on the
same seeded inputs.

Bars: bf16 inputs with fp32 accumulation -> relative Frobenius error <= 5e-3
and max |err| <= 1e-2 * max |ref|; fp32 throughout -> both <= 1e-5; the
integer worked example -> bit-exact.  Large workloads are checked on a
seeded 64-row subset (rows are independent for the forward and for dx);
weight gradients reduce over all tokens, so they are checked in full.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import tensor_sharded_transformer_amd as tp

from test_oracle_pins import load_golden

pytestmark = pytest.mark.gpu

BF16_TOL = (5e-3, 1e-2)
F32_TOL = (1e-5, 1e-5)


def cuda(t):
    return t.contiguous().to("cuda")


def assert_close(got, ref, tol, what=""):
    ok, rf, rm = O.within(got, ref, tol)
    assert ok, f"{what}: rel_frob={rf:.3e} rel_max={rm:.3e} (tol {tol})"


def dt_of(t):
    return tp.TP_BF16 if t.dtype == torch.bfloat16 else tp.TP_F32


def fwd(x, w1, wup, w2, act, out_dtype=None, saved=False):
    T, d = x.shape
    ff_i = w1.shape[1]
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_workspace(T, d, ff_i, dt_of(x), act))
    y = torch.empty(T, d, dtype=out_dtype or x.dtype, device="cuda")
    sv = None
    if saved:
        sv = torch.empty(T, (2 if act == "swiglu" else 1) * ff_i, dtype=x.dtype, device="cuda")
    tp.tp_mlp_shard_fwd(x, w1, wup, w2, y, act, ws, sv)
    return y, sv


def bwd(x, w1, wup, w2, saved, dy, act):
    T, d = x.shape
    ff_i = w1.shape[1]
    ws = tp.new_workspace(tp.tp_mlp_shard_bwd_workspace(T, d, ff_i, dt_of(x), act))
    dw1 = torch.empty_like(w1)
    dwup = torch.empty_like(wup) if wup is not None else None
    dw2 = torch.empty_like(w2)
    dx = torch.empty_like(x)
    tp.tp_mlp_shard_bwd(x, w1, wup, w2, saved, dy, dw1, dwup, dw2, dx, act, ws)
    return dw1, dwup, dw2, dx


def shard(w1, wup, w2, p, i):
    """Host-side slicing of the unsharded weights with the library's own ranges."""
    b, n = tp.tp_shard_range(w1.shape[1], p, i)
    return (w1[:, b:b + n].contiguous(), None if wup is None else wup[:, b:b + n].contiguous(),
            w2[b:b + n, :].contiguous())


# ---------------------------------------------------------------------------
# The pages' worked example, bit-exact on the GPU.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_worked_example_exact(dtype):
    g = load_golden("worked_example.txt")
    x = cuda(torch.tensor(g["x"][None, :], dtype=dtype))
    A = torch.tensor(g["A"], dtype=dtype)
    Bm = torch.tensor(g["B"], dtype=dtype)
    p = int(g["tp"][0])
    parts = []
    for i in range(p):
        w1_i, _, w2_i = shard(A, None, Bm, p, i)
        w1_i, w2_i = cuda(w1_i), cuda(w2_i)
        h = torch.empty(1, 1, dtype=dtype, device="cuda")
        tp.tp_col_linear(x, w1_i, None, None, h, "relu")
        y_i, _ = fwd(x, w1_i, None, w2_i, "relu", out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert h.item() == g["y"][i]
        parts.append(y_i)
    z = torch.empty(1, 2, dtype=torch.float32, device="cuda")
    tp.tp_partial_sum(parts, None, z)
    assert z.cpu().numpy().tolist() == [g["z"].tolist()]


# ---------------------------------------------------------------------------
# Identity operand: the product must reproduce the other operand exactly
# (checks tile staging, the MFMA output mapping and the edge masks).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,N", [(64, 200), (300, 520), (1000, 1032)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_identity_times_w_is_w(T, N, dtype):
    x = cuda(torch.eye(T, dtype=dtype))
    w = W.normal((T, N), 1.0, 42, T + N, "f32").to(dtype)
    z = torch.empty(T, N, dtype=torch.float32, device="cuda")
    tp.tp_row_linear_partial(x, cuda(w), z)
    torch.cuda.synchronize()
    assert torch.equal(z.cpu(), w.float())


# ---------------------------------------------------------------------------
# Tiny fp32 MLP, p = 4 (x 4x64, W1 64x256, W2 256x64, ReLU).
# ---------------------------------------------------------------------------
def test_tiny_fp32_p4():
    w = W.TINY
    t = W.mlp_unsharded(w)
    x = cuda(t["x"])
    parts = []
    for i in range(w.p):
        w1_i, _, w2_i = shard(t["w1"], None, t["w2"], w.p, i)
        y_i, _ = fwd(x, cuda(w1_i), None, cuda(w2_i), w.act)
        o1, _, o2 = O.shard_mlp_weights(t["w1"], None, t["w2"], w.p, i)
        ref_i, _ = O.mlp_shard_fwd(O.to64(t["x"]), o1, None, o2, w.act)
        assert_close(y_i, ref_i, F32_TOL, f"shard {i}")
        parts.append(y_i)
    y = torch.empty(w.T, w.d, dtype=torch.float32, device="cuda")
    tp.tp_partial_sum(parts, None, y)
    ref = O.mlp_full(O.to64(t["x"]), O.to64(t["w1"]), None, O.to64(t["w2"]), w.act)
    assert_close(y, ref, F32_TOL, "sum of partials vs unsharded")


# ---------------------------------------------------------------------------
# Ragged shapes (nothing a multiple of the tile sizes), every activation.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("act", ["relu", "gelu", "swiglu", "none"])
@pytest.mark.parametrize("T,d,ff,p", [(5, 72, 120, 3), (77, 200, 168, 3), (300, 1000, 784, 2)])
def test_ragged_forward_and_sum(act, T, d, ff, p):
    w = W.MlpWorkload("ragged", T=T, d=d, ff=ff, p=p, act=act, dtype="bf16", seed=T + d)
    t = W.mlp_unsharded(w)
    x = cuda(t["x"])
    x64 = O.to64(t["x"])
    parts = []
    for i in range(p):
        w1_i, wup_i, w2_i = shard(t["w1"], t.get("w_up"), t["w2"], p, i)
        y_i, sv = fwd(x, cuda(w1_i), None if wup_i is None else cuda(wup_i), cuda(w2_i), act,
                      out_dtype=torch.float32, saved=True)
        o1, ou, o2 = O.shard_mlp_weights(t["w1"], t.get("w_up"), t["w2"], p, i)
        ref_i, ref_sv = O.mlp_shard_fwd(x64, o1, ou, o2, act)
        assert_close(y_i, ref_i, BF16_TOL, f"y_{i}")
        if act == "swiglu":
            ff_i = w1_i.shape[1]
            assert_close(sv[:, :ff_i], ref_sv["g"], BF16_TOL, "saved G")
            assert_close(sv[:, ff_i:], ref_sv["u"], BF16_TOL, "saved U")
        else:
            assert_close(sv, ref_sv["a"], BF16_TOL, "saved A")
        # the pieces separately: column GEMM + act, then row partial
        h = torch.empty(T, w1_i.shape[1], dtype=torch.bfloat16, device="cuda")
        tp.tp_col_linear(x, cuda(w1_i), None if wup_i is None else cuda(wup_i), None, h, act)
        assert_close(h, O.col_linear(x64, o1, ou, None, act), BF16_TOL, "h_i")
        # row partial on its own seeded input (never a GPU output fed to the oracle)
        h_in = W.normal((T, w1_i.shape[1]), 1.0, w.seed, 50 + i)
        z = torch.empty(T, d, dtype=torch.float32, device="cuda")
        tp.tp_row_linear_partial(cuda(h_in), cuda(w2_i), z)
        assert_close(z, O.row_linear_partial(O.to64(h_in), o2), BF16_TOL, "row partial")
        parts.append(y_i)
    y = torch.empty(T, d, dtype=torch.float32, device="cuda")
    tp.tp_partial_sum(parts, None, y)
    ref = O.mlp_full(x64, O.to64(t["w1"]), None if "w_up" not in t else O.to64(t["w_up"]), O.to64(t["w2"]), act)
    assert_close(y, ref, BF16_TOL, "sum of partials vs unsharded")


def test_act_inplace_matches_oracle():
    for act in ("relu", "gelu", "swiglu"):
        h = W.normal((37, 99), 2.0, 5, 1)
        up = W.normal((37, 99), 1.0, 5, 2) if act == "swiglu" else None
        hd = cuda(h)
        tp.tp_act_inplace(hd, None if up is None else cuda(up), act)
        ref = O.act_apply(O.to64(h), act, None if up is None else O.to64(up))
        assert_close(hd, ref, BF16_TOL, act)
        # fp32 variant
        hf = cuda(h.float())
        tp.tp_act_inplace(hf, None if up is None else cuda(up.float()), act)
        assert_close(hf, ref, (2e-6, 2e-6), act + " f32")


def test_col_linear_with_bias_is_a_slice():
    x = W.normal((50, 96), 1.0, 9, 1)
    w = W.normal((96, 240), 0.1, 9, 2)
    b = W.normal((240,), 1.0, 9, 3)
    full = O.col_linear(O.to64(x), O.to64(w), bias=O.to64(b), act="gelu")
    for i in range(3):
        s, n = tp.tp_shard_range(240, 3, i)
        y = torch.empty(50, n, dtype=torch.bfloat16, device="cuda")
        tp.tp_col_linear(cuda(x), cuda(w[:, s:s + n]), None, cuda(b[s:s + n]), y, "gelu")
        assert_close(y, full[:, s:s + n], BF16_TOL, f"shard {i}")


def test_partial_sum_bias_once_and_dtypes():
    zs = [W.normal((33, 80), 1.0, 11, i) for i in range(5)]
    bias = W.normal((80,), 1.0, 11, 9)
    ref = O.partial_sum([O.to64(z) for z in zs], O.to64(bias))
    for out in (torch.float32, torch.bfloat16):
        y = torch.empty(33, 80, dtype=out, device="cuda")
        tp.tp_partial_sum([cuda(z) for z in zs], cuda(bias), y)
        assert_close(y, ref, F32_TOL if out == torch.float32 else BF16_TOL, str(out))
    # fp32 inputs, odd sizes (scalar path)
    zf = [W.normal((7, 13), 1.0, 12, i, "f32") for i in range(3)]
    y = torch.empty(7, 13, dtype=torch.float32, device="cuda")
    tp.tp_partial_sum([cuda(z) for z in zf], None, y)
    assert_close(y, O.partial_sum([O.to64(z) for z in zf]), F32_TOL, "f32 ragged")


# ---------------------------------------------------------------------------
# Sequence-parallel boundary: a rank's rows of the partials' sum + residual,
# then RMSNorm (ragged N takes the scalar path; the last case is the prefill
# size, T=4096, N=8192, p=8).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("p,T,N,in_dt,out_dt,with_bias", [
    (1, 3, 1000, "bf16", "bf16", False),
    (3, 12, 1000, "bf16", "f32", True),
    (4, 8, 4100, "f32", "f32", False),
    (2, 6, 77, "bf16", "bf16", True),
    (8, 4096, 8192, "bf16", "bf16", False),
    (2, 4, 32768, "bf16", "f32", True),        # the largest row the kernel takes (whole row in LDS)
    (2, 4, 32768, "f32", "f32", False),
    (1, 2, 32761, "bf16", "bf16", False),      # odd row length: the scalar path
])
def test_rs_residual_rmsnorm(p, T, N, in_dt, out_dt, with_bias):
    seed = p * 1000 + N
    zs = [W.normal((T, N), 1.0, seed, i, in_dt) for i in range(p)]
    bias = W.normal((N,), 1.0, seed, 90, in_dt) if with_bias else None
    norm_w = W.normal((N,), 1.0, seed, 91, out_dt)
    eps = 1e-5
    dz = [cuda(z) for z in zs]
    odt = torch.bfloat16 if out_dt == "bf16" else torch.float32
    tol = BF16_TOL if out_dt == "bf16" else F32_TOL
    ranks = range(p) if T * N < 10 ** 6 else (5,)
    for rank in ranks:
        res = W.normal((T // p, N), 1.0, seed, 100 + rank, out_dt)
        r_out = torch.empty(T // p, N, dtype=odt, device="cuda")
        y = torch.empty(T // p, N, dtype=odt, device="cuda")
        tp.tp_rs_residual_rmsnorm(dz, rank, None if bias is None else cuda(bias), cuda(res), cuda(norm_w), eps,
                                  r_out, y)
        ref_s, ref_y = O.rs_residual_rmsnorm([O.to64(z) for z in zs], rank, O.to64(res), O.to64(norm_w), eps,
                                             None if bias is None else O.to64(bias))
        assert_close(r_out, ref_s, tol, f"residual, rank {rank}")
        assert_close(y, ref_y, tol, f"normalized, rank {rank}")
        # the residual may be updated in place
        r_io = cuda(res)
        y2 = torch.empty_like(y)
        tp.tp_rs_residual_rmsnorm(dz, rank, None if bias is None else cuda(bias), r_io, cuda(norm_w), eps, r_io, y2)
        assert torch.equal(r_io, r_out) and torch.equal(y2, y)


def test_zero_tokens_is_a_noop():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    w1 = torch.zeros(64, 32, dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros(32, 64, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    tp.tp_mlp_shard_fwd(x, w1, None, w2, y, "relu", None)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Large single GEMM through the 256x256 tiles with ragged edges.
# ---------------------------------------------------------------------------
def test_large_ragged_row_partial():
    T, K, N = 2000, 264, 8100
    x = W.normal((T, K), 1.0, 21, 1)
    w = W.normal((K, N), 0.02, 21, 2)
    z = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    tp.tp_row_linear_partial(cuda(x), cuda(w), z)
    rows = W.row_subset(T, 64, 21)
    assert_close(z[rows], O.matmul(O.to64(x[rows]), O.to64(w)), BF16_TOL, "rows")


# ---------------------------------------------------------------------------
# The 70B-class SwiGLU shard at decode (T=64, split-K path) and prefill.
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def rank0_weights():
    return W.mlp_rank_weights(W.DECODE, 0)


def test_decode_T64_shard(rank0_weights):
    w = W.DECODE
    x = W.mlp_input(w)
    wt = rank0_weights
    y, sv = fwd(cuda(x), cuda(wt["w1"]), cuda(wt["w_up"]), cuda(wt["w2"]), "swiglu", saved=True)
    ref, rsv = O.mlp_shard_fwd(O.to64(x), O.to64(wt["w1"]), O.to64(wt["w_up"]), O.to64(wt["w2"]), "swiglu")
    assert_close(y, ref, BF16_TOL, "y_0 decode")
    assert_close(sv[:, :w.ff_i], rsv["g"], BF16_TOL, "G")
    # determinism: the split-K reduction order is fixed
    y2, _ = fwd(cuda(x), cuda(wt["w1"]), cuda(wt["w_up"]), cuda(wt["w2"]), "swiglu")
    assert torch.equal(y, y2)


# ---------------------------------------------------------------------------
# Decode-size forward (weight-streaming kernels, h written straight into the
# row GEMM's packed activations): ragged T and d, every activation, both
# output types.  Asking for the saved activations takes the per-element
# epilogue instead of the staged one; the sums are the same, so the two agree
# bit for bit.  Two calls in a row on one workspace with different x check
# that nothing stale is read and that the counters are left zero.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("act", ["swiglu", "relu", "gelu", "none"])
@pytest.mark.parametrize("T,d,ff_i", [(1, 1024, 512), (40, 1000, 384), (64, 2056, 1024)])
def test_decode_step(act, T, d, ff_i):
    seed = 7 * T + d + ff_i
    w1 = W.normal((d, ff_i), 0.05, seed, 1)
    wup = W.normal((d, ff_i), 0.05, seed, 2) if act == "swiglu" else None
    w2 = W.normal((ff_i, d), 0.05, seed, 3)
    xs = [W.normal((T, d), 1.0, seed, 4 + r) for r in range(2)]
    dw1, dwup, dw2 = cuda(w1), None if wup is None else cuda(wup), cuda(w2)
    o1, ou, o2 = O.to64(w1), None if wup is None else O.to64(wup), O.to64(w2)
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_workspace(T, d, ff_i, tp.TP_BF16, act))
    for out in (torch.bfloat16, torch.float32):
        for r, x in enumerate(xs):
            ref, _ = O.mlp_shard_fwd(O.to64(x), o1, ou, o2, act)
            y = torch.empty(T, d, dtype=out, device="cuda")
            tp.tp_mlp_shard_fwd(cuda(x), dw1, dwup, dw2, y, act, ws)
            assert_close(y, ref, BF16_TOL, f"call {r}, out {out}")
            y2, _ = fwd(cuda(x), dw1, dwup, dw2, act, out_dtype=out, saved=True)
            assert torch.equal(y, y2), "staged and per-element epilogues differ"


def test_decode_step_repeats(rank0_weights):
    """The 70B-class decode shard, many back-to-back steps on one workspace
    (each relies on the previous one having re-zeroed the split-K counters)."""
    w = W.DECODE
    x = W.mlp_input(w)
    wt = rank0_weights
    args = [cuda(wt["w1"]), cuda(wt["w_up"]), cuda(wt["w2"])]
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_workspace(w.T, w.d, w.ff_i, tp.TP_BF16, "swiglu"))
    xd = cuda(x)
    ys = [torch.empty(w.T, w.d, dtype=torch.bfloat16, device="cuda") for _ in range(20)]
    for y in ys:
        tp.tp_mlp_shard_fwd(xd, *args, y, "swiglu", ws)
    torch.cuda.synchronize()
    ref, _ = O.mlp_shard_fwd(O.to64(x), O.to64(wt["w1"]), O.to64(wt["w_up"]), O.to64(wt["w2"]), "swiglu")
    assert_close(ys[-1], ref, BF16_TOL, "last of 20")
    for y in ys[:-1]:
        assert torch.equal(y, ys[-1])


@pytest.mark.parametrize("shift_gate,shift_up", [(0, 0), (128, 128), (640, 640), (384, 0), (896, 256)])
def test_decode_weight_address_classes(shift_gate, shift_up):
    """Decode GEMMs whose weight bytes start at different 128-byte offsets:
    the extra K splits land on other column strips (or are off when gate and
    up disagree); every case matches the oracle, and two calls agree bit for
    bit."""
    T, d, ff_i = 64, 2048, 1024
    w1 = W.normal((d, ff_i), 0.05, 41, 1)
    wup = W.normal((d, ff_i), 0.05, 41, 2)
    x = W.normal((T, d), 1.0, 41, 3)

    def at_offset(w, shift):
        # the weight rows start `shift` bytes into a larger buffer (row stride unchanged)
        n = w.numel() + 4096
        buf = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
        view = buf[shift // 2: shift // 2 + w.numel()].view(w.shape)
        view.copy_(cuda(w))
        return view

    g, u = at_offset(w1, shift_gate), at_offset(wup, shift_up)
    assert (g.data_ptr() - u.data_ptr()) % 128 == (shift_gate - shift_up) % 128
    ws = tp.new_workspace(tp.tp_col_linear_workspace(T, d, ff_i, tp.TP_BF16, "swiglu"))
    h = torch.empty(T, ff_i, dtype=torch.bfloat16, device="cuda")
    tp.tp_col_linear(cuda(x), g, u, None, h, "swiglu", ws)
    ref = O.col_linear(O.to64(x), O.to64(w1), O.to64(wup), None, "swiglu")
    assert_close(h, ref, BF16_TOL, f"gate +{shift_gate} B, up +{shift_up} B")
    h2 = torch.empty_like(h)
    tp.tp_col_linear(cuda(x), g, u, None, h2, "swiglu", ws)
    assert torch.equal(h, h2)


def test_decode_step_graph_replay():
    """The decode step captured as a HIP graph: several replays, with other
    eager calls and synchronisations between them, each bit-identical to the
    eager step (the step issues no memset; its split-K counters re-zero
    themselves)."""
    T, d, ff_i = 64, 2048, 1024
    w1, wup, w2 = (cuda(W.normal(s, 0.05, 31, k)) for k, s in ((1, (d, ff_i)), (2, (d, ff_i)), (3, (ff_i, d))))
    x = cuda(W.normal((T, d), 1.0, 31, 4))
    x_other = cuda(W.normal((T, d), 1.0, 31, 5))
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_workspace(T, d, ff_i, tp.TP_BF16, "swiglu"))
    ws_other = tp.new_workspace(tp.tp_mlp_shard_fwd_workspace(T, d, ff_i, tp.TP_BF16, "swiglu"))
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    y_other = torch.empty_like(y)
    tp.tp_mlp_shard_fwd(x, w1, wup, w2, y, "swiglu", ws)
    torch.cuda.synchronize()
    y_eager = y.clone()
    ref, _ = O.mlp_shard_fwd(O.to64(x.cpu()), O.to64(w1.cpu()), O.to64(wup.cpu()), O.to64(w2.cpu()), "swiglu")
    assert_close(y_eager, ref, BF16_TOL, "eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tp.tp_mlp_shard_fwd(x, w1, wup, w2, y, "swiglu", ws)
    for r in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r}"
        tp.tp_mlp_shard_fwd(x_other, w1, wup, w2, y_other, "swiglu", ws_other)
        tp.tp_mlp_shard_fwd(x_other, w1, wup, w2, y_other, "swiglu", ws)   # the graph's workspace, eagerly
        torch.cuda.synchronize()


def test_prefill_T4096_shard(rank0_weights):
    w = W.PREFILL
    x = W.mlp_input(w)
    wt = rank0_weights
    y, _ = fwd(cuda(x), cuda(wt["w1"]), cuda(wt["w_up"]), cuda(wt["w2"]), "swiglu")
    rows = W.row_subset(w.T, 64, w.seed)
    ref, _ = O.mlp_shard_fwd(O.to64(x[rows]), O.to64(wt["w1"]), O.to64(wt["w_up"]), O.to64(wt["w2"]), "swiglu")
    assert_close(y[rows], ref, BF16_TOL, "y_0 prefill rows")
    y2, _ = fwd(cuda(x), cuda(wt["w1"]), cuda(wt["w_up"]), cuda(wt["w2"]), "swiglu")
    assert torch.equal(y, y2)


# ---------------------------------------------------------------------------
# GQA projections (h=8192, 64 Q heads, 8 KV heads, head_dim 128, p=8).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("wl", [W.GQA_DECODE, W.GQA_PREFILL], ids=lambda w: w.name)
def test_gqa_projections(wl):
    t = W.gqa_unsharded(wl)
    rows = W.row_subset(wl.T, 64, wl.seed)
    x = cuda(t["x"])
    x64 = O.to64(t["x"][rows])
    parts = []
    for i in range(wl.p):
        qb, ql, kb, kl = tp.tp_gqa_shard(wl.n_q, wl.n_kv, wl.head_dim, wl.p, i)
        wqkv = torch.cat([t["wq"][:, qb:qb + ql], t["wk"][:, kb:kb + kl], t["wv"][:, kb:kb + kl]], 1).contiguous()
        assert wqkv.shape == (8192, 1280)
        if i in (0, wl.p - 1):
            ws = tp.new_workspace(tp.tp_col_linear_workspace(wl.T, wl.h, 1280, tp.TP_BF16, "none"))
            qkv = torch.empty(wl.T, 1280, dtype=torch.bfloat16, device="cuda")
            tp.tp_col_linear(x, cuda(wqkv), None, None, qkv, "none", ws)
            ref = O.matmul(x64, O.gqa_local_qkv_weight(t["wq"], t["wk"], t["wv"], wl.n_q, wl.n_kv, wl.head_dim,
                                                       wl.p, i))
            assert_close(qkv[rows], ref, BF16_TOL, f"qkv rank {i}")
        a_i = cuda(t["attn"][:, qb:qb + ql])
        wo_i = cuda(t["wo"][qb:qb + ql, :])
        ws = tp.new_workspace(tp.tp_row_linear_partial_workspace(wl.T, ql, wl.h, tp.TP_BF16))
        o_i = torch.empty(wl.T, wl.h, dtype=torch.bfloat16, device="cuda")
        tp.tp_row_linear_partial(a_i, wo_i, o_i, ws)
        parts.append(o_i)
    y = torch.empty(wl.T, wl.h, dtype=torch.float32, device="cuda")
    tp.tp_partial_sum(parts, None, y)
    ref = O.matmul(O.to64(t["attn"][rows]), O.to64(t["wo"]))
    assert_close(y[rows], ref, BF16_TOL, "sum of o_proj partials")
    ref0 = O.matmul(O.to64(t["attn"][rows][:, :1024]), O.to64(t["wo"][:1024]))
    assert_close(parts[0][rows], ref0, BF16_TOL, "o_proj partial rank 0")


# ---------------------------------------------------------------------------
# Backward.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("act,ff", [("swiglu", 168), ("relu", 168), ("gelu", 168), ("none", 168),
                                    ("swiglu", 174), ("gelu", 174)])
def test_backward_small_ragged(act, ff):
    """ff = 168: 56 columns per shard (the dh epilogue's 16-byte path);
    ff = 174: 58 (its element-wise path)."""
    w = W.MlpWorkload("bwd_small", T=70, d=136, ff=ff, p=3, act=act, dtype="bf16", seed=31)
    t = W.mlp_unsharded(w, with_dy=True)
    x, dy = cuda(t["x"]), cuda(t["dy"])
    dxs = []
    for i in range(w.p):
        w1_i, wup_i, w2_i = (None if v is None else cuda(v) for v in shard(t["w1"], t.get("w_up"), t["w2"], w.p, i))
        _, sv = fwd(x, w1_i, wup_i, w2_i, act, saved=True)
        dw1, dwup, dw2, dx = bwd(x, w1_i, wup_i, w2_i, sv, dy, act)
        o1, ou, o2 = O.shard_mlp_weights(t["w1"], t.get("w_up"), t["w2"], w.p, i)
        ref = O.mlp_shard_bwd(O.to64(t["x"]), o1, ou, o2, O.to64(t["dy"]), act)
        assert_close(dw1, ref["dw1"], BF16_TOL, "dW1")
        assert_close(dw2, ref["dw2"], BF16_TOL, "dW2")
        if act == "swiglu":
            assert_close(dwup, ref["dw_up"], BF16_TOL, "dWup")
        assert_close(dx, ref["dx"], BF16_TOL, "dx_i")
        dxs.append(dx)
    y = torch.empty_like(x, dtype=torch.float32)
    tp.tp_partial_sum(dxs, None, y)
    full = O.mlp_full_bwd(O.to64(t["x"]), O.to64(t["w1"]), None if "w_up" not in t else O.to64(t["w_up"]),
                          O.to64(t["w2"]), O.to64(t["dy"]), act)
    assert_close(y, full["dx"], BF16_TOL, "sum of dx partials")


def test_backward_T2048_all_shards():
    w = W.BACKWARD
    t = W.mlp_unsharded(w, with_dy=True)
    x, dy = cuda(t["x"]), cuda(t["dy"])
    rows = W.row_subset(w.T, 64, w.seed)
    x64, dy64 = O.to64(t["x"]), O.to64(t["dy"])
    dxs = []
    for i in range(w.p):
        w1_i, wup_i, w2_i = (cuda(v) for v in shard(t["w1"], t["w_up"], t["w2"], w.p, i))
        _, sv = fwd(x, w1_i, wup_i, w2_i, "swiglu", saved=True)
        dw1, dwup, dw2, dx = bwd(x, w1_i, wup_i, w2_i, sv, dy, "swiglu")
        if i in (0, w.p - 1):
            o1, ou, o2 = O.shard_mlp_weights(t["w1"], t["w_up"], t["w2"], w.p, i)
            ref = O.mlp_shard_bwd(x64, o1, ou, o2, dy64, "swiglu")
            assert_close(dw1, ref["dw1"], BF16_TOL, f"dW1_{i}")
            assert_close(dwup, ref["dw_up"], BF16_TOL, f"dWup_{i}")
            assert_close(dw2, ref["dw2"], BF16_TOL, f"dW2_{i}")
            assert_close(dx[rows], ref["dx"][rows], BF16_TOL, f"dx_{i}")
        dxs.append(dx)
    y = torch.empty(w.T, w.d, dtype=torch.float32, device="cuda")
    tp.tp_partial_sum(dxs, None, y)
    full = O.mlp_shard_bwd(x64[rows], O.to64(t["w1"]), O.to64(t["w_up"]), O.to64(t["w2"]), dy64[rows], "swiglu")
    assert_close(y[rows], full["dx"], BF16_TOL, "sum of the 8 dx partials vs unsharded dx")


# ---------------------------------------------------------------------------
# Backward of the attention projections (linear shards).
# ---------------------------------------------------------------------------
def lin_bwd(x, w, dy, want_dw=True, want_dx=True):
    T, K = (dy.shape[0], w.shape[0]) if w is not None else (dy.shape[0], x.shape[1])
    N = dy.shape[1]
    ws = tp.new_workspace(tp.tp_linear_shard_bwd_workspace(T, K, N, dt_of(dy)))
    dw = torch.full((K, N), 7.0, dtype=dy.dtype, device="cuda") if want_dw else None
    dx = torch.full((T, K), 7.0, dtype=dy.dtype, device="cuda") if want_dx else None
    tp.tp_linear_shard_bwd(x, w, dy, dw, dx, ws)
    return dw, dx


@pytest.mark.parametrize("T,K,N", [(77, 200, 131), (300, 1000, 264), (5, 72, 1280), (640, 1024, 520)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_linear_shard_bwd_ragged(T, K, N, dtype):
    x = W.normal((T, K), 1.0, 61, 1, dtype)
    w = W.normal((K, N), 0.02, 61, 2, dtype)
    dy = W.normal((T, N), 1.0, 61, 3, dtype)
    dw, dx = lin_bwd(cuda(x), cuda(w), cuda(dy))
    ref = O.linear_shard_bwd(x, w, dy)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    assert_close(dw, ref["dw"], tol, "dW")
    assert_close(dx, ref["dx"], tol, "dx")
    # one output at a time gives the same values
    dw1, none_x = lin_bwd(cuda(x), None, cuda(dy), want_dx=False)
    none_w, dx1 = lin_bwd(None, cuda(w), cuda(dy), want_dw=False)
    assert none_x is None and none_w is None
    assert torch.equal(dw1, dw) and torch.equal(dx1, dx)


def test_linear_shard_bwd_empty():
    dy = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(0, 32, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(32, 64, dtype=torch.bfloat16, device="cuda")
    dw, dx = lin_bwd(x, w, dy)
    assert dx.shape == (0, 32) and bool((dw == 0).all())          # T = 0: zero weight gradient
    dy = torch.ones(16, 0, dtype=torch.bfloat16, device="cuda")
    x = torch.ones(16, 32, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(32, 0, dtype=torch.bfloat16, device="cuda")
    dw, dx = lin_bwd(x, w, dy)
    assert dw.shape == (32, 0) and bool((dx == 0).all())          # N = 0: zero input gradient


@pytest.mark.parametrize("T", [4096, 64])
def test_attention_projection_backward(T):
    """The 70B-class GQA projections' backward on every rank: QKV
    column-parallel (dW_qkv_i in full for ranks 0 and 7, the 8 dx partials
    summed against the unsharded dx) and o_proj row-parallel (dW_o_i in full,
    dX_i on sampled rows)."""
    wl = W.GQA_BWD
    t = W.gqa_unsharded(wl)
    g = W.gqa_grads(wl, T)
    x_all = t["x"][:T]
    attn = t["attn"][:T]
    rows = W.row_subset(T, 64, wl.seed)
    x = cuda(x_all)
    dy = cuda(g["dy"])
    x64, dy64 = O.to64(x_all), O.to64(g["dy"])
    dxs = []
    for i in range(wl.p):
        qb, ql, kb, kl = tp.tp_gqa_shard(wl.n_q, wl.n_kv, wl.head_dim, wl.p, i)
        wqkv = torch.cat([t["wq"][:, qb:qb + ql], t["wk"][:, kb:kb + kl], t["wv"][:, kb:kb + kl]], 1)
        dqkv = torch.cat([g["dq"][:, qb:qb + ql], g["dk"][:, kb:kb + kl], g["dv"][:, kb:kb + kl]], 1)
        dw, dx = lin_bwd(x, cuda(wqkv), cuda(dqkv))
        dxs.append(dx)
        a_i, wo_i = attn[:, qb:qb + ql], t["wo"][qb:qb + ql, :]
        dwo, da = lin_bwd(cuda(a_i), cuda(wo_i), dy)
        if i in (0, wl.p - 1):
            ref = O.linear_shard_bwd(x64, wqkv, dqkv)
            assert_close(dw, ref["dw"], BF16_TOL, f"dW_qkv rank {i}")
            assert_close(dx[rows], ref["dx"][rows], BF16_TOL, f"dx partial rank {i}")
            ref = O.linear_shard_bwd(a_i, wo_i, dy64)
            assert_close(dwo, ref["dw"], BF16_TOL, f"dW_o rank {i}")
            assert_close(da[rows], ref["dx"][rows], BF16_TOL, f"dX rank {i}")
    y = torch.empty(T, wl.h, dtype=torch.float32, device="cuda")
    tp.tp_partial_sum(dxs, None, y)
    full = sum(O.linear_shard_bwd(x64[rows], t[w_], g[d_][rows])["dx"] for w_, d_ in (("wq", "dq"), ("wk", "dk"), ("wv", "dv")))
    assert_close(y[rows], full, BF16_TOL, "sum of the 8 QKV dx partials vs unsharded dx")


# ---------------------------------------------------------------------------
# Local grouped-query attention.
# ---------------------------------------------------------------------------
def attn(qkv, n_q, n_kv, causal, scale):
    out = torch.full((qkv.shape[0], n_q * 128), 7.0, dtype=torch.bfloat16, device="cuda")
    return tp.tp_gqa_attention_fwd(qkv, out, n_q, n_kv, 128, causal, scale)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("T,n_q,n_kv,std", [(1, 8, 1, 1.0), (5, 8, 1, 1.0), (77, 8, 1, 1.81), (200, 4, 2, 1.0),
                                            (300, 2, 2, 3.0), (129, 8, 1, 1.81), (640, 8, 1, 1.81)])
def test_attention_ragged(causal, T, n_q, n_kv, std):
    qkv = W.normal((T, (n_q + 2 * n_kv) * 128), std, 71 + T, 1)
    scale = 128 ** -0.5
    got = attn(cuda(qkv), n_q, n_kv, causal, scale)
    ref = O.gqa_attention(qkv, n_q, n_kv, 128, causal, scale)
    assert_close(got, ref, BF16_TOL, f"attention T={T} causal={causal}")


@pytest.mark.parametrize("causal", [True, False])
def test_attention_T4096_rank_heads(causal):
    """A 70B-class rank's 8 query heads over its 1 KV head at T=4096, on 64
    sampled query rows (each row depends only on its own query)."""
    wl = W.GQA_ATTN
    qkv = W.attention_qkv(wl)
    n_q, n_kv = wl.n_q // wl.p, wl.n_kv // wl.p
    scale = wl.head_dim ** -0.5
    got = attn(cuda(qkv), n_q, n_kv, causal, scale)
    rows = sorted(set(W.row_subset(wl.T, 62, wl.seed) + [0, wl.T - 1]))
    ref = O.gqa_attention(qkv, n_q, n_kv, wl.head_dim, causal, scale, rows=rows)
    assert_close(got[rows], ref, BF16_TOL, "attention rows")
    again = attn(cuda(qkv), n_q, n_kv, causal, scale)
    assert torch.equal(got, again)          # deterministic


@pytest.mark.parametrize("T,n_q,n_kv,causal", [(4000, 8, 1, True), (4000, 8, 1, False), (1000, 8, 2, True),
                                                (2113, 4, 4, False), (8192, 8, 1, True)])
def test_attention_ragged_long(T, n_q, n_kv, causal):
    """Lengths that leave partial key tiles and uneven key ranges across the
    workgroup's groups, on 48 sampled query rows plus the first and last."""
    qkv = W.normal((T, (n_q + 2 * n_kv) * 128), 1.81, 90 + T, 1)
    scale = 128 ** -0.5
    got = attn(cuda(qkv), n_q, n_kv, causal, scale)
    rows = sorted(set(W.row_subset(T, 48, T) + [0, T - 1]))
    ref = O.gqa_attention(qkv, n_q, n_kv, 128, causal, scale, rows=rows)
    assert_close(got[rows], ref, BF16_TOL, f"attention T={T}")


def test_attention_between_the_projections():
    """QKV projection -> local attention -> o_proj partial on one rank, chained
    through the C ABI, against the fp64 oracle chain on sampled rows.

    The chain hands its intermediates (qkv, then the attention output) from
    one launch to the next as bf16 tensors, the precision every activation in
    these workloads is stored in.  The oracle chain rounds its own fp64 qkv and
    attention output to bf16 (round to nearest even) at the same two points and
    is fp64 everywhere else, so each stage is held to one kernel's tolerance."""
    wl = W.GQA_PREFILL
    T = 512
    t = W.gqa_unsharded(wl)
    i = 2
    qb, ql, kb, kl = tp.tp_gqa_shard(wl.n_q, wl.n_kv, wl.head_dim, wl.p, i)
    wqkv = torch.cat([t["wq"][:, qb:qb + ql], t["wk"][:, kb:kb + kl], t["wv"][:, kb:kb + kl]], 1).contiguous()
    x = t["x"][:T].contiguous()
    qkv = torch.empty(T, 1280, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(tp.tp_col_linear_workspace(T, wl.h, 1280, tp.TP_BF16, "none"))
    tp.tp_col_linear(cuda(x), cuda(wqkv), None, None, qkv, "none", ws)
    a = attn(qkv, 8, 1, True, 128 ** -0.5)
    wo_i = cuda(t["wo"][qb:qb + ql, :])
    z = torch.empty(T, wl.h, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(tp.tp_row_linear_partial_workspace(T, ql, wl.h, tp.TP_BF16))
    tp.tp_row_linear_partial(a, wo_i, z, ws)
    rows = W.row_subset(T, 32, 7)

    def bf16(v):   # the chain's intermediate precision
        return O.to64(torch.from_numpy(v).to(torch.bfloat16))

    qkv64 = O.matmul(O.to64(x), O.gqa_local_qkv_weight(t["wq"], t["wk"], t["wv"], wl.n_q, wl.n_kv, wl.head_dim,
                                                       wl.p, i))
    assert_close(qkv, qkv64, BF16_TOL, "qkv projection")
    a64 = O.gqa_attention(bf16(qkv64), 8, 1, 128, True, 128 ** -0.5, rows=rows)
    z64 = O.row_linear_partial(bf16(a64), O.to64(t["wo"][qb:qb + ql, :]))
    for what, got, ref in (("attention on the projected qkv", a[rows], a64), ("o_proj partial", z[rows], z64)):
        _, rf, rm = O.within(got, ref)
        print(f"{what}: rel_frob={rf:.3e} rel_max={rm:.3e}")
        assert_close(got, ref, BF16_TOL, what)


# ---------------------------------------------------------------------------
# fp8 (E4M3) weights at decode sizes.
# ---------------------------------------------------------------------------
def packed(q):
    """Device copy of (K, N) row-major codes in the strip-major order."""
    dst = torch.empty(q.shape, dtype=torch.uint8, device="cuda")
    return tp.tp_fp8_pack_strips(cuda(q), dst)


@pytest.mark.parametrize("K,N", [(1, 64), (5, 128), (1000, 3584), (33, 1088)])
def test_fp8_pack_strips_is_the_strip_permutation(K, N):
    q = torch.randint(0, 256, (K, N), dtype=torch.uint8)
    want = q.reshape(K, N // 64, 64).permute(1, 0, 2).contiguous().reshape(K, N)
    assert torch.equal(packed(q).cpu(), want)


@pytest.mark.parametrize("T,K,N", [(1, 1000, 256), (40, 4096, 1088), (64, 1000, 3584), (33, 2056, 512)])
@pytest.mark.parametrize("act", ["none", "relu", "gelu", "swiglu"])
def test_fp8_col_linear(T, K, N, act):
    x = W.normal((T, K), 1.0, 81, 1)
    q = W.e4m3_codes((K, N), 81, 2)
    if N == 256:   # every finite code, both signs and the subnormals, somewhere in the matrix
        allc = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
        q[:2] = allc.repeat(4)[: 2 * N].view(2, N)
    sc = W.column_scales(N, 81, 3)
    qu = W.e4m3_codes((K, N), 81, 4) if act == "swiglu" else None
    su = W.column_scales(N, 81, 5) if act == "swiglu" else None
    bias = W.normal((N,), 0.1, 81, 6) if act in ("relu", "gelu") else None
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(tp.tp_linear_fp8_workspace(T, K, N, act))
    tp.tp_col_linear_fp8(cuda(x), packed(q), cuda(sc), None if qu is None else packed(qu),
                         None if su is None else cuda(su), None if bias is None else cuda(bias), y, act, ws)
    ref = O.col_linear_fp8(x, q, sc, qu, su, bias, act)
    assert_close(y, ref, BF16_TOL, f"fp8 col linear {act}")


@pytest.mark.parametrize("out_dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,K,N", [(64, 3584, 8192), (7, 1000, 1024)])
def test_fp8_row_linear_partial(T, K, N, out_dt):
    x = W.normal((T, K), 1.0, 82, 1)
    q = W.e4m3_codes((K, N), 82, 2)
    sc = W.column_scales(N, 82, 3)
    z = torch.full((T, N), 7.0, dtype=out_dt, device="cuda")
    ws = tp.new_workspace(tp.tp_linear_fp8_workspace(T, K, N, "none"))
    qp = packed(q)
    tp.tp_row_linear_partial_fp8(cuda(x), qp, cuda(sc), z, ws)
    assert_close(z, O.row_linear_partial_fp8(x, q, sc), BF16_TOL, "fp8 row partial")
    again = torch.empty_like(z)
    tp.tp_row_linear_partial_fp8(cuda(x), qp, cuda(sc), again, ws)
    assert torch.equal(z, again)


def test_fp8_decode_shard_T64():
    """The 70B-class SwiGLU shard at decode size with fp8 weights: gate/up
    column-parallel then down row-parallel, all 64 rows against the fp64
    chain."""
    T, d, ff_i = 64, 8192, 3584
    x = W.normal((T, d), 1.0, 83, 1)
    qg, qu, qd = W.e4m3_codes((d, ff_i), 83, 2), W.e4m3_codes((d, ff_i), 83, 3), W.e4m3_codes((ff_i, d), 83, 4)
    sg, su, sd = W.column_scales(ff_i, 83, 5), W.column_scales(ff_i, 83, 6), W.column_scales(d, 83, 7)
    h = torch.empty(T, ff_i, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(max(tp.tp_linear_fp8_workspace(T, d, ff_i, "swiglu"),
                              tp.tp_linear_fp8_workspace(T, ff_i, d, "none")))
    tp.tp_col_linear_fp8(cuda(x), packed(qg), cuda(sg), packed(qu), cuda(su), None, h, "swiglu", ws)
    tp.tp_row_linear_partial_fp8(h, packed(qd), cuda(sd), y, ws)
    h64 = O.col_linear_fp8(x, qg, sg, qu, su, None, "swiglu")
    assert_close(h, h64, BF16_TOL, "fp8 gate/up + SwiGLU")
    assert_close(y, O.row_linear_partial_fp8(h64, qd, sd), BF16_TOL, "fp8 shard output")


@pytest.mark.parametrize("T,act", [(64, "swiglu"), (1, "swiglu"), (40, "gelu"), (33, "relu")])
def test_fp8_mlp_shard_fwd(T, act):
    """The fused fp8 shard (h handed to the row GEMM in packed form) against the
    fp64 chain, and bitwise against the two separate fp8 linears."""
    d, ff_i = 8192, 3584
    x = W.normal((T, d), 1.0, 84, 1)
    q1, qd = W.e4m3_codes((d, ff_i), 84, 2), W.e4m3_codes((ff_i, d), 84, 4)
    qu = W.e4m3_codes((d, ff_i), 84, 3) if act == "swiglu" else None
    s1, sd = W.column_scales(ff_i, 84, 5), W.column_scales(d, 84, 7)
    su = W.column_scales(ff_i, 84, 6) if act == "swiglu" else None
    p1, pu, p2 = packed(q1), None if qu is None else packed(qu), packed(qd)
    c1, cu, c2 = cuda(s1), None if su is None else cuda(su), cuda(sd)
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_fp8_workspace(T, d, ff_i, act))
    tp.tp_mlp_shard_fwd_fp8(cuda(x), p1, c1, pu, cu, p2, c2, y, act, ws)
    h64 = O.col_linear_fp8(x, q1, s1, qu, su, None, act)
    assert_close(y, O.row_linear_partial_fp8(h64, qd, sd), BF16_TOL, f"fp8 shard {act}")
    h = torch.empty(T, ff_i, dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y)
    ws2 = tp.new_workspace(max(tp.tp_linear_fp8_workspace(T, d, ff_i, act), tp.tp_linear_fp8_workspace(T, ff_i, d)))
    tp.tp_col_linear_fp8(cuda(x), p1, c1, pu, cu, None, h, act, ws2)
    tp.tp_row_linear_partial_fp8(h, p2, c2, y2, ws2)
    assert torch.equal(y, y2)


# ---------------------------------------------------------------------------
# fp8 (E4M3) weights packed in MFMA fragment order (k-pairs of 16-column strips).
# ---------------------------------------------------------------------------
def packed8(q):
    """Device copy of (K, N) row-major codes in the packed fp8 layout."""
    return tp.tp_pack_weight_fp8(cuda(q))


def packed8_layout_cpu(q):
    """The packed fp8 layout written out: chunk (pair p, strip s), lane l, byte
    8h + j holds code[64p + 32h + 8(l // 16) + j, 16s + l % 16], zero padded."""
    K, N = q.shape
    nkp, ns = (K + 63) // 64, (N + 15) // 16
    qp = torch.zeros(nkp * 64, ns * 16, dtype=torch.uint8)
    qp[:K, :N] = q
    return qp.reshape(nkp, 2, 4, 8, ns, 16).permute(0, 4, 2, 5, 1, 3).reshape(-1)


@pytest.mark.parametrize("K,N", [(1, 16), (5, 40), (130, 24), (1000, 3584), (64, 4096)])
def test_pack_weight_fp8_is_the_fragment_permutation(K, N):
    q = torch.randint(0, 256, (K, N), dtype=torch.uint8, generator=torch.Generator().manual_seed(7 * K + N))
    assert torch.equal(packed8(q).cpu(), packed8_layout_cpu(q))


@pytest.mark.parametrize("T,K,N", [(1, 1000, 256), (40, 4096, 1088), (64, 1000, 3584), (33, 2056, 520),
                                   (64, 8192, 1280)])
@pytest.mark.parametrize("act", ["none", "relu", "gelu", "swiglu"])
def test_fp8_col_linear_packed(T, K, N, act):
    """Ragged K (not whole k-pairs) and N (not whole strips), every activation,
    every finite code with both signs and the subnormals at N = 256."""
    x = W.normal((T, K), 1.0, 85, 1)
    q = W.e4m3_codes((K, N), 85, 2)
    if N == 256:
        allc = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
        q[:2] = allc.repeat(4)[: 2 * N].view(2, N)
    sc = W.column_scales(N, 85, 3)
    qu = W.e4m3_codes((K, N), 85, 4) if act == "swiglu" else None
    su = W.column_scales(N, 85, 5) if act == "swiglu" else None
    bias = W.normal((N,), 0.1, 85, 6) if act in ("relu", "gelu") else None
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(tp.tp_linear_packed_fp8_workspace(T, K, N, act))
    tp.tp_col_linear_packed_fp8(cuda(x), packed8(q), cuda(sc), None if qu is None else packed8(qu),
                                None if su is None else cuda(su), None if bias is None else cuda(bias), y, act, K, N,
                                ws)
    assert_close(y, O.col_linear_fp8(x, q, sc, qu, su, bias, act), BF16_TOL, f"packed fp8 col linear {act}")


@pytest.mark.parametrize("out_dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,K,N", [(64, 3584, 8192), (7, 1000, 1000), (1, 33, 24)])
def test_fp8_row_linear_partial_packed(T, K, N, out_dt):
    x = W.normal((T, K), 1.0, 86, 1)
    q = W.e4m3_codes((K, N), 86, 2)
    sc = W.column_scales(N, 86, 3)
    z = torch.full((T, N), 7.0, dtype=out_dt, device="cuda")
    ws = tp.new_workspace(tp.tp_linear_packed_fp8_workspace(T, K, N, "none"))
    qp = packed8(q)
    tp.tp_row_linear_partial_packed_fp8(cuda(x), qp, cuda(sc), z, N, ws)
    assert_close(z, O.row_linear_partial_fp8(x, q, sc), BF16_TOL, "packed fp8 row partial")
    again = torch.empty_like(z)
    tp.tp_row_linear_partial_packed_fp8(cuda(x), qp, cuda(sc), again, N, ws)
    assert torch.equal(z, again)


@pytest.mark.parametrize("T,act", [(64, "swiglu"), (1, "swiglu"), (40, "gelu"), (33, "relu")])
def test_fp8_mlp_shard_fwd_packed(T, act):
    """The 70B-class shard at decode size on packed fp8 codes (h handed to the
    row GEMM in operand order) against the fp64 chain, and bitwise against the
    two separate packed fp8 linears."""
    d, ff_i = 8192, 3584
    x = W.normal((T, d), 1.0, 87, 1)
    q1, qd = W.e4m3_codes((d, ff_i), 87, 2), W.e4m3_codes((ff_i, d), 87, 4)
    qu = W.e4m3_codes((d, ff_i), 87, 3) if act == "swiglu" else None
    s1, sd = W.column_scales(ff_i, 87, 5), W.column_scales(d, 87, 7)
    su = W.column_scales(ff_i, 87, 6) if act == "swiglu" else None
    p1, pu, p2 = packed8(q1), None if qu is None else packed8(qu), packed8(qd)
    c1, cu, c2 = cuda(s1), None if su is None else cuda(su), cuda(sd)
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_packed_fp8_workspace(T, d, ff_i, act))
    tp.tp_mlp_shard_fwd_packed_fp8(cuda(x), p1, c1, pu, cu, p2, c2, y, act, ff_i, ws)
    h64 = O.col_linear_fp8(x, q1, s1, qu, su, None, act)
    assert_close(y, O.row_linear_partial_fp8(h64, qd, sd), BF16_TOL, f"packed fp8 shard {act}")
    h = torch.empty(T, ff_i, dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y)
    ws2 = tp.new_workspace(max(tp.tp_linear_packed_fp8_workspace(T, d, ff_i, act),
                               tp.tp_linear_packed_fp8_workspace(T, ff_i, d)))
    tp.tp_col_linear_packed_fp8(cuda(x), p1, c1, pu, cu, None, h, act, d, ff_i, ws2)
    assert_close(h, h64, BF16_TOL, f"packed fp8 h {act}")
    tp.tp_row_linear_partial_packed_fp8(h, p2, c2, y2, d, ws2)
    assert torch.equal(y, y2)


def test_one_workspace_serves_every_entry_point():
    """One zero-initialised workspace reused across entry points and shapes in
    sequence gives bitwise the results each call gives with a fresh one (the
    split-K counters stay in their reserved, zero region)."""
    T, d, ff_i = 64, 2048, 512
    x = cuda(W.normal((T, d), 1.0, 91, 1))
    w1, wu, w2 = (cuda(W.normal(sh, 0.02, 91, k)) for k, sh in ((2, (d, ff_i)), (3, (d, ff_i)), (4, (ff_i, d))))
    q, sc = packed(W.e4m3_codes((ff_i, d), 91, 5)), cuda(W.column_scales(d, 91, 6))
    a = cuda(W.normal((T, 1024), 1.0, 91, 7))
    wo = cuda(W.normal((1024, 4096), 0.02, 91, 8))
    calls = {
        "mlp": (lambda ws: tp.tp_mlp_shard_fwd(x, w1, wu, w2, torch.empty(T, d, dtype=torch.bfloat16, device="cuda"),
                                               "swiglu", ws),
                tp.tp_mlp_shard_fwd_workspace(T, d, ff_i, tp.TP_BF16, "swiglu")),
        "col": (lambda ws: tp.tp_col_linear(x, w1, wu, None, torch.empty(T, ff_i, dtype=torch.bfloat16,
                                                                         device="cuda"), "swiglu", ws),
                tp.tp_col_linear_workspace(T, d, ff_i, tp.TP_BF16, "swiglu")),
        "row": (lambda ws: tp.tp_row_linear_partial(a, wo, torch.empty(T, 4096, dtype=torch.bfloat16, device="cuda"),
                                                    ws),
                tp.tp_row_linear_partial_workspace(T, 1024, 4096, tp.TP_BF16)),
        "fp8": (lambda ws: tp.tp_row_linear_partial_fp8(x[:, :ff_i].contiguous(), q, sc,
                                                        torch.empty(T, d, dtype=torch.bfloat16, device="cuda"), ws),
                tp.tp_linear_fp8_workspace(T, ff_i, d, "none")),
    }
    fresh = {k: f(tp.new_workspace(n)) for k, (f, n) in calls.items()}
    shared = tp.new_workspace(max(n for _, n in calls.values()))
    for order in (["mlp", "col", "row", "fp8"], ["fp8", "row", "col", "mlp"], ["col", "mlp", "fp8", "row"]):
        for k in order:
            assert torch.equal(calls[k][0](shared), fresh[k]), f"{k} after {order}"


@pytest.mark.parametrize("T", [64, 300])
def test_empty_contraction(T):
    """K = 0: the column-parallel linear gives act(bias) in every row and the
    row-parallel partial gives zeros (decode and tiled sizes, with and without
    a workspace)."""
    N = 256
    x = torch.empty(T, 0, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(0, N, dtype=torch.bfloat16, device="cuda")
    bias = cuda(W.normal((N,), 1.0, 95, 1))
    for with_ws in (True, False):
        ws = tp.new_workspace(tp.tp_col_linear_workspace(T, 0, N, tp.TP_BF16, "relu")) if with_ws else None
        y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
        tp.tp_col_linear(x, w, None, bias, y, "relu", ws)
        assert torch.equal(y, torch.relu(bias.float()).to(torch.bfloat16).expand(T, N))
        ws = tp.new_workspace(tp.tp_row_linear_partial_workspace(T, 0, N, tp.TP_BF16)) if with_ws else None
        z = torch.full((T, N), 7.0, dtype=torch.float32, device="cuda")
        tp.tp_row_linear_partial(x, w, z, ws)
        assert bool((z == 0).all())


def test_empty_intermediate_and_no_tokens():
    """ff_i = 0: the shard's partial is zero and so is its dx_i; T = 0: the
    weight gradients are zero."""
    T, d = 16, 128
    x = cuda(W.normal((T, d), 1.0, 96, 1))
    e_w1 = torch.empty(d, 0, dtype=torch.bfloat16, device="cuda")
    e_w2 = torch.empty(0, d, dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, d), 7.0, dtype=torch.bfloat16, device="cuda")
    tp.tp_mlp_shard_fwd(x, e_w1, None, e_w2, y, "relu", None)
    assert bool((y == 0).all())
    dy = cuda(W.normal((T, d), 1.0, 96, 2))
    dx = torch.full((T, d), 7.0, dtype=torch.bfloat16, device="cuda")
    sv = torch.empty(T, 0, dtype=torch.bfloat16, device="cuda")
    tp.tp_mlp_shard_bwd(x, e_w1, None, e_w2, sv, dy, torch.empty_like(e_w1), None, torch.empty_like(e_w2), dx,
                        "relu", None)
    assert bool((dx == 0).all())
    w1 = cuda(W.normal((d, 64), 0.02, 96, 3))
    w2 = cuda(W.normal((64, d), 0.02, 96, 4))
    g1 = torch.full_like(w1, 7.0)
    g2 = torch.full_like(w2, 7.0)
    x0 = torch.empty(0, d, dtype=torch.bfloat16, device="cuda")
    tp.tp_mlp_shard_bwd(x0, w1, None, w2, torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"),
                        torch.empty(0, d, dtype=torch.bfloat16, device="cuda"), g1, None, g2,
                        torch.empty(0, d, dtype=torch.bfloat16, device="cuda"), "relu", None)
    assert bool((g1 == 0).all()) and bool((g2 == 0).all())


def test_block_rows_graph_replay():
    """Local attention, the fp8 decode shard and the sequence-parallel boundary
    captured together in one HIP graph: several replays with eager calls in
    between, each bit-identical to the eager results (none of them issues a
    memset)."""
    T, d, ff_i = 64, 2048, 512
    qkv = cuda(W.normal((256, 1280), 1.81, 97, 1))
    att = torch.empty(256, 1024, dtype=torch.bfloat16, device="cuda")
    x = cuda(W.normal((T, d), 1.0, 97, 2))
    q1, qu, q2 = (packed(W.e4m3_codes(sh, 97, k)) for k, sh in ((3, (d, ff_i)), (4, (d, ff_i)), (5, (ff_i, d))))
    s1, su, s2 = cuda(W.column_scales(ff_i, 97, 6)), cuda(W.column_scales(ff_i, 97, 7)), cuda(W.column_scales(d, 97, 8))
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_fp8_workspace(T, d, ff_i, "swiglu"))
    zs = [cuda(W.normal((T, d), 1.0, 97, 10 + i)) for i in range(4)]
    res, nw = cuda(W.normal((T // 4, d), 1.0, 97, 20)), cuda(W.normal((d,), 1.0, 97, 21))
    r_out = torch.empty_like(res)
    yn = torch.empty_like(res)

    def run():
        tp.tp_gqa_attention_fwd(qkv, att, 8, 1, 128, True, 128 ** -0.5)
        tp.tp_mlp_shard_fwd_fp8(x, q1, s1, qu, su, q2, s2, y, "swiglu", ws)
        tp.tp_rs_residual_rmsnorm(zs, 1, None, res, nw, 1e-5, r_out, yn)

    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (att, y, r_out, yn)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for r in range(3):
        for t in (att, y, r_out, yn):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((att, y, r_out, yn), eager):
            assert torch.equal(a, b), f"replay {r}"
        run()   # eager calls on the same buffers and workspace between replays
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Mixture of experts, experts sharded in place.
# ---------------------------------------------------------------------------
def moe_run(t, k, out_dt=torch.bfloat16):
    T, d = t["x"].shape
    E, _, ff_i = t["w1"].shape
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    tp.tp_moe_route(cuda(t["logits"]), k, idx, gate)
    y = torch.full((T, d), 7.0, dtype=out_dt, device="cuda")
    ws = tp.new_workspace(tp.tp_moe_shard_fwd_workspace(T, d, ff_i, E, k))
    tp.tp_moe_shard_fwd(cuda(t["x"]), idx, gate, cuda(t["w1"]), cuda(t["w_up"]), cuda(t["w2"]), y, ws)
    return idx, gate, y


@pytest.mark.parametrize("T,d,ff_i,E,k", [(1, 64, 32, 4, 2), (77, 256, 96, 16, 4), (300, 512, 200, 8, 8),
                                         (513, 128, 64, 64, 1), (200, 640, 120, 8, 2), (64, 384, 40, 4, 3)])
def test_moe_small(T, d, ff_i, E, k):
    wl = W.MoeWorkload("moe_small", T=T, d=d, ff=ff_i, E=E, k=k, p=1, seed=40 + T)
    t = W.moe_rank_inputs(wl)
    idx, gate, y = moe_run(t, k)
    ridx, rgate = O.moe_route(t["logits"], k)
    assert torch.equal(idx.cpu().long(), torch.from_numpy(ridx)), "routing decisions"
    np.testing.assert_allclose(gate.cpu().numpy(), rgate, rtol=1e-5, atol=1e-6)
    ref = O.moe_shard_fwd(t["x"], ridx, rgate, t["w1"], t["w_up"], t["w2"])
    assert_close(y, ref, BF16_TOL, "moe block")
    _, _, y2 = moe_run(t, k, torch.float32)
    assert_close(y2, ref, BF16_TOL, "moe block, fp32 out")


@pytest.mark.parametrize("E,k", [(128, 8), (1024, 16), (65, 5)])
def test_moe_route_ties_nan_and_infinities(E, k):
    """Routing with many equal logits, against the oracle bit for bit.  Small
    integer logits tie everywhere; planted rows put equal maxima on the lanes
    the wave arg-max pairs up (l and l^1, l^2, l^4, l^16, l^32) and on the
    register slots of one lane (e and e + 64, ...); other rows hold NaN (ranks
    as -inf) and -inf logits, some with fewer finite logits than k."""
    rng = np.random.default_rng(E * 100 + k)
    T = 96
    lg = rng.integers(0, 4, size=(T, E)).astype(np.float32)
    for t in range(0, 32):                       # butterfly and slot partners of one lane, equal maxima
        l = int(rng.integers(0, 64))
        lg[t] = 0.0
        for e in (l, l ^ 1, l ^ 2, l ^ 4, l ^ 16, l ^ 32, l + 64, l + 128, (l ^ 1) + 64):
            if e < E:
                lg[t, e] = 5.0
    lg[32:40] = 1.0                              # every logit equal
    for t in range(40, 64):                      # NaN and -inf sprinkled over integer logits
        lg[t, rng.choice(E, E // 3, replace=False)] = np.nan
        lg[t, rng.choice(E, E // 4, replace=False)] = -np.inf
    for t in range(64, 72):                      # fewer finite logits than k
        lg[t] = np.nan
        lg[t, rng.choice(E, E // 2, replace=False)] = -np.inf
        lg[t, rng.choice(E, k // 2, replace=False)] = 2.0
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    tp.tp_moe_route(cuda(torch.from_numpy(lg)), k, idx, gate)
    ridx, rgate = O.moe_route(lg, k)
    assert torch.equal(idx.cpu().long(), torch.from_numpy(ridx)), "routing decisions"
    np.testing.assert_allclose(gate.cpu().numpy(), rgate, rtol=1e-5, atol=1e-7)


def test_moe_qwen3_class_rank_T4096():
    """A Qwen3-MoE-class layer's rank share (128 experts, top-8, d=2048,
    ff_i=96) at T=4096 on 64 sampled tokens, and run-to-run bitwise equal."""
    wl = W.MOE_PREFILL
    t = W.moe_rank_inputs(wl)
    idx, gate, y = moe_run(t, wl.k)
    rows = W.row_subset(wl.T, 64, wl.seed)
    ridx, rgate = O.moe_route(t["logits"][rows], wl.k)
    assert torch.equal(idx[rows].cpu().long(), torch.from_numpy(ridx))
    ref = O.moe_shard_fwd(t["x"][rows], ridx, rgate, t["w1"], t["w_up"], t["w2"])
    assert_close(y[rows], ref, BF16_TOL, "moe rank rows")
    _, _, y_again = moe_run(t, wl.k)
    assert torch.equal(y, y_again)


def test_moe_x_of_2gib_takes_the_gathered_path():
    """x of exactly 2 GiB (65536 x 16384 bf16) is past the GEMM's 32-bit row
    offsets, so the routed rows are first gathered into the grouped order;
    checked on 32 sampled tokens."""
    T, d, ff_i, E, k, seed = 65536, 16384, 8, 2, 1, 61
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    for i in range(0, T, 4096):
        x[i:i + 4096] = torch.randn(4096, d, generator=g, device="cuda")
    logits = W.normal((T, E), 1.0, seed, W.S_ROUTER, "f32")
    w1 = W.normal((E, d, ff_i), W.WEIGHT_STD, seed, W.S_MW1)
    w_up = W.normal((E, d, ff_i), W.WEIGHT_STD, seed, W.S_MWUP)
    w2 = W.normal((E, ff_i, d), W.WEIGHT_STD, seed, W.S_MW2)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    tp.tp_moe_route(cuda(logits), k, idx, gate)
    y = torch.full((T, d), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(tp.tp_moe_shard_fwd_workspace(T, d, ff_i, E, k))
    tp.tp_moe_shard_fwd(x, idx, gate, cuda(w1), cuda(w_up), cuda(w2), y, ws)
    rows = W.row_subset(T, 32, seed)
    ridx, rgate = O.moe_route(logits[rows], k)
    assert torch.equal(idx[rows].cpu().long(), torch.from_numpy(ridx))
    ref = O.moe_shard_fwd(x[rows].cpu(), ridx, rgate, w1, w_up, w2)
    assert_close(y[rows], ref, BF16_TOL, "moe rows, gathered x")
    del ws, x
    torch.cuda.empty_cache()


def test_moe_dropped_slots_contribute_nothing():
    """Slots whose expert index lies outside [0, E) are skipped: the result
    equals the block with those slots' gates set to zero."""
    wl = W.MoeWorkload("moe_drop", T=150, d=128, ff=64, E=8, k=3, p=1, seed=62)
    t = W.moe_rank_inputs(wl)
    ridx, rgate = O.moe_route(t["logits"], wl.k)
    bad = np.zeros_like(ridx, dtype=bool)
    bad[::7, 1] = True
    bad[3::11, 2] = True
    idx_in = ridx.copy()
    idx_in[::7, 1] = -1
    idx_in[3::11, 2] = wl.E
    idx = torch.from_numpy(idx_in.astype(np.int32)).cuda()
    gate = torch.from_numpy(rgate.astype(np.float32)).cuda()
    y = torch.full((wl.T, wl.d), 7.0, dtype=torch.float32, device="cuda")
    ws = tp.new_workspace(tp.tp_moe_shard_fwd_workspace(wl.T, wl.d, wl.ff_i, wl.E, wl.k))
    tp.tp_moe_shard_fwd(cuda(t["x"]), idx, gate, cuda(t["w1"]), cuda(t["w_up"]), cuda(t["w2"]), y, ws)
    g_ref = np.where(bad, 0.0, gate.cpu().numpy().astype(np.float64))
    ref = O.moe_shard_fwd(t["x"], np.where(bad, 0, ridx), g_ref, t["w1"], t["w_up"], t["w2"])
    assert_close(y, ref, BF16_TOL, "moe with dropped slots")


@pytest.mark.parametrize("T,d,ff_i,E,k", [(40, 64, 8, 1024, 16), (33, 128, 16, 1000, 16), (5, 64, 8, 65, 1)])
def test_moe_at_the_expert_and_slot_limits(T, d, ff_i, E, k):
    """E up to 1024 and k = 16: every register slot of the routing waves, the
    planning scan across all 16 waves of its workgroup, more tiles than its
    threads, and an E that is not a multiple of 64."""
    wl = W.MoeWorkload("moe_limits", T=T, d=d, ff=ff_i, E=E, k=k, p=1, seed=63 + E)
    t = W.moe_rank_inputs(wl)
    idx, gate, y = moe_run(t, k, torch.float32)
    ridx, rgate = O.moe_route(t["logits"], k)
    assert torch.equal(idx.cpu().long(), torch.from_numpy(ridx)), "routing decisions"
    np.testing.assert_allclose(gate.cpu().numpy(), rgate, rtol=1e-5, atol=1e-6)
    ref = O.moe_shard_fwd(t["x"], ridx, rgate, t["w1"], t["w_up"], t["w2"])
    assert_close(y, ref, BF16_TOL, "moe block at the limits")


def test_moe_graph_replay():
    """Routing and the MoE block captured in one HIP graph: several replays,
    with an eager MoE call on the graph's workspace between them, each
    bit-identical to the eager result (the grouping state is rebuilt by every
    call and nothing issues a memset)."""
    wl = W.MoeWorkload("moe_graph", T=300, d=256, ff=64, E=16, k=4, p=1, seed=64)
    t = W.moe_rank_inputs(wl)
    other = W.moe_rank_inputs(W.MoeWorkload("moe_graph_other", T=300, d=256, ff=64, E=16, k=4, p=1, seed=65))
    x, lg, w1, wu, w2 = (cuda(t[n]) for n in ("x", "logits", "w1", "w_up", "w2"))
    x2, lg2 = cuda(other["x"]), cuda(other["logits"])
    idx = torch.empty(wl.T, wl.k, dtype=torch.int32, device="cuda")
    gate = torch.empty(wl.T, wl.k, dtype=torch.float32, device="cuda")
    idx2, gate2 = torch.empty_like(idx), torch.empty_like(gate)
    y = torch.empty(wl.T, wl.d, dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y)
    ws = tp.new_workspace(tp.tp_moe_shard_fwd_workspace(wl.T, wl.d, wl.ff_i, wl.E, wl.k))

    def step():
        tp.tp_moe_route(lg, wl.k, idx, gate)
        tp.tp_moe_shard_fwd(x, idx, gate, w1, wu, w2, y, ws)

    step()
    torch.cuda.synchronize()
    y_eager = y.clone()
    ridx, rgate = O.moe_route(t["logits"], wl.k)
    assert_close(y_eager, O.moe_shard_fwd(t["x"], ridx, rgate, t["w1"], t["w_up"], t["w2"]), BF16_TOL, "eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r}"
        tp.tp_moe_route(lg2, wl.k, idx2, gate2)
        tp.tp_moe_shard_fwd(x2, idx2, gate2, w1, wu, w2, y2, ws)   # the graph's workspace, eagerly
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Packed weights (decode-sized calls): the layout is a pure rearrangement
# (bitwise against the same permutation built on the CPU); the linears and the
# feed-forward shard on packed weights against the oracle on ragged shapes
# (T up to 64, K not a multiple of 32 or 8, N not a multiple of 16, an odd
# number of 16-column strips) and at the 70B-class decode shape.
# ---------------------------------------------------------------------------
def packed_layout_cpu(w):
    """w (K, N) -> the packed bytes: chunk (k-block b, strip s) in block-major
    order, lane 16q + c, element j holds w[32b + 8q + j][16s + c] (zero padded)."""
    K, N = w.shape
    nkb, ns = (K + 31) // 32, (N + 15) // 16
    wp = torch.zeros(nkb * 32, ns * 16, dtype=w.dtype)
    wp[:K, :N] = w
    t = wp.reshape(nkb, 4, 8, ns, 16).permute(0, 3, 1, 4, 2).contiguous()  # b, s, q, c, j
    return t.reshape(-1).view(torch.uint8)


def pk(w):
    return tp.tp_pack_weight(cuda(w))


@pytest.mark.parametrize("K,N", [(1, 1), (5, 17), (100, 131), (33, 48), (8192, 1280), (3584, 8192)])
def test_pack_weight_is_the_fragment_permutation(K, N):
    w = W.normal((K, N), 1.0, 91, K + N)
    got = pk(w).cpu()
    assert got.numel() == tp.tp_packed_weight_bytes(K, N)
    assert torch.equal(got, packed_layout_cpu(w))


@pytest.mark.parametrize("act", ["none", "relu", "gelu", "swiglu"])
@pytest.mark.parametrize("T,K,N", [(1, 256, 48), (5, 1000, 200), (17, 100, 131), (33, 96, 16), (64, 520, 264)])
def test_col_linear_packed_ragged(act, T, K, N):
    seed = 3 * T + K + N
    x = W.normal((T, K), 1.0, seed, 1)
    w = W.normal((K, N), 0.05, seed, 2)
    wu = W.normal((K, N), 0.05, seed, 3) if act == "swiglu" else None
    b = W.normal((N,), 0.5, seed, 4) if act != "swiglu" else None
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(tp.tp_linear_packed_workspace(T, K, N, act))
    tp.tp_col_linear_packed(cuda(x), pk(w), None if wu is None else pk(wu), None if b is None else cuda(b), y, act,
                            K, N, ws)
    ref = O.col_linear(O.to64(x), O.to64(w), None if wu is None else O.to64(wu), None if b is None else O.to64(b), act)
    assert_close(y, ref, BF16_TOL, f"col_linear_packed {act}")


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("T,K,N", [(1, 64, 16), (9, 333, 72), (40, 1024, 8192), (64, 3584, 136)])
def test_row_linear_partial_packed(out, T, K, N):
    seed = 5 * T + K + N
    x = W.normal((T, K), 1.0, seed, 1)
    w = W.normal((K, N), 0.05, seed, 2)
    z = torch.full((T, N), 7.0, dtype=torch.bfloat16 if out == "bf16" else torch.float32, device="cuda")
    ws = tp.new_workspace(tp.tp_linear_packed_workspace(T, K, N))
    tp.tp_row_linear_partial_packed(cuda(x), pk(w), z, N, ws)
    assert_close(z, O.row_linear_partial(O.to64(x), O.to64(w)), BF16_TOL, "row partial packed")


def test_gqa_projections_packed_decode_T64_all_ranks():
    """The decode GQA projections on packed weights, as the bench times them
    (70B-class, T=64): QKV of ranks 0 and 7 (all 64 rows) against the oracle,
    and the eight ranks' packed o_proj partials summed against the unsharded
    product (and rank 0's partial alone)."""
    wl = W.GQA_DECODE
    t = W.gqa_unsharded(wl)
    x = cuda(t["x"])
    x64 = O.to64(t["x"])
    wsq = tp.new_workspace(tp.tp_linear_packed_workspace(wl.T, wl.h, 1280, "none"))
    parts = []
    for i in range(wl.p):
        qb, ql, kb, kl = tp.tp_gqa_shard(wl.n_q, wl.n_kv, wl.head_dim, wl.p, i)
        if i in (0, wl.p - 1):
            wqkv = torch.cat([t["wq"][:, qb:qb + ql], t["wk"][:, kb:kb + kl], t["wv"][:, kb:kb + kl]], 1).contiguous()
            qkv = torch.full((wl.T, 1280), 7.0, dtype=torch.bfloat16, device="cuda")
            tp.tp_col_linear_packed(x, pk(wqkv), None, None, qkv, "none", wl.h, 1280, wsq)
            ref = O.matmul(x64, O.gqa_local_qkv_weight(t["wq"], t["wk"], t["wv"], wl.n_q, wl.n_kv, wl.head_dim,
                                                       wl.p, i))
            assert_close(qkv, ref, BF16_TOL, f"packed qkv rank {i}")
        a_i = cuda(t["attn"][:, qb:qb + ql])
        wso = tp.new_workspace(tp.tp_linear_packed_workspace(wl.T, ql, wl.h))
        o_i = torch.full((wl.T, wl.h), 7.0, dtype=torch.bfloat16, device="cuda")
        tp.tp_row_linear_partial_packed(a_i, pk(t["wo"][qb:qb + ql, :].contiguous()), o_i, wl.h, wso)
        parts.append(o_i)
    y = torch.empty(wl.T, wl.h, dtype=torch.float32, device="cuda")
    tp.tp_partial_sum(parts, None, y)
    assert_close(y, O.matmul(O.to64(t["attn"]), O.to64(t["wo"])), BF16_TOL, "sum of packed o_proj partials")
    ref0 = O.matmul(O.to64(t["attn"][:, :1024]), O.to64(t["wo"][:1024]))
    assert_close(parts[0], ref0, BF16_TOL, "packed o_proj partial rank 0")


def packed_act_layout_cpu(x):
    """The packed activation layout written out: chunk (k-block b, 16-row tile
    i), lane l holds x[16i + l % 16, 32b + 8(l // 16) + j], j = 0..7, zero
    padded to whole tiles and k-blocks."""
    T, K = x.shape
    mt = 1 if T <= 16 else (2 if T <= 32 else 4)
    nkb = (K + 31) // 32
    xp = torch.zeros(mt * 16, nkb * 32, dtype=x.dtype)
    xp[:T, :K] = x
    return xp.reshape(mt, 16, nkb, 4, 8).permute(2, 0, 3, 1, 4).reshape(-1)


@pytest.mark.parametrize("T,K,offset", [(64, 8192, 0), (33, 1000, 0), (16, 72, 0), (17, 3584, 0), (5, 1003, 0),
                                        (64, 1024, 1)])
def test_pack_act_is_the_fragment_permutation(T, K, offset):
    """Whole and ragged tiles (T = 16, 17, 33, 64, 5), ragged k-blocks (K = 1000,
    1003) and rows 2 bytes off 16-byte alignment (the element-wise load path)."""
    x = W.normal((T, K), 1.0, 41 + T + K, 1)
    buf = torch.empty(T * K + offset, dtype=torch.bfloat16, device="cuda")
    xd = buf[offset:].view(T, K)     # contiguous; offset 1 leaves the rows 2 bytes off 16-byte alignment
    xd.copy_(cuda(x))
    want = packed_act_layout_cpu(x)
    got = tp.tp_pack_act(xd)
    assert torch.equal(got.view(torch.bfloat16).cpu()[: want.numel()], want)


def test_packed_split_k_qkv_decode_shape_is_deterministic():
    """The rank's fused QKV projection at T=64 (1280 columns: 80 strips, so K
    is split across workgroups): against the oracle, and bitwise run to run."""
    wl = W.GQA_DECODE
    t = W.gqa_unsharded(wl)
    qb, ql, kb, kl = tp.tp_gqa_shard(wl.n_q, wl.n_kv, wl.head_dim, wl.p, 5)
    wqkv = torch.cat([t["wq"][:, qb:qb + ql], t["wk"][:, kb:kb + kl], t["wv"][:, kb:kb + kl]], 1).contiguous()
    x = cuda(t["x"])
    wp = pk(wqkv)
    ws = tp.new_workspace(tp.tp_linear_packed_workspace(wl.T, wl.h, 1280, "none"))
    outs = []
    for _ in range(2):
        y = torch.empty(wl.T, 1280, dtype=torch.bfloat16, device="cuda")
        outs.append(tp.tp_col_linear_packed(x, wp, None, None, y, "none", wl.h, 1280, ws))
    assert_close(outs[0], O.matmul(O.to64(t["x"]), O.to64(wqkv)), BF16_TOL, "qkv packed")
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("act,T,d,ff_i,out", [("swiglu", 37, 1000, 264, "bf16"), ("gelu", 5, 512, 48, "bf16"),
                                               ("relu", 64, 256, 64, "f32"), ("none", 16, 136, 40, "bf16"),
                                               ("swiglu", 64, 2056, 1024, "f32")])
def test_mlp_shard_fwd_packed_ragged(act, T, d, ff_i, out):
    seed = 11 * T + d + ff_i
    x = W.normal((T, d), 1.0, seed, 1)
    w1 = W.normal((d, ff_i), 0.05, seed, 2)
    wu = W.normal((d, ff_i), 0.05, seed, 3) if act == "swiglu" else None
    w2 = W.normal((ff_i, d), 0.05, seed, 4)
    y = torch.full((T, d), 7.0, dtype=torch.bfloat16 if out == "bf16" else torch.float32, device="cuda")
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_packed_workspace(T, d, ff_i, act))
    # two calls on one workspace: nothing stale is read, the counters are left zero
    for rep in range(2):
        xr = x if rep == 0 else W.normal((T, d), 1.0, seed, 5)
        tp.tp_mlp_shard_fwd_packed(cuda(xr), pk(w1), None if wu is None else pk(wu), pk(w2), y, act, ff_i, ws)
        ref, _ = O.mlp_shard_fwd(O.to64(xr), O.to64(w1), None if wu is None else O.to64(wu), O.to64(w2), act)
        assert_close(y, ref, BF16_TOL, f"packed shard {act} call {rep}")


def test_mlp_shard_fwd_packed_decode_T64(rank0_weights):
    """The 70B-class decode shard (T=64, d=8192, ff_i=3584) on packed weights,
    every row, and bitwise run to run."""
    w = W.DECODE
    x = cuda(W.mlp_input(w))
    wt = rank0_weights
    w1p, wup, w2p = pk(wt["w1"]), pk(wt["w_up"]), pk(wt["w2"])
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_packed_workspace(w.T, w.d, w.ff_i, "swiglu"))
    ys = []
    for _ in range(2):
        y = torch.empty(w.T, w.d, dtype=torch.bfloat16, device="cuda")
        ys.append(tp.tp_mlp_shard_fwd_packed(x, w1p, wup, w2p, y, "swiglu", w.ff_i, ws))
    ref, _ = O.mlp_shard_fwd(O.to64(x), O.to64(wt["w1"]), O.to64(wt["w_up"]), O.to64(wt["w2"]), "swiglu")
    _, rf, rm = O.within(ys[0], ref)
    print(f"packed decode shard: rel_frob={rf:.3e} rel_max={rm:.3e}")
    assert_close(ys[0], ref, BF16_TOL, "y_0 decode, packed weights")
    assert torch.equal(ys[0], ys[1])


@pytest.mark.parametrize("act,out", [("swiglu", "bf16"), ("none", "f32"), ("gelu", "bf16")])
def test_linear_packed_gemm_on_prepacked_activations(act, out):
    """tp_pack_act + tp_linear_packed_gemm give bitwise what the one-call
    linears give (the same kernels run)."""
    T, K, N = 48, 776, 392
    x = cuda(W.normal((T, K), 1.0, 93, 1))
    w = pk(W.normal((K, N), 0.05, 93, 2))
    wu = pk(W.normal((K, N), 0.05, 93, 3)) if act == "swiglu" else None
    xp = tp.tp_pack_act(x)
    ws = tp.new_workspace(tp.tp_linear_packed_workspace(T, K, N, act))
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    y = tp.tp_linear_packed_gemm(xp, w, wu, None, torch.empty(T, N, dtype=odt, device="cuda"), act, K, ws)
    ref = torch.empty(T, N, dtype=odt, device="cuda")
    if act == "none":
        tp.tp_row_linear_partial_packed(x, w, ref, N, ws)
    else:
        tp.tp_col_linear_packed(x, w, wu, None, ref, act, K, N, ws)
    assert torch.equal(y, ref)


@pytest.mark.parametrize("T,K,act", [(64, 1024, "none"), (37, 1024, "swiglu"), (1, 32, "gelu"), (17, 544, "none"),
                                     (64, 992, "relu"), (48, 4096, "swiglu")])
def test_packed_linears_reading_row_major_x(T, K, act):
    """Launches that read few activation bytes in all (here N = 520: 33
    strip groups; K a multiple of 32) take the activation fragments straight
    from row-major x (rows past T as zeros) instead of a packed copy: against
    the oracle, and bitwise against the same GEMM on x packed beforehand (only
    the source of the fragments differs)."""
    N = 520
    seed = 7 * T + K
    x = W.normal((T, K), 1.0, seed, 1)
    w = W.normal((K, N), 0.05, seed, 2)
    wu = W.normal((K, N), 0.05, seed, 3) if act == "swiglu" else None
    wp, wup = pk(w), None if wu is None else pk(wu)
    ws = tp.new_workspace(tp.tp_linear_packed_workspace(T, K, N, act))
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    if act == "none":
        tp.tp_row_linear_partial_packed(cuda(x), wp, y, N, ws)
        ref = O.row_linear_partial(O.to64(x), O.to64(w))
    else:
        tp.tp_col_linear_packed(cuda(x), wp, wup, None, y, act, K, N, ws)
        ref = O.col_linear(O.to64(x), O.to64(w), None if wu is None else O.to64(wu), None, act)
    assert_close(y, ref, BF16_TOL, f"row-major x, T={T} K={K} {act}")
    via_packed = tp.tp_linear_packed_gemm(tp.tp_pack_act(cuda(x)), wp, wup, None,
                                          torch.empty(T, N, dtype=torch.bfloat16, device="cuda"), act, K, ws)
    assert torch.equal(y, via_packed)


@pytest.mark.parametrize("T,K,N,act,same_cuts", [(64, 8192, 3584, "swiglu", True), (37, 8192, 3584, "none", True),
                                                 (1, 8192, 8192, "gelu", True), (17, 4096, 8192, "relu", True),
                                                 (48, 3584, 8192, "none", True), (64, 8192, 1280, "none", False),
                                                 (64, 64, 200000, "none", False)])
def test_packed_linears_staging_row_major_x(T, K, N, act, same_cuts):
    """Launches that read many activation bytes (more than 48 MiB of
    fragments in all; K a multiple of 64, bf16 weights) load row-major x in
    whole 128-byte lines and turn them into fragments through LDS, with no
    packing launch: against the oracle, and against the same GEMM on x packed
    beforehand. The fragments are the same values, but the staged launch cuts
    K into whole 64-row k-pairs, and from 64 strips on it runs two strips per
    workgroup: where both launches cut K at the same k-blocks (every shape
    here but K=8192, N=1280, whose 80 strips run as 40 pairs x 6 K splits
    staged against 80 single strips x 3 splits packed) the two agree bit for
    bit; otherwise their fp32 sums differ in order only.
    K=64, N=200000: one k-pair for four waves (three stream nothing) over
    6250 workgroups; the packed launch spreads its two k-blocks over two
    waves, so there too only the order of the sums differs."""
    seed = 11 * T + K + N
    x = W.normal((T, K), 1.0, seed, 1)
    w = W.normal((K, N), 0.02, seed, 2)
    wu = W.normal((K, N), 0.02, seed, 3) if act == "swiglu" else None
    wp, wup = pk(w), None if wu is None else pk(wu)
    ws = tp.new_workspace(tp.tp_linear_packed_workspace(T, K, N, act))
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    if act == "none":
        tp.tp_row_linear_partial_packed(cuda(x), wp, y, N, ws)
        ref = O.row_linear_partial(O.to64(x), O.to64(w))
    else:
        tp.tp_col_linear_packed(cuda(x), wp, wup, None, y, act, K, N, ws)
        ref = O.col_linear(O.to64(x), O.to64(w), None if wu is None else O.to64(wu), None, act)
    assert_close(y, ref, BF16_TOL, f"staged row-major x, T={T} K={K} N={N} {act}")
    via_packed = tp.tp_linear_packed_gemm(tp.tp_pack_act(cuda(x)), wp, wup, None,
                                          torch.empty(T, N, dtype=torch.bfloat16, device="cuda"), act, K, ws)
    if same_cuts:
        assert torch.equal(y, via_packed)
    else:   # one bf16 rounding apart at most
        d = (y.float() - via_packed.float()).abs()
        assert (d <= 2.0 ** -7 * via_packed.float().abs() + 1e-4).all()


@pytest.mark.parametrize("T,K,act", [(64, 1024, "none"), (37, 1024, "swiglu"), (1, 64, "gelu"), (33, 4096, "none")])
def test_packed_fp8_linears_reading_row_major_x(T, K, act):
    """The packed fp8 linears take their bf16 activation fragments straight
    from row-major x when K is a multiple of 64 and the launch reads few
    activation bytes: against the oracle, and bitwise against the same call
    on an unaligned copy of x (which takes the packing launch)."""
    N = 520
    seed = 5 * T + K
    x = W.normal((T, K), 1.0, seed, 1)
    q = W.e4m3_codes((K, N), seed, 2)
    sc = W.column_scales(N, seed, 3)
    qu = W.e4m3_codes((K, N), seed, 4) if act == "swiglu" else None
    su = W.column_scales(N, seed, 5) if act == "swiglu" else None
    qp, qup = packed8(q), None if qu is None else packed8(qu)
    c, cu = cuda(sc), None if su is None else cuda(su)
    ws = tp.new_workspace(tp.tp_linear_packed_fp8_workspace(T, K, N, act))
    xa = cuda(x)
    buf = torch.empty(T * K + 1, dtype=torch.bfloat16, device="cuda")
    xu = buf[1:].view(T, K)      # 2 bytes past a 16-byte boundary: packed by a launch of its own
    xu.copy_(xa)
    outs = []
    for xin in (xa, xu):
        y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
        if act == "none":
            tp.tp_row_linear_partial_packed_fp8(xin, qp, c, y, N, ws)
        else:
            tp.tp_col_linear_packed_fp8(xin, qp, c, qup, cu, None, y, act, K, N, ws)
        outs.append(y)
    ref = (O.row_linear_partial_fp8(x, q, sc) if act == "none" else O.col_linear_fp8(x, q, sc, qu, su, None, act))
    assert_close(outs[0], ref, BF16_TOL, f"fp8 row-major x, T={T} K={K} {act}")
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("act,K", [("swiglu", 2048), ("gelu", 1000), ("swiglu", 1000)])
def test_decode_size_linears_without_a_workspace(act, K):
    """Decode-size calls made without a workspace run unsplit (slower,
    documented in the header): K=1000 on the streaming kernel with the
    activation slice in LDS, K=2048 (slice too large) on the register-staged
    tiled kernel; the results meet the oracle's tolerance either way."""
    T, N = 40, 1000
    x = W.normal((T, K), 1.0, 95, 1)
    w = W.normal((K, N), 0.05, 95, 2)
    wu = W.normal((K, N), 0.05, 95, 3) if act == "swiglu" else None
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    tp.tp_col_linear(cuda(x), cuda(w), None if wu is None else cuda(wu), None, y, act)
    ref = O.col_linear(O.to64(x), O.to64(w), None if wu is None else O.to64(wu), None, act)
    assert_close(y, ref, BF16_TOL, "col linear, no workspace")
    z = torch.full((T, 1024), 7.0, dtype=torch.float32, device="cuda")
    h = W.normal((T, N), 1.0, 95, 4)
    w2 = W.normal((N, 1024), 0.05, 95, 5)
    tp.tp_row_linear_partial(cuda(h), cuda(w2), z)
    assert_close(z, O.row_linear_partial(O.to64(h), O.to64(w2)), BF16_TOL, "row partial, no workspace")


def _at_offset(t, offset_bytes):
    """A device copy of t whose data starts `offset_bytes` past a 4 KiB-aligned base."""
    n = t.numel() * t.element_size()
    buf = torch.empty(n + 8192, dtype=torch.uint8, device="cuda")
    base = (-buf.data_ptr()) % 4096
    view = buf[base + offset_bytes: base + offset_bytes + n].view(t.dtype).view(t.shape)
    view.copy_(t.to("cuda"))
    return view, buf


def test_weight_address_class_changes_only_the_last_bits():
    """The row-major decode kernel gives the column strips whose weight bytes
    fall in one address class (bits 7-9 equal to 3) extra K splits, so the
    summation order, and with it the rounding, follows the weight buffer's
    address: the same inputs at two addresses of different classes agree to
    fp32 rounding and both meet the oracle's tolerance, but need not be
    bitwise equal.  The packed-weight path splits by shape only: its results
    are bitwise independent of the address."""
    T, d, ff = 64, 4096, 1792
    x = W.normal((T, d), 1.0, 97, 1)
    w1 = W.normal((d, ff), 0.02, 97, 2)
    wu = W.normal((d, ff), 0.02, 97, 3)
    w2 = W.normal((ff, d), 0.02, 97, 4)
    ref, _ = O.mlp_shard_fwd(O.to64(x), O.to64(w1), O.to64(wu), O.to64(w2), "swiglu")
    xs = cuda(x)
    outs, outs_packed, keep = [], [], []
    for off in (0, 3 * 128):   # weight pointer bits 7-9: class 0, then class 3
        a1, b1 = _at_offset(w1, off)
        au, bu = _at_offset(wu, off)
        a2, b2 = _at_offset(w2, off)
        keep += [b1, bu, b2]
        assert (a1.data_ptr() >> 7) & 7 == off // 128
        y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
        ws = tp.new_workspace(tp.tp_mlp_shard_fwd_workspace(T, d, ff, tp.TP_BF16, "swiglu"))
        tp.tp_mlp_shard_fwd(xs, a1, au, a2, y, "swiglu", ws)
        assert_close(y, ref, BF16_TOL, f"row-major weights at offset {off}")
        outs.append(y)
        pw = [_at_offset(tp.tp_pack_weight(a).cpu(), off) for a in (a1, au, a2)]
        keep += [b for _, b in pw]
        yp = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
        wsp = tp.new_workspace(tp.tp_mlp_shard_fwd_packed_workspace(T, d, ff, "swiglu"))
        tp.tp_mlp_shard_fwd_packed(xs, pw[0][0], pw[1][0], pw[2][0], yp, "swiglu", ff, wsp)
        assert_close(yp, ref, BF16_TOL, f"packed weights at offset {off}")
        outs_packed.append(yp)
    _, rf, _ = O.within(outs[1], outs[0])
    assert rf < 2e-3, rf           # bf16 outputs of two fp32 summation orders
    assert torch.equal(outs_packed[0], outs_packed[1])


@pytest.mark.parametrize("K", [4096, 4095])
def test_tiled_split_k_when_tiles_are_few(K):
    """A GEMM with at most one 128x128 tile per CU and a long K is split in
    two across workgroups (aligned operands: the pipelined kernel with one
    arrival ticket per workgroup; K = 4095: the register-staged kernel with one
    per wave); ragged N, bias + GELU epilogue, and bitwise run to run."""
    T, N = 200, 520
    x = W.normal((T, K), 1.0, 99, 1)
    w = W.normal((K, N), 0.02, 99, 2)
    b = W.normal((N,), 0.5, 99, 3)
    ws = tp.new_workspace(tp.tp_col_linear_workspace(T, K, N, tp.TP_BF16, "gelu"))
    assert ws is not None   # the split needs a workspace
    outs = []
    for _ in range(2):
        y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
        outs.append(tp.tp_col_linear(cuda(x), cuda(w), None, cuda(b), y, "gelu", ws))
    ref = O.col_linear(O.to64(x), O.to64(w), None, O.to64(b), "gelu")
    assert_close(outs[0], ref, BF16_TOL, f"split-K tiled GEMM, K={K}")
    assert torch.equal(outs[0], outs[1])
