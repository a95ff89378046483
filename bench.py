#!/usr/bin/env python3
"""Benchmark: one tensor-parallel rank's SwiGLU MLP shard on one MI355X.

A step is one rank's shard forward of a 70B-class SwiGLU MLP at decode size
(T=64 tokens, d=8192, ff_i=28672/8=3584, bf16): the activations rearranged
into the matrix cores' operand order, the column-parallel gate/up GEMM with
the SwiGLU epilogue fused, then the row-parallel down GEMM writing the
full-shape partial y_i.  The weights are read in the packed layout they are
rearranged into once, when a shard is loaded (tp_pack_weight; outside the
timed region, like the fp8 strips); the same step on (in, out) row-major
weights is a row.  Inputs are resident in HBM before timing starts; three
distinct weight sets (528 MB) rotate so the 256 MB Infinity Cache cannot serve
them.  The headline value is algorithmic bytes (weights + x + y_i) per second.

The same JSON line carries:
  roofline      the dominant kernel (the fused gate/up GEMM on packed weights,
                reading row-major x as the step does) launched alone and timed
                with HIP events on its stream: algorithmic bytes / launch time
                vs 8 TB/s;
  rows          the other hot-path rows: prefill shard (T=4096), GQA
                projections (T=4096 and 64), the shard backward (T=2048,
                d=4096, ff_i=1792), the fp32 sum of partials and the
                sequence-parallel boundary (a rank's rows of the sum +
                residual, then RMSNorm);
  cpu_baseline  the fp64 oracle computing the same decode step on the host.

Rows named context_* time something that is not this library (the vendor
GEMM, torch.matmul on hipBLASLt, on the prefill shapes) for comparison.

    python bench.py [--steps K] [--warmup W] [--rows all|none|prefill,gqa,bwd,sum,calib]

--rows calib adds a plain device-to-device copy of 117,440,512 bytes (five
launches), the known-size kernel that scales the FETCH_SIZE / WRITE_SIZE
counters of the same profiling run.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "per-rank sharded MLP TFLOP/s (prefill) & GB/s (decode), % of MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6    # MI355X dense bf16 MFMA (256 CUs x 4096 flop/clk x 2.4 GHz)

# HBM bytes per launch of the roofline kernel (the packed gate/up GEMM) from
# rocprofv3 PMC (FETCH_SIZE + WRITE_SIZE, each scaled by what the same counter
# reads for a plain copy of known size: run with --rows calib), keyed by the
# sha256 of the kernel's source files when the counters were taken; reported
# as null once that source has changed.
TRAFFIC_GATE_UP = 129_663_418
TRAFFIC_SOURCE_SHA256 = "642d2cc9f301f10093845a4163d3d9c80585ba8392914460f01361e8f0fb94f3"
KERNEL_SOURCES = [os.path.join(ROOT, "tensor_sharded_transformer_amd", "csrc", f)
                  for f in ("gemm_packed.hip", "tp_device.h", "tp_kernels.h")]


def source_sha256(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_gpu(fn, steps: int, warmup: int, repeats: int = 3, warm_s: float = 0.05) -> float:
    """Milliseconds per call of fn(i), timed with HIP events on the current
    stream (the stream the library launches on): `warmup` untimed calls and
    at least `warm_s` seconds of untimed calls (the clocks settle under load),
    then the best of `repeats` timed runs of `steps` calls."""
    import torch
    # one call counter throughout: a timed run resumes the rotation over
    # weight sets where the previous calls left it, so it never starts on a
    # set still held in the Infinity Cache
    i = 0
    for _ in range(warmup):
        fn(i)
        i += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    best = float("inf")
    for _ in range(repeats):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(s)
        for _ in range(steps):
            fn(i)
            i += 1
        end.record(s)
        torch.cuda.synchronize()
        best = min(best, start.elapsed_time(end) / steps)
    return best


def gpu_normal(shape, std, seed, dev):
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * std).to(torch.bfloat16)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--rows", default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's shard only; --gpus {args.gpus} is not supported "
              "(the per-rank work is independent of the group size; run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import workloads as W
    import tensor_sharded_transformer_amd as tp

    dev = "cuda:0"
    torch.cuda.set_device(0)
    tp.load()

    # ---------------- headline: decode shard step -------------------------------
    wl = W.DECODE
    T, d, ff_i = wl.T, wl.d, wl.ff_i
    R = 3
    log(f"bench: generating {R} weight sets for {wl.name} ...")
    sets = []
    for r in range(R):
        wt = W.mlp_rank_weights(wl, r)
        sets.append({k: v.to(dev) for k, v in wt.items()})
        del wt
    x = W.mlp_input(wl).to(dev)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    # the packed layout of every weight set, made once (a weight-load-time step)
    psets = [{k: tp.tp_pack_weight(v) for k, v in st.items()} for st in sets]
    torch.cuda.synchronize()
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_packed_workspace(T, d, ff_i, "swiglu"), dev)

    def step(i):
        s = psets[i % R]
        tp.tp_mlp_shard_fwd_packed(x, s["w1"], s["w_up"], s["w2"], y, "swiglu", ff_i, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(args.warmup, args.warmup + args.steps):   # the rotation continues from the warmup
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    bytes_step = (3 * d * ff_i + 2 * T * d) * 2     # weights + x + y_i, bf16
    value = bytes_step / (ms * 1e-3) / 1e9
    log(f"bench: decode shard {ms * 1e3:.1f} us/step -> {value:.0f} GB/s ({value / HBM_PEAK_GBS:.1%} of HBM); "
        f"wall {wall:.3f}s")

    # ---------------- roofline: the fused gate/up GEMM kernel alone -----------------
    # one launch per call: the packed GEMM reading row-major x, as in the step
    h = torch.empty(T, ff_i, dtype=torch.bfloat16, device=dev)
    ws_c = tp.new_workspace(tp.tp_linear_packed_workspace(T, d, ff_i, "swiglu"), dev)

    def gate_up(i):
        s = psets[i % R]
        tp.tp_col_linear_packed(x, s["w1"], s["w_up"], None, h, "swiglu", d, ff_i, ws_c)

    k_ms = time_gpu(gate_up, args.steps, args.warmup)
    k_bytes = (2 * d * ff_i + T * d + T * ff_i) * 2
    k_gbs = k_bytes / (k_ms * 1e-3) / 1e9
    fresh = TRAFFIC_SOURCE_SHA256 is not None and source_sha256(KERNEL_SOURCES) == TRAFFIC_SOURCE_SHA256
    roofline = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": TRAFFIC_GATE_UP if fresh else None,
                "kernel": "packed_gemm_kernel<4, 2, true, 2, unsigned short, false, 2, 8>: fused gate/up weight-streaming "
                          "GEMM with the SwiGLU epilogue, packed weights, row-major x staged through LDS",
                "algorithmic_bytes": k_bytes, "avg_launch_us": round(k_ms * 1e3, 2)}
    log(f"bench: gate/up GEMM {k_ms * 1e3:.1f} us -> {k_gbs:.0f} GB/s")

    rows = {}
    want = set(["decode", "prefill", "gqa", "attn", "bwd", "fp8", "moe", "sum"]) if args.rows == "all" else (
        set() if args.rows == "none" else set(args.rows.split(",")))
    steps_r = max(10, args.steps // 2)

    if "decode" in want:
        # the down GEMM alone (packed h, packed W2) and the same step on row-major weights
        hp = torch.empty(tp.tp_packed_act_bytes(T, ff_i), dtype=torch.uint8, device=dev)
        tp.tp_pack_act(h, hp)
        ws_d = tp.new_workspace(tp.tp_linear_packed_workspace(T, ff_i, d), dev)
        # alone, three W2 sets (176 MB) would sit in the 256 MB Infinity Cache:
        # rotate six distinct buffers (352 MB) so the GEMM streams from HBM
        w2s = [psets[r]["w2"] for r in range(R)] + [psets[r]["w2"].clone() for r in range(R)]
        t_ = time_gpu(lambda i: tp.tp_linear_packed_gemm(hp, w2s[i % len(w2s)], None, None, y, "none", ff_i, ws_d),
                      args.steps, 200)
        b_ = (d * ff_i + T * ff_i + T * d) * 2
        rows["decode_down_gemm_packed_T64"] = {"us": round(t_ * 1e3, 2), "GB/s": round(b_ / t_ / 1e6, 1),
                                               "frac_hbm": round(b_ / t_ / 1e6 / HBM_PEAK_GBS, 4),
                                               "algorithmic_bytes": b_}
        ws_r = tp.new_workspace(tp.tp_mlp_shard_fwd_workspace(T, d, ff_i, tp.TP_BF16, "swiglu"), dev)
        t_ = time_gpu(lambda i: tp.tp_mlp_shard_fwd(x, sets[i % R]["w1"], sets[i % R]["w_up"], sets[i % R]["w2"], y,
                                                    "swiglu", ws_r), args.steps, 200)
        rows["decode_shard_T64_rowmajor_weights"] = {"us": round(t_ * 1e3, 2),
                                                     "GB/s": round(bytes_step / t_ / 1e6, 1),
                                                     "frac_hbm": round(bytes_step / t_ / 1e6 / HBM_PEAK_GBS, 4)}
        del hp, ws_d, ws_r, w2s

    if "calib" in want:
        src = torch.ones(8192, 7168, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        t_ = time_gpu(lambda i: dst.copy_(src), 5, 0)
        rows["calib_copy_117440512B"] = {"us": round(t_ * 1e3, 2),
                                         "GB/s_rd+wr": round(2 * src.numel() * 2 / t_ / 1e6, 1)}
        del src, dst

    if "moe" in want:
        # one rank's share of a Qwen3-MoE-class layer (128 experts, top-8, hidden
        # 2048, expert intermediate 768 / 8 ranks) at T=4096: routing, grouping,
        # the two grouped GEMMs and the combine
        wm = W.MOE_PREFILL
        gm = torch.Generator(device=dev)
        gm.manual_seed(51)
        rn = lambda *shp, sd=1.0, dt=torch.bfloat16: (torch.randn(*shp, generator=gm, device=dev) * sd).to(dt)
        xm, lm = rn(wm.T, wm.d), rn(wm.T, wm.E, dt=torch.float32)
        w1m, wum, w2m = rn(wm.E, wm.d, wm.ff_i, sd=0.02), rn(wm.E, wm.d, wm.ff_i, sd=0.02), rn(wm.E, wm.ff_i, wm.d, sd=0.02)
        idxm = torch.empty(wm.T, wm.k, dtype=torch.int32, device=dev)
        gatem = torch.empty(wm.T, wm.k, dtype=torch.float32, device=dev)
        ym = torch.empty(wm.T, wm.d, dtype=torch.bfloat16, device=dev)
        wsm = tp.new_workspace(tp.tp_moe_shard_fwd_workspace(wm.T, wm.d, wm.ff_i, wm.E, wm.k), dev)

        def moe_step(i):
            tp.tp_moe_route(lm, wm.k, idxm, gatem)
            tp.tp_moe_shard_fwd(xm, idxm, gatem, w1m, wum, w2m, ym, wsm)

        t_ = time_gpu(moe_step, steps_r, 3)
        fl = wm.T * wm.k * 6 * wm.d * wm.ff_i
        rows["moe_qwen3_class_rank_T4096"] = {"us": round(t_ * 1e3, 1), "TFLOP/s": round(fl / t_ / 1e9, 1),
                                              "frac_mfma": round(fl / t_ / 1e9 / BF16_PEAK_TFLOPS, 4)}
        del xm, lm, w1m, wum, w2m, idxm, gatem, ym, wsm

    if "fp8" in want:
        # the decode shard step with fp8 (E4M3) weights and per-column scales:
        # gate/up column-parallel GEMM + SwiGLU, then the down row-parallel partial;
        # codes packed once in MFMA fragment order (the row), and the same step on
        # 64-column strip-major codes (a row of its own)
        R8 = 4   # 4 x 88 MB of weights rotate, more than the 256 MB Infinity Cache holds
        g8 = torch.Generator(device=dev)
        raw8 = []
        for r in range(R8):
            g8.manual_seed(100 + r)
            codes = lambda shp: (torch.randn(*shp, generator=g8, device=dev) * 64.0).clamp_(-448, 448).to(
                torch.float8_e4m3fn).view(torch.uint8)
            sc = lambda n: (0.5 + torch.rand(n, generator=g8, device=dev)) * (0.02 / 64.0)
            raw8.append((codes((d, ff_i)), sc(ff_i), codes((d, ff_i)), sc(ff_i), codes((ff_i, d)), sc(d)))
        b8 = 3 * d * ff_i + (2 * ff_i + d) * 4 + 2 * T * d * 2
        y8 = torch.empty(T, d, dtype=torch.bfloat16, device=dev)

        sets8 = [(tp.tp_pack_weight_fp8(qg), sg, tp.tp_pack_weight_fp8(qu), su, tp.tp_pack_weight_fp8(qd), sd)
                 for qg, sg, qu, su, qd, sd in raw8]
        ws8 = tp.new_workspace(tp.tp_mlp_shard_fwd_packed_fp8_workspace(T, d, ff_i, "swiglu"), dev)

        def step8(i):
            qg, sg, qu, su, qd, sd = sets8[i % R8]
            tp.tp_mlp_shard_fwd_packed_fp8(x, qg, sg, qu, su, qd, sd, y8, "swiglu", ff_i, ws8)

        t_ = time_gpu(step8, steps_r, 3)
        rows["decode_fp8_weights_shard_T64"] = {"us": round(t_ * 1e3, 2), "GB/s": round(b8 / t_ / 1e6, 1),
                                                "frac_hbm": round(b8 / t_ / 1e6 / HBM_PEAK_GBS, 4),
                                                "algorithmic_bytes": b8}
        del sets8, ws8

        def strips(q):   # the strip-major order the strip-major fp8 linears read
            return tp.tp_fp8_pack_strips(q, torch.empty_like(q))
        sets8 = [(strips(qg), sg, strips(qu), su, strips(qd), sd) for qg, sg, qu, su, qd, sd in raw8]
        ws8 = tp.new_workspace(tp.tp_mlp_shard_fwd_fp8_workspace(T, d, ff_i, "swiglu"), dev)

        def step8s(i):
            qg, sg, qu, su, qd, sd = sets8[i % R8]
            tp.tp_mlp_shard_fwd_fp8(x, qg, sg, qu, su, qd, sd, y8, "swiglu", ws8)

        t_ = time_gpu(step8s, steps_r, 3)
        rows["decode_fp8_weights_shard_T64_stripmajor"] = {"us": round(t_ * 1e3, 2), "GB/s": round(b8 / t_ / 1e6, 1),
                                                           "frac_hbm": round(b8 / t_ / 1e6 / HBM_PEAK_GBS, 4)}
        del sets8, y8, ws8, raw8

    if "sum" in want:
        # every sum row rotates more partials than the 256 MB Infinity Cache holds
        NS_ = 40   # 40 x 8 MB at decode size
        parts = [torch.randn(T, d, device=dev).to(torch.bfloat16) for _ in range(8)]
        pbuf = [[t.clone() for t in parts] for _ in range(NS_)]
        yf = torch.empty(T, d, dtype=torch.float32, device=dev)
        # a few-microsecond kernel: call the C ABI with prepared pointer arrays
        # so host-side argument marshalling does not leave the GPU idle
        import ctypes
        lib = tp.load()
        parrs = [(ctypes.c_void_p * 8)(*[t.data_ptr() for t in ps_]) for ps_ in pbuf]
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        yptr = ctypes.c_void_p(yf.data_ptr())
        t_ = time_gpu(lambda i: lib.tp_partial_sum(parrs[i % NS_], 8, None, yptr, T, d, tp.TP_BF16, tp.TP_F32, stream),
                      steps_r, 5)
        del pbuf, parrs
        b_ = (8 * T * d * 2 + T * d * 4)
        rows["sum_partials_decode_p8"] = {"us": round(t_ * 1e3, 2), "GB/s": round(b_ / t_ / 1e6, 1),
                                          "frac_hbm": round(b_ / t_ / 1e6 / HBM_PEAK_GBS, 4)}
        T5, d5 = W.BACKWARD.T, W.BACKWARD.d
        parts = [[torch.randn(T5, d5, device=dev).to(torch.bfloat16) for _ in range(8)] for _ in range(3)]
        yf = torch.empty(T5, d5, dtype=torch.float32, device=dev)
        t_ = time_gpu(lambda i: tp.tp_partial_sum(parts[i % 3], None, yf), steps_r, 5)
        b_ = (8 * T5 * d5 * 2 + T5 * d5 * 4)
        rows["sum_partials_dx_p8_T2048"] = {"us": round(t_ * 1e3, 2), "GB/s": round(b_ / t_ / 1e6, 1),
                                            "frac_hbm": round(b_ / t_ / 1e6 / HBM_PEAK_GBS, 4)}
        del parts
        # sequence-parallel boundary at prefill size: one rank's 512 rows of 8
        # partials (4096 x 8192 bf16) + residual, then RMSNorm; the rank rotates
        # over all 8 so the partials read (8 x 67 MB) exceed the Infinity Cache
        Ts, ps = W.PREFILL.T, 8
        parts = [torch.randn(Ts, d, device=dev).to(torch.bfloat16) for _ in range(ps)]
        res = torch.randn(Ts // ps, d, device=dev).to(torch.bfloat16)
        nw = torch.randn(d, device=dev).to(torch.bfloat16)
        r_out = torch.empty_like(res)
        yn = torch.empty_like(res)
        t_ = time_gpu(lambda i: tp.tp_rs_residual_rmsnorm(parts, i % ps, None, res, nw, 1e-5, r_out, yn), steps_r, 5)
        b_ = (ps * (Ts // ps) * d + 3 * (Ts // ps) * d + d) * 2
        rows["sp_rs_residual_rmsnorm_T4096_p8"] = {"us": round(t_ * 1e3, 2), "GB/s": round(b_ / t_ / 1e6, 1),
                                                   "frac_hbm": round(b_ / t_ / 1e6 / HBM_PEAK_GBS, 4)}
        del parts, res, r_out, yn

    if "prefill" in want:
        xp = W.mlp_input(W.PREFILL).to(dev)
        Tp = W.PREFILL.T
        yp = torch.empty(Tp, d, dtype=torch.bfloat16, device=dev)
        wsp = tp.new_workspace(tp.tp_mlp_shard_fwd_workspace(Tp, d, ff_i, tp.TP_BF16, "swiglu"), dev)
        t_ = time_gpu(lambda i: tp.tp_mlp_shard_fwd(xp, sets[i % R]["w1"], sets[i % R]["w_up"], sets[i % R]["w2"],
                                                    yp, "swiglu", wsp), steps_r, 3)
        fl = 3 * 2 * Tp * d * ff_i
        rows["prefill_mlp_shard_T4096"] = {"us": round(t_ * 1e3, 1), "TFLOP/s": round(fl / t_ / 1e9, 1),
                                           "frac_mfma": round(fl / t_ / 1e9 / BF16_PEAK_TFLOPS, 4)}
        hp = torch.empty(Tp, ff_i, dtype=torch.bfloat16, device=dev)
        # the same rotating weight sets as the shard (one set would stay in the Infinity Cache)
        t_ = time_gpu(lambda i: tp.tp_col_linear(xp, sets[i % R]["w1"], sets[i % R]["w_up"], None, hp, "swiglu"),
                      steps_r, 3)
        fl = 2 * 2 * Tp * d * ff_i
        rows["prefill_gate_up_gemm"] = {"us": round(t_ * 1e3, 1), "TFLOP/s": round(fl / t_ / 1e9, 1),
                                        "frac_mfma": round(fl / t_ / 1e9 / BF16_PEAK_TFLOPS, 4)}
        t_ = time_gpu(lambda i: tp.tp_row_linear_partial(hp, sets[i % R]["w2"], yp), steps_r, 3)
        fl = 2 * Tp * d * ff_i
        rows["prefill_down_gemm"] = {"us": round(t_ * 1e3, 1), "TFLOP/s": round(fl / t_ / 1e9, 1),
                                     "frac_mfma": round(fl / t_ / 1e9 / BF16_PEAK_TFLOPS, 4)}
        # context, not this library: the vendor GEMM (torch.matmul -> hipBLASLt)
        # on the same two shapes, without the activation epilogue
        wcat = torch.cat([sets[0]["w1"], sets[0]["w_up"]], dim=1)
        zc = torch.empty(Tp, 2 * ff_i, dtype=torch.bfloat16, device=dev)
        t_ = time_gpu(lambda i: torch.matmul(xp, wcat, out=zc), steps_r, 3)
        fl = 2 * 2 * Tp * d * ff_i
        rows["context_vendor_matmul_4096x8192x7168"] = {"us": round(t_ * 1e3, 1), "TFLOP/s": round(fl / t_ / 1e9, 1),
                                                        "frac_mfma": round(fl / t_ / 1e9 / BF16_PEAK_TFLOPS, 4)}
        t_ = time_gpu(lambda i: torch.matmul(hp, sets[0]["w2"], out=yp), steps_r, 3)
        fl = 2 * Tp * d * ff_i
        rows["context_vendor_matmul_4096x3584x8192"] = {"us": round(t_ * 1e3, 1), "TFLOP/s": round(fl / t_ / 1e9, 1),
                                                        "frac_mfma": round(fl / t_ / 1e9 / BF16_PEAK_TFLOPS, 4)}
        del xp, yp, wsp, hp, wcat, zc

    if "gqa" in want:
        h_, q_, o_ = 8192, 1280, 1024
        for Tg in (4096, 64):
            nset = 1 if Tg > 64 else 32    # >= 512 MB of weights rotate at decode size
            wqkv = gpu_normal((nset, h_, q_), 0.02, 11, dev)
            wo = gpu_normal((nset, o_, h_), 0.02, 12, dev)
            xg = gpu_normal((Tg, h_), 1.0, 13, dev)
            ag = gpu_normal((Tg, o_), 1.0, 14, dev)
            qkv = torch.empty(Tg, q_, dtype=torch.bfloat16, device=dev)
            og = torch.empty(Tg, h_, dtype=torch.bfloat16, device=dev)
            wsq = tp.new_workspace(tp.tp_col_linear_workspace(Tg, h_, q_, tp.TP_BF16, "none"), dev)
            wso = tp.new_workspace(tp.tp_row_linear_partial_workspace(Tg, o_, h_, tp.TP_BF16), dev)
            tq = time_gpu(lambda i: tp.tp_col_linear(xg, wqkv[i % nset], None, None, qkv, "none", wsq), steps_r, 3)
            to = time_gpu(lambda i: tp.tp_row_linear_partial(ag, wo[i % nset], og, wso), steps_r, 3)
            if Tg <= 64:
                # decode size: the same projections on (in, out) row-major weights are
                # rows of their own; the headline rows read packed weights
                bq = (h_ * q_ + Tg * h_ + Tg * q_) * 2
                bo = (o_ * h_ + Tg * o_ + Tg * h_) * 2
                rows[f"gqa_qkv_T{Tg}_rowmajor_weights"] = {"us": round(tq * 1e3, 2), "GB/s": round(bq / tq / 1e6, 1)}
                rows[f"gqa_oproj_T{Tg}_rowmajor_weights"] = {"us": round(to * 1e3, 2), "GB/s": round(bo / to / 1e6, 1)}
                pq = [tp.tp_pack_weight(wqkv[j]) for j in range(nset)]
                po = [tp.tp_pack_weight(wo[j]) for j in range(nset)]
                wsq = tp.new_workspace(tp.tp_linear_packed_workspace(Tg, h_, q_), dev)
                wso = tp.new_workspace(tp.tp_linear_packed_workspace(Tg, o_, h_), dev)
                tq = time_gpu(lambda i: tp.tp_col_linear_packed(xg, pq[i % nset], None, None, qkv, "none", h_, q_, wsq),
                              steps_r, 3)
                to = time_gpu(lambda i: tp.tp_row_linear_partial_packed(ag, po[i % nset], og, h_, wso), steps_r, 3)
                del pq, po
            if Tg > 64:
                fq, fo = 2 * Tg * h_ * q_, 2 * Tg * o_ * h_
                rows[f"gqa_qkv_T{Tg}"] = {"us": round(tq * 1e3, 1), "TFLOP/s": round(fq / tq / 1e9, 1),
                                          "frac_mfma": round(fq / tq / 1e9 / BF16_PEAK_TFLOPS, 4)}
                rows[f"gqa_oproj_T{Tg}"] = {"us": round(to * 1e3, 1), "TFLOP/s": round(fo / to / 1e9, 1),
                                            "frac_mfma": round(fo / to / 1e9 / BF16_PEAK_TFLOPS, 4)}
            else:
                bq = (h_ * q_ + Tg * h_ + Tg * q_) * 2
                bo = (o_ * h_ + Tg * o_ + Tg * h_) * 2
                rows[f"gqa_qkv_T{Tg}"] = {"us": round(tq * 1e3, 2), "GB/s": round(bq / tq / 1e6, 1),
                                          "frac_hbm": round(bq / tq / 1e6 / HBM_PEAK_GBS, 4)}
                rows[f"gqa_oproj_T{Tg}"] = {"us": round(to * 1e3, 2), "GB/s": round(bo / to / 1e6, 1),
                                            "frac_hbm": round(bo / to / 1e6 / HBM_PEAK_GBS, 4)}
            del wqkv, wo, xg, ag, qkv, og

    if "attn" in want:
        # local attention over one rank's 8 query heads and 1 KV head (70B-class GQA), T=4096
        wa = W.GQA_ATTN
        na_q, na_kv, hd_ = wa.n_q // wa.p, wa.n_kv // wa.p, wa.head_dim
        qkva = gpu_normal((wa.T, (na_q + 2 * na_kv) * hd_), 1.81, 41, dev)
        outa = torch.empty(wa.T, na_q * hd_, dtype=torch.bfloat16, device=dev)
        for causal in (True, False):
            t_ = time_gpu(lambda i: tp.tp_gqa_attention_fwd(qkva, outa, na_q, na_kv, hd_, causal, hd_ ** -0.5),
                          steps_r, 3)
            fl = 4 * (wa.T * (wa.T + 1) // 2 if causal else wa.T * wa.T) * hd_ * na_q
            rows[f"attention_{'causal' if causal else 'full'}_T4096_8q1kv"] = {
                "us": round(t_ * 1e3, 1), "TFLOP/s": round(fl / t_ / 1e9, 1),
                "frac_mfma": round(fl / t_ / 1e9 / BF16_PEAK_TFLOPS, 4)}
        del qkva, outa

    if "bwd" in want:
        wb = W.BACKWARD
        Tb, db, fb = wb.T, wb.d, wb.ff_i
        x5 = gpu_normal((Tb, db), 1.0, 21, dev)
        dy5 = gpu_normal((Tb, db), 1.0, 22, dev)
        w1 = gpu_normal((db, fb), 0.02, 23, dev)
        wu = gpu_normal((db, fb), 0.02, 24, dev)
        w2 = gpu_normal((fb, db), 0.02, 25, dev)
        sv = torch.empty(Tb, 2 * fb, dtype=torch.bfloat16, device=dev)
        y5 = torch.empty(Tb, db, dtype=torch.bfloat16, device=dev)
        wsf = tp.new_workspace(tp.tp_mlp_shard_fwd_workspace(Tb, db, fb, tp.TP_BF16, "swiglu"), dev)
        tp.tp_mlp_shard_fwd(x5, w1, wu, w2, y5, "swiglu", wsf, sv)
        wsb = tp.new_workspace(tp.tp_mlp_shard_bwd_workspace(Tb, db, fb, tp.TP_BF16, "swiglu"), dev)
        g1, gu, g2, gx = (torch.empty_like(t) for t in (w1, wu, w2, x5))
        t_ = time_gpu(lambda i: tp.tp_mlp_shard_bwd(x5, w1, wu, w2, sv, dy5, g1, gu, g2, gx, "swiglu", wsb),
                      steps_r, 3)
        fl = 4 * 3 * db * fb * Tb
        rows["bwd_mlp_shard_T2048"] = {"us": round(t_ * 1e3, 1), "TFLOP/s": round(fl / t_ / 1e9, 1),
                                       "frac_mfma": round(fl / t_ / 1e9 / BF16_PEAK_TFLOPS, 4)}

    if "bwd" in want:
        # backward of one rank's attention projections (70B-class GQA, T=4096):
        # QKV column-parallel (dW_qkv_i, dx_i partial) and o_proj row-parallel
        # (dW_o_i, dX_i), four GEMMs of 2*T*h*(1280 or 1024) each
        Ta, ha, qa, oa = 4096, 8192, 1280, 1024
        xa = gpu_normal((Ta, ha), 1.0, 31, dev)
        wqa = gpu_normal((ha, qa), 0.02, 32, dev)
        dqa = gpu_normal((Ta, qa), 1.0, 33, dev)
        aa = gpu_normal((Ta, oa), 1.0, 34, dev)
        woa = gpu_normal((oa, ha), 0.02, 35, dev)
        dya = gpu_normal((Ta, ha), 1.0, 36, dev)
        gq, gxa, go, gaa = (torch.empty_like(t) for t in (wqa, xa, woa, aa))
        wsa = tp.new_workspace(max(tp.tp_linear_shard_bwd_workspace(Ta, ha, qa, tp.TP_BF16),
                                   tp.tp_linear_shard_bwd_workspace(Ta, oa, ha, tp.TP_BF16)), dev)

        def attn_bwd(i):
            tp.tp_linear_shard_bwd(xa, wqa, dqa, gq, gxa, wsa)
            tp.tp_linear_shard_bwd(aa, woa, dya, go, gaa, wsa)

        t_ = time_gpu(attn_bwd, steps_r, 3)
        fl = 4 * Ta * ha * (qa + oa)
        rows["bwd_attn_proj_shard_T4096"] = {"us": round(t_ * 1e3, 1), "TFLOP/s": round(fl / t_ / 1e9, 1),
                                             "frac_mfma": round(fl / t_ / 1e9 / BF16_PEAK_TFLOPS, 4)}
        del xa, wqa, dqa, aa, woa, dya, gq, gxa, go, gaa, wsa

    # ---------------- CPU baseline: the fp64 oracle on the same decode step ------------
    cpu = None
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle as O
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
        except Exception:
            cores = os.cpu_count()
        wt = W.mlp_rank_weights(wl, 0)
        w64 = {k: O.to64(v) for k, v in wt.items()}
        x64 = O.to64(W.mlp_input(wl))
        reps, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and reps < 100000:
            c0 = time.perf_counter()
            O.mlp_shard_fwd(x64, w64["w1"], w64["w_up"], w64["w2"], "swiglu")
            t_cpu += time.perf_counter() - c0
            reps += 1
        per = t_cpu / reps
        cpu = {"value": round(bytes_step / per / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"full decode shard step (T=64, d=8192, ff_i=3584, fp64 numpy) x {reps} reps, "
                         f"{per:.3f} s/step",
               "ms_per_step": round(per * 1e3, 2)}
        log(f"bench: oracle {per * 1e3:.1f} ms/step on {cores} threads")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights, bf16)",
        "config": {"workload": wl.name, "T": T, "d": d, "ff_i": ff_i, "p": wl.p, "act": "swiglu",
                   "weight_sets_rotated": R, "algorithmic_bytes_per_step": bytes_step,
                   "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
