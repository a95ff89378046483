"""Thin ctypes binding over libtpshard.so (the C ABI in include/tpshard.h).

Argument marshalling only: every function below checks that the torch tensors
it is given have the shapes/dtypes the C entry point documents, passes their
device pointers and the current HIP stream, and raises ``TpError`` on a
non-zero status.  All arithmetic happens in the library's HIP kernels; there
is no fallback path: if the library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

from . import build as _build

TP_BF16, TP_F32 = 0, 1
NOALLOC_SCRATCH_BYTES = 32 << 20   # TP_NOALLOC_SCRATCH_BYTES in include/tpshard.h
ACT = {"none": 0, "relu": 1, "gelu": 2, "swiglu": 3}
STATUS = {0: "TP_OK", 1: "TP_ERR_NULL", 2: "TP_ERR_SHAPE", 3: "TP_ERR_DTYPE", 4: "TP_ERR_ACT",
          5: "TP_ERR_WORKSPACE", 6: "TP_ERR_UNSUPPORTED", 7: "TP_ERR_HIP"}


class TpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None

c_p = ctypes.c_void_p
c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/tpshard.h
SIGNATURES = {
    "tp_col_linear": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_int, c_p]),
    "tp_col_linear_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int, c_int]),
    "tp_act_inplace": (c_int, [c_p, c_p, c_i64, c_i64, c_int, c_int, c_p]),
    "tp_row_linear_partial": (c_int, [c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_int, c_p]),
    "tp_row_linear_partial_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int]),
    "tp_mlp_shard_fwd_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int, c_int]),
    "tp_mlp_shard_fwd": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_int, c_int,
                                 c_p]),
    "tp_mlp_shard_fwd_noalloc": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i64, c_int, c_int, c_int,
                                         c_p]),
    "tp_mlp_shard_bwd_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int, c_int]),
    "tp_mlp_shard_bwd": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64,
                                 c_int, c_int, c_p]),
    "tp_linear_shard_bwd_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int]),
    "tp_linear_shard_bwd": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_p]),
    "tp_gqa_attention_fwd": (c_int, [c_p, c_p, c_i64, c_int, c_int, c_int, c_int, ctypes.c_float, c_p]),
    "tp_linear_fp8_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int]),
    "tp_fp8_pack_strips": (c_int, [c_p, c_p, c_i64, c_i64, c_p]),
    "tp_moe_route": (c_int, [c_p, c_i64, c_int, c_int, c_p, c_p, c_p]),
    "tp_moe_shard_fwd_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int, c_int]),
    "tp_moe_shard_fwd": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_int,
                                 c_int, c_p]),
    "tp_mlp_shard_fwd_fp8_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int]),
    "tp_mlp_shard_fwd_fp8": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int,
                                     c_int, c_p]),
    "tp_col_linear_fp8": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_p]),
    "tp_row_linear_partial_fp8": (c_int, [c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_p]),
    "tp_packed_weight_bytes": (c_sz, [c_i64, c_i64]),
    "tp_pack_weight": (c_int, [c_p, c_p, c_i64, c_i64, c_p]),
    "tp_linear_packed_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int]),
    "tp_col_linear_packed": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_p]),
    "tp_row_linear_partial_packed": (c_int, [c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_p]),
    "tp_packed_act_bytes": (c_sz, [c_i64, c_i64]),
    "tp_pack_act": (c_int, [c_p, c_p, c_i64, c_i64, c_p]),
    "tp_linear_packed_gemm": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_int, c_p]),
    "tp_mlp_shard_fwd_packed_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int]),
    "tp_mlp_shard_fwd_packed": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_int, c_p]),
    "tp_packed_fp8_weight_bytes": (c_sz, [c_i64, c_i64]),
    "tp_pack_weight_fp8": (c_int, [c_p, c_p, c_i64, c_i64, c_p]),
    "tp_linear_packed_fp8_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int]),
    "tp_col_linear_packed_fp8": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int,
                                         c_p]),
    "tp_row_linear_partial_packed_fp8": (c_int, [c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64, c_int, c_p]),
    "tp_mlp_shard_fwd_packed_fp8_workspace": (c_sz, [c_i64, c_i64, c_i64, c_int]),
    "tp_mlp_shard_fwd_packed_fp8": (c_int, [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_i64, c_i64, c_i64,
                                            c_int, c_int, c_p]),
    "tp_partial_sum": (c_int, [ctypes.POINTER(c_p), c_int, c_p, c_p, c_i64, c_i64, c_int, c_int, c_p]),
    "tp_rs_residual_rmsnorm": (c_int, [ctypes.POINTER(c_p), c_int, c_int, c_p, c_p, c_p, ctypes.c_float, c_p, c_p,
                                       c_i64, c_i64, c_int, c_int, c_p]),
    "tp_workspace_init": (c_int, [c_p, c_sz, c_p]),
    "tp_shard_range": (c_int, [c_i64, c_int, c_int, ctypes.POINTER(c_i64), ctypes.POINTER(c_i64)]),
    "tp_gqa_shard": (c_int, [c_int, c_int, c_int, c_int, c_int, ctypes.POINTER(c_i64), ctypes.POINTER(c_i64),
                             ctypes.POINTER(c_i64), ctypes.POINTER(c_i64)]),
    "tp_status_string": (ctypes.c_char_p, [c_int]),
    "tp_last_error": (ctypes.c_char_p, []),
    "tp_abi_version": (c_int, []),
}


def lib_path() -> str:
    return _build.LIB


def load() -> ctypes.CDLL:
    """Loads the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m tensor_sharded_transformer_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise TpError(status, load().tp_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dtypes(dtype, **named) -> None:
    """Every given tensor must have `dtype` (the kernels read raw bytes)."""
    for nm, t in named.items():
        if t is not None and t.dtype != dtype:
            raise TypeError(f"{nm} must be {dtype}, got {t.dtype}")


def _shape(t: torch.Tensor, shape, name: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


# ---- workspaces ---------------------------------------------------------------
def new_workspace(nbytes: int, device=None) -> Optional[torch.Tensor]:
    """A zero-filled byte buffer (the library keeps its counter region zero)."""
    if nbytes == 0:
        return None
    return torch.zeros(int(nbytes), dtype=torch.uint8, device=device or "cuda")


# ---- host helpers ----------------------------------------------------------------
def tp_shard_range(n_total: int, p: int, i: int):
    b, ln = c_i64(), c_i64()
    _check(load().tp_shard_range(n_total, p, i, ctypes.byref(b), ctypes.byref(ln)))
    return b.value, ln.value


def tp_gqa_shard(n_q: int, n_kv: int, head_dim: int, p: int, i: int):
    out = [c_i64() for _ in range(4)]
    _check(load().tp_gqa_shard(n_q, n_kv, head_dim, p, i, *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)


def tp_abi_version() -> int:
    return load().tp_abi_version()


# ---- device entry points ----------------------------------------------------------
def tp_col_linear(x, w, w_up, bias, y, act: str = "none", ws: Optional[torch.Tensor] = None):
    T, K = x.shape
    N = w.shape[1]
    _shape(w, (K, N), "w")
    _shape(y, (T, N), "y")
    if w_up is not None:
        _shape(w_up, (K, N), "w_up")
    _dtypes(x.dtype, w=w, w_up=w_up, bias=bias, y=y)
    ws_bytes = 0 if ws is None else ws.numel()
    _check(load().tp_col_linear(_ptr(x), _ptr(w), _ptr(w_up), _ptr(bias), _ptr(y), _ptr(ws), ws_bytes, T, K, N,
                                _dt(x), ACT[act], _stream()))
    return y


def tp_col_linear_workspace(T: int, K: int, N_i: int, dtype: int, act: str) -> int:
    return load().tp_col_linear_workspace(T, K, N_i, dtype, ACT[act])


def tp_act_inplace(h, up, act: str):
    T, N = h.shape
    if up is not None:
        _shape(up, (T, N), "up")
    _dtypes(h.dtype, up=up)
    _check(load().tp_act_inplace(_ptr(h), _ptr(up), T, N, _dt(h), ACT[act], _stream()))
    return h


def tp_row_linear_partial(x_i, w_i, z_i, ws: Optional[torch.Tensor] = None):
    T, K = x_i.shape
    N = w_i.shape[1]
    _shape(w_i, (K, N), "w_i")
    _shape(z_i, (T, N), "z_i")
    _dtypes(x_i.dtype, w_i=w_i)
    ws_bytes = 0 if ws is None else ws.numel()
    _check(load().tp_row_linear_partial(_ptr(x_i), _ptr(w_i), _ptr(z_i), _ptr(ws), ws_bytes, T, K, N, _dt(x_i),
                                        _dt(z_i), _stream()))
    return z_i


def tp_row_linear_partial_workspace(T: int, K_i: int, N: int, dtype: int) -> int:
    return load().tp_row_linear_partial_workspace(T, K_i, N, dtype)


def tp_mlp_shard_fwd_workspace(T: int, d: int, ff_i: int, dtype: int, act: str) -> int:
    return load().tp_mlp_shard_fwd_workspace(T, d, ff_i, dtype, ACT[act])


def tp_mlp_shard_fwd(x, w1_i, w_up_i, w2_i, y_i, act: str, ws: torch.Tensor, saved=None):
    T, d = x.shape
    ff_i = w1_i.shape[1]
    _shape(w1_i, (d, ff_i), "w1_i")
    _shape(w2_i, (ff_i, d), "w2_i")
    _shape(y_i, (T, d), "y_i")
    if w_up_i is not None:
        _shape(w_up_i, (d, ff_i), "w_up_i")
    if saved is not None:
        _shape(saved, (T, (2 if act == "swiglu" else 1) * ff_i), "saved")
    _dtypes(x.dtype, w1_i=w1_i, w_up_i=w_up_i, w2_i=w2_i, saved=saved)
    _check(load().tp_mlp_shard_fwd(_ptr(x), _ptr(w1_i), _ptr(w_up_i), _ptr(w2_i), _ptr(y_i), _ptr(saved), _ptr(ws),
                                   ws.numel() if ws is not None else 0, T, d, ff_i, _dt(x), _dt(y_i), ACT[act],
                                   _stream()))
    return y_i


def tp_mlp_shard_fwd_noalloc(x, w1_i, w_up_i, w2_i, y_i, act: str, saved=None):
    """tp_mlp_shard_fwd with the library's static device scratch instead of a workspace."""
    T, d = x.shape
    ff_i = w1_i.shape[1]
    _shape(w1_i, (d, ff_i), "w1_i")
    _shape(w2_i, (ff_i, d), "w2_i")
    _shape(y_i, (T, d), "y_i")
    if w_up_i is not None:
        _shape(w_up_i, (d, ff_i), "w_up_i")
    if saved is not None:
        _shape(saved, (T, (2 if act == "swiglu" else 1) * ff_i), "saved")
    _dtypes(x.dtype, w1_i=w1_i, w_up_i=w_up_i, w2_i=w2_i, saved=saved)
    _check(load().tp_mlp_shard_fwd_noalloc(_ptr(x), _ptr(w1_i), _ptr(w_up_i), _ptr(w2_i), _ptr(y_i), _ptr(saved),
                                           T, d, ff_i, _dt(x), _dt(y_i), ACT[act], _stream()))
    return y_i


def tp_mlp_shard_bwd_workspace(T: int, d: int, ff_i: int, dtype: int, act: str) -> int:
    return load().tp_mlp_shard_bwd_workspace(T, d, ff_i, dtype, ACT[act])


def tp_mlp_shard_bwd(x, w1_i, w_up_i, w2_i, saved, dy, dw1_i, dw_up_i, dw2_i, dx_i, act: str, ws: torch.Tensor):
    T, d = x.shape
    ff_i = w1_i.shape[1]
    for t, shp, nm in ((dy, (T, d), "dy"), (dw1_i, (d, ff_i), "dw1_i"), (dw2_i, (ff_i, d), "dw2_i"),
                       (dx_i, (T, d), "dx_i"), (w2_i, (ff_i, d), "w2_i")):
        _shape(t, shp, nm)
    if dw_up_i is not None:
        _shape(dw_up_i, (d, ff_i), "dw_up_i")
    _dtypes(x.dtype, w1_i=w1_i, w_up_i=w_up_i, w2_i=w2_i, saved=saved, dy=dy, dw1_i=dw1_i, dw_up_i=dw_up_i,
            dw2_i=dw2_i, dx_i=dx_i)
    _check(load().tp_mlp_shard_bwd(_ptr(x), _ptr(w1_i), _ptr(w_up_i), _ptr(w2_i), _ptr(saved), _ptr(dy),
                                   _ptr(dw1_i), _ptr(dw_up_i), _ptr(dw2_i), _ptr(dx_i), _ptr(ws),
                                   ws.numel() if ws is not None else 0, T, d, ff_i, _dt(x), ACT[act], _stream()))


def tp_linear_shard_bwd_workspace(T: int, K: int, N: int, dtype: int) -> int:
    return load().tp_linear_shard_bwd_workspace(T, K, N, dtype)


def tp_linear_shard_bwd(x, w, dy, dw, dx, ws: Optional[torch.Tensor] = None):
    """dw = x^T dy and dx = dy w^T for one rank's shard of y = x w (either
    output may be None to skip it)."""
    K, N = (w if w is not None else dw).shape
    T = dy.shape[0]
    _shape(dy, (T, N), "dy")
    if x is not None:
        _shape(x, (T, K), "x")
    if dw is not None:
        _shape(dw, (K, N), "dw")
    if dx is not None:
        _shape(dx, (T, K), "dx")
    _dtypes(dy.dtype, x=x, w=w, dw=dw, dx=dx)
    _check(load().tp_linear_shard_bwd(_ptr(x), _ptr(w), _ptr(dy), _ptr(dw), _ptr(dx), _ptr(ws),
                                      ws.numel() if ws is not None else 0, T, K, N, _dt(dy), _stream()))


def tp_gqa_attention_fwd(qkv, out, n_q: int, n_kv: int, head_dim: int, causal: bool, scale: float):
    """Attention over a rank's local heads: qkv (T, (n_q + 2 n_kv) head_dim)
    rows [Q | K | V] -> out (T, n_q head_dim)."""
    T = qkv.shape[0]
    _shape(qkv, (T, (n_q + 2 * n_kv) * head_dim), "qkv")
    _shape(out, (T, n_q * head_dim), "out")
    _dtypes(torch.bfloat16, qkv=qkv, out=out)
    _check(load().tp_gqa_attention_fwd(_ptr(qkv), _ptr(out), T, n_q, n_kv, head_dim, int(bool(causal)), scale,
                                       _stream()))
    return out


def _fp8_codes(t: torch.Tensor, name: str) -> None:
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError(f"{name} must hold e4m3 codes (uint8 or float8_e4m3fn)")


def tp_linear_fp8_workspace(T: int, K: int, N: int, act: str = "none") -> int:
    return load().tp_linear_fp8_workspace(T, K, N, ACT[act])


def tp_fp8_pack_strips(src, dst):
    """(K, N) row-major fp8 codes -> the 64-column strip-major order (dst, K*N bytes)."""
    K, N = src.shape
    _fp8_codes(src, "src")
    _fp8_codes(dst, "dst")
    if dst.numel() != K * N:
        raise ValueError("dst must hold K*N codes")
    _check(load().tp_fp8_pack_strips(_ptr(src), _ptr(dst), K, N, _stream()))
    return dst


def tp_mlp_shard_fwd_fp8_workspace(T: int, d: int, ff_i: int, act: str) -> int:
    return load().tp_mlp_shard_fwd_fp8_workspace(T, d, ff_i, ACT[act])


def tp_mlp_shard_fwd_fp8(x, wq1_i, s1_i, wq_up_i, s_up_i, wq2_i, s2_i, y_i, act: str, ws: torch.Tensor):
    """Decode-size shard forward with strip-major fp8 weights and per-column scales."""
    T, d = x.shape
    ff_i = wq1_i.shape[1]
    for t, nm in ((wq1_i, "wq1_i"), (wq2_i, "wq2_i")):
        _fp8_codes(t, nm)
    _shape(wq1_i, (d, ff_i), "wq1_i")
    _shape(wq2_i, (ff_i, d), "wq2_i")
    _shape(s1_i, (ff_i,), "s1_i")
    _shape(s2_i, (d,), "s2_i")
    _shape(y_i, (T, d), "y_i")
    if wq_up_i is not None:
        _fp8_codes(wq_up_i, "wq_up_i")
        _shape(wq_up_i, (d, ff_i), "wq_up_i")
    _dtypes(torch.bfloat16, x=x)
    _dtypes(torch.float32, s1_i=s1_i, s_up_i=s_up_i, s2_i=s2_i)
    _check(load().tp_mlp_shard_fwd_fp8(_ptr(x), _ptr(wq1_i), _ptr(s1_i), _ptr(wq_up_i), _ptr(s_up_i), _ptr(wq2_i),
                                       _ptr(s2_i), _ptr(y_i), _ptr(ws), ws.numel() if ws is not None else 0, T, d,
                                       ff_i, _dt(y_i), ACT[act], _stream()))
    return y_i


def tp_moe_route(logits, k: int, idx, gate):
    """Top-k experts per token (idx int32 (T, k)) and their renormalised
    softmax gates (fp32 (T, k)) from fp32 router logits (T, E)."""
    T, E = logits.shape
    if logits.dtype != torch.float32 or idx.dtype != torch.int32 or gate.dtype != torch.float32:
        raise TypeError("logits and gate are float32, idx int32")
    _shape(idx, (T, k), "idx")
    _shape(gate, (T, k), "gate")
    _check(load().tp_moe_route(_ptr(logits), T, E, k, _ptr(idx), _ptr(gate), _stream()))
    return idx, gate


def tp_moe_shard_fwd_workspace(T: int, d: int, ff_i: int, E: int, k: int) -> int:
    return load().tp_moe_shard_fwd_workspace(T, d, ff_i, E, k)


def tp_moe_shard_fwd(x, idx, gate, w1, w_up, w2, y_i, ws: torch.Tensor):
    """This rank's partial of the MoE block (experts sharded in place)."""
    T, d = x.shape
    E, _, ff_i = w1.shape
    k = idx.shape[1]
    _shape(w1, (E, d, ff_i), "w1")
    _shape(w_up, (E, d, ff_i), "w_up")
    _shape(w2, (E, ff_i, d), "w2")
    _shape(idx, (T, k), "idx")
    _shape(gate, (T, k), "gate")
    _shape(y_i, (T, d), "y_i")
    if idx.dtype != torch.int32 or gate.dtype != torch.float32:
        raise TypeError("idx must be int32 and gate float32")
    _dtypes(torch.bfloat16, x=x, w1=w1, w_up=w_up, w2=w2)
    _check(load().tp_moe_shard_fwd(_ptr(x), _ptr(idx), _ptr(gate), _ptr(w1), _ptr(w_up), _ptr(w2), _ptr(y_i),
                                   _ptr(ws), ws.numel() if ws is not None else 0, T, d, ff_i, E, k, _dt(y_i),
                                   _stream()))
    return y_i


def tp_col_linear_fp8(x, wq, scale, wq_up, scale_up, bias, y, act: str, ws: torch.Tensor):
    """y = act(x (e4m3(wq) * scale) [+ bias]); SWIGLU: silu(x W) * (x W_up).
    wq / wq_up: (K, N)-shaped buffers holding the codes strip-major (see
    tp_fp8_pack_strips)."""
    T, K = x.shape
    N = wq.shape[1]
    _fp8_codes(wq, "wq")
    _shape(wq, (K, N), "wq")
    _shape(scale, (N,), "scale")
    _shape(y, (T, N), "y")
    if wq_up is not None:
        _fp8_codes(wq_up, "wq_up")
        _shape(wq_up, (K, N), "wq_up")
    _dtypes(torch.bfloat16, x=x, bias=bias, y=y)
    _dtypes(torch.float32, scale=scale, scale_up=scale_up)
    _check(load().tp_col_linear_fp8(_ptr(x), _ptr(wq), _ptr(scale), _ptr(wq_up), _ptr(scale_up), _ptr(bias), _ptr(y),
                                    _ptr(ws), ws.numel() if ws is not None else 0, T, K, N, ACT[act], _stream()))
    return y


def tp_row_linear_partial_fp8(x_i, wq_i, scale_i, z_i, ws: torch.Tensor):
    """z_i = x_i (e4m3(wq_i) * scale_i), the full-shape partial (wq_i strip-major)."""
    T, K = x_i.shape
    N = wq_i.shape[1]
    _fp8_codes(wq_i, "wq_i")
    _shape(wq_i, (K, N), "wq_i")
    _shape(scale_i, (N,), "scale_i")
    _shape(z_i, (T, N), "z_i")
    _dtypes(torch.bfloat16, x_i=x_i)
    _dtypes(torch.float32, scale_i=scale_i)
    _check(load().tp_row_linear_partial_fp8(_ptr(x_i), _ptr(wq_i), _ptr(scale_i), _ptr(z_i), _ptr(ws),
                                            ws.numel() if ws is not None else 0, T, K, N, _dt(z_i), _stream()))
    return z_i


def tp_partial_sum(zs: Sequence[torch.Tensor], bias, y):
    T, N = y.shape
    for z in zs:
        _shape(z, (T, N), "z")
        _dtypes(zs[0].dtype, z=z)
    _dtypes(zs[0].dtype if zs else y.dtype, bias=bias)
    arr = (c_p * len(zs))(*[_ptr(z) for z in zs])
    _check(load().tp_partial_sum(arr, len(zs), _ptr(bias), _ptr(y), T, N, _dt(zs[0]), _dt(y), _stream()))
    return y


def tp_rs_residual_rmsnorm(zs: Sequence[torch.Tensor], rank: int, bias, residual_in, norm_w, eps: float,
                           residual_out, y):
    """Rank `rank`'s rows of sum(zs) (+ bias) + residual_in -> residual_out, and
    their RMSNorm (scale norm_w, epsilon eps) -> y."""
    p = len(zs)
    T, N = zs[0].shape
    for z in zs:
        _shape(z, (T, N), "z")
    rows = T // p if p else 0
    _shape(residual_in, (rows, N), "residual_in")
    _shape(residual_out, (rows, N), "residual_out")
    _shape(y, (rows, N), "y")
    _shape(norm_w, (N,), "norm_w")
    for z in zs:
        _dtypes(zs[0].dtype, z=z)
    _dtypes(zs[0].dtype, bias=bias)
    _dtypes(y.dtype, residual_in=residual_in, residual_out=residual_out, norm_w=norm_w)
    arr = (c_p * p)(*[_ptr(z) for z in zs])
    _check(load().tp_rs_residual_rmsnorm(arr, p, rank, _ptr(bias), _ptr(residual_in), _ptr(norm_w), eps,
                                         _ptr(residual_out), _ptr(y), T, N, _dt(zs[0]), _dt(y), _stream()))
    return y


def tp_workspace_init(ws: torch.Tensor):
    _check(load().tp_workspace_init(_ptr(ws), ws.numel(), _stream()))


# ---- packed weights (decode-sized calls) -------------------------------------------
def tp_packed_weight_bytes(K: int, N: int) -> int:
    return load().tp_packed_weight_bytes(K, N)


def tp_pack_weight(w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """(K, N) bf16 row-major -> the packed layout (a flat uint8 tensor of
    tp_packed_weight_bytes(K, N) bytes); `out` may be given."""
    K, N = w.shape
    _dtypes(torch.bfloat16, w=w)
    nbytes = tp_packed_weight_bytes(K, N)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    if out.numel() * out.element_size() < nbytes:
        raise ValueError(f"out holds {out.numel() * out.element_size()} bytes < {nbytes}")
    _check(load().tp_pack_weight(_ptr(w), _ptr(out), K, N, _stream()))
    return out


def tp_linear_packed_workspace(T: int, K: int, N: int, act: str = "none") -> int:
    return load().tp_linear_packed_workspace(T, K, N, ACT[act])


def _packed(t, K, N, name):
    if t is not None and t.numel() * t.element_size() < tp_packed_weight_bytes(K, N):
        raise ValueError(f"{name}: packed weight of {t.numel() * t.element_size()} bytes < "
                         f"{tp_packed_weight_bytes(K, N)}")


def tp_col_linear_packed(x, w_packed, w_up_packed, bias, y, act: str, K: int, N_i: int, ws: torch.Tensor):
    T = x.shape[0]
    _shape(x, (T, K), "x")
    _shape(y, (T, N_i), "y")
    _packed(w_packed, K, N_i, "w_packed")
    _packed(w_up_packed, K, N_i, "w_up_packed")
    if bias is not None:
        _shape(bias, (N_i,), "bias")
    _dtypes(torch.bfloat16, x=x, y=y, bias=bias)
    _check(load().tp_col_linear_packed(_ptr(x), _ptr(w_packed), _ptr(w_up_packed), _ptr(bias), _ptr(y), _ptr(ws),
                                       ws.numel() if ws is not None else 0, T, K, N_i, ACT[act], _stream()))
    return y


def tp_row_linear_partial_packed(x_i, w_packed, z_i, N: int, ws: torch.Tensor):
    T, K_i = x_i.shape
    _shape(z_i, (T, N), "z_i")
    _packed(w_packed, K_i, N, "w_packed")
    _dtypes(torch.bfloat16, x_i=x_i)
    _check(load().tp_row_linear_partial_packed(_ptr(x_i), _ptr(w_packed), _ptr(z_i), _ptr(ws),
                                               ws.numel() if ws is not None else 0, T, K_i, N, _dt(z_i), _stream()))
    return z_i


def tp_mlp_shard_fwd_packed_workspace(T: int, d: int, ff_i: int, act: str) -> int:
    return load().tp_mlp_shard_fwd_packed_workspace(T, d, ff_i, ACT[act])


def tp_mlp_shard_fwd_packed(x, w1_packed, w_up_packed, w2_packed, y_i, act: str, ff_i: int, ws: torch.Tensor):
    T, d = x.shape
    _shape(y_i, (T, d), "y_i")
    _packed(w1_packed, d, ff_i, "w1_packed")
    _packed(w_up_packed, d, ff_i, "w_up_packed")
    _packed(w2_packed, ff_i, d, "w2_packed")
    _dtypes(torch.bfloat16, x=x)
    _check(load().tp_mlp_shard_fwd_packed(_ptr(x), _ptr(w1_packed), _ptr(w_up_packed), _ptr(w2_packed), _ptr(y_i),
                                          _ptr(ws), ws.numel() if ws is not None else 0, T, d, ff_i, _dt(y_i),
                                          ACT[act], _stream()))
    return y_i


# ---- packed fp8 weights -----------------------------------------------------------
def tp_packed_fp8_weight_bytes(K: int, N: int) -> int:
    return load().tp_packed_fp8_weight_bytes(K, N)


def tp_pack_weight_fp8(codes: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """(K, N) row-major e4m3 codes -> the packed fp8 layout (a flat uint8 tensor
    of tp_packed_fp8_weight_bytes(K, N) bytes); `out` may be given."""
    K, N = codes.shape
    _fp8_codes(codes, "codes")
    nbytes = tp_packed_fp8_weight_bytes(K, N)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    if out.numel() * out.element_size() < nbytes:
        raise ValueError(f"out holds {out.numel() * out.element_size()} bytes < {nbytes}")
    _check(load().tp_pack_weight_fp8(_ptr(codes), _ptr(out), K, N, _stream()))
    return out


def _packed8(t, K, N, name):
    if t is not None and t.numel() * t.element_size() < tp_packed_fp8_weight_bytes(K, N):
        raise ValueError(f"{name}: packed fp8 weight of {t.numel() * t.element_size()} bytes < "
                         f"{tp_packed_fp8_weight_bytes(K, N)}")


def tp_linear_packed_fp8_workspace(T: int, K: int, N: int, act: str = "none") -> int:
    return load().tp_linear_packed_fp8_workspace(T, K, N, ACT[act])


def tp_col_linear_packed_fp8(x, wq_packed, scale, wq_up_packed, scale_up, bias, y, act: str, K: int, N_i: int,
                             ws: torch.Tensor):
    T = x.shape[0]
    _shape(x, (T, K), "x")
    _shape(y, (T, N_i), "y")
    _packed8(wq_packed, K, N_i, "wq_packed")
    _packed8(wq_up_packed, K, N_i, "wq_up_packed")
    _shape(scale, (N_i,), "scale")
    if scale_up is not None:
        _shape(scale_up, (N_i,), "scale_up")
    if bias is not None:
        _shape(bias, (N_i,), "bias")
    _dtypes(torch.bfloat16, x=x, y=y, bias=bias)
    _dtypes(torch.float32, scale=scale, scale_up=scale_up)
    _check(load().tp_col_linear_packed_fp8(_ptr(x), _ptr(wq_packed), _ptr(scale), _ptr(wq_up_packed), _ptr(scale_up),
                                           _ptr(bias), _ptr(y), _ptr(ws), ws.numel() if ws is not None else 0, T, K,
                                           N_i, ACT[act], _stream()))
    return y


def tp_row_linear_partial_packed_fp8(x_i, wq_packed, scale_i, z_i, N: int, ws: torch.Tensor):
    T, K_i = x_i.shape
    _shape(z_i, (T, N), "z_i")
    _packed8(wq_packed, K_i, N, "wq_packed")
    _shape(scale_i, (N,), "scale_i")
    _dtypes(torch.bfloat16, x_i=x_i)
    _dtypes(torch.float32, scale_i=scale_i)
    _check(load().tp_row_linear_partial_packed_fp8(_ptr(x_i), _ptr(wq_packed), _ptr(scale_i), _ptr(z_i), _ptr(ws),
                                                   ws.numel() if ws is not None else 0, T, K_i, N, _dt(z_i),
                                                   _stream()))
    return z_i


def tp_mlp_shard_fwd_packed_fp8_workspace(T: int, d: int, ff_i: int, act: str) -> int:
    return load().tp_mlp_shard_fwd_packed_fp8_workspace(T, d, ff_i, ACT[act])


def tp_mlp_shard_fwd_packed_fp8(x, wq1_packed, s1_i, wq_up_packed, s_up_i, wq2_packed, s2_i, y_i, act: str, ff_i: int,
                                ws: torch.Tensor):
    T, d = x.shape
    _shape(y_i, (T, d), "y_i")
    _packed8(wq1_packed, d, ff_i, "wq1_packed")
    _packed8(wq_up_packed, d, ff_i, "wq_up_packed")
    _packed8(wq2_packed, ff_i, d, "wq2_packed")
    _shape(s1_i, (ff_i,), "s1_i")
    _shape(s2_i, (d,), "s2_i")
    if s_up_i is not None:
        _shape(s_up_i, (ff_i,), "s_up_i")
    _dtypes(torch.bfloat16, x=x)
    _dtypes(torch.float32, s1_i=s1_i, s_up_i=s_up_i, s2_i=s2_i)
    _check(load().tp_mlp_shard_fwd_packed_fp8(_ptr(x), _ptr(wq1_packed), _ptr(s1_i), _ptr(wq_up_packed),
                                              _ptr(s_up_i), _ptr(wq2_packed), _ptr(s2_i), _ptr(y_i), _ptr(ws),
                                              ws.numel() if ws is not None else 0, T, d, ff_i, _dt(y_i), ACT[act],
                                              _stream()))
    return y_i


def tp_packed_act_bytes(T: int, K: int) -> int:
    return load().tp_packed_act_bytes(T, K)


def tp_pack_act(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x (T, K) bf16 -> the packed-activation bytes (flat uint8)."""
    T, K = x.shape
    _dtypes(torch.bfloat16, x=x)
    nbytes = tp_packed_act_bytes(T, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    if out.numel() * out.element_size() < nbytes:
        raise ValueError(f"out holds {out.numel() * out.element_size()} bytes < {nbytes}")
    _check(load().tp_pack_act(_ptr(x), _ptr(out), T, K, _stream()))
    return out


def tp_linear_packed_gemm(x_packed, w_packed, w_up_packed, bias, y, act: str, K: int, ws: torch.Tensor):
    T, N = y.shape
    if x_packed.numel() * x_packed.element_size() < tp_packed_act_bytes(T, K):
        raise ValueError("x_packed is smaller than the packed activations")
    _packed(w_packed, K, N, "w_packed")
    _packed(w_up_packed, K, N, "w_up_packed")
    if bias is not None:
        _shape(bias, (N,), "bias")
        _dtypes(torch.bfloat16, bias=bias)
    _check(load().tp_linear_packed_gemm(_ptr(x_packed), _ptr(w_packed), _ptr(w_up_packed), _ptr(bias), _ptr(y),
                                        _ptr(ws), ws.numel() if ws is not None else 0, T, K, N, ACT[act], _dt(y),
                                        _stream()))
    return y
