"""CPU tests of the C ABI: the library loads, exports every declared symbol,
its host helpers agree with the oracle, and every invalid-argument path
returns its status code before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

import oracle as O
import tensor_sharded_transformer_amd as tp
from tensor_sharded_transformer_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
OK, NULL, SHAPE, DTYPE, ACTE, WS = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        pytest.skip("libtpshard.so not built")
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(tp_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("tp_col_linear", "tp_act_inplace", "tp_row_linear_partial", "tp_mlp_shard_fwd", "tp_mlp_shard_bwd",
              "tp_partial_sum", "tp_shard_range", "tp_gqa_shard"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(B.SIGNATURES)


def test_abi_version(lib):
    assert tp.tp_abi_version() == 1


@pytest.mark.parametrize("n,p", [(256, 4), (28672, 8), (3, 3), (14336, 8), (1280, 1)])
def test_shard_range_matches_oracle(lib, n, p):
    for i in range(p):
        assert tp.tp_shard_range(n, p, i) == O.shard_range(n, p, i)


def test_shard_range_errors(lib):
    b, ln = ctypes.c_int64(), ctypes.c_int64()
    assert lib.tp_shard_range(10, 4, 0, ctypes.byref(b), ctypes.byref(ln)) == SHAPE
    assert lib.tp_shard_range(8, 0, 0, ctypes.byref(b), ctypes.byref(ln)) == SHAPE
    assert lib.tp_shard_range(8, 2, 2, ctypes.byref(b), ctypes.byref(ln)) == SHAPE
    assert lib.tp_shard_range(-8, 2, 0, ctypes.byref(b), ctypes.byref(ln)) == SHAPE
    assert lib.tp_shard_range(8, 2, 0, None, ctypes.byref(ln)) == NULL
    assert "divisible" in lib.tp_last_error().decode() or lib.tp_last_error()


def test_gqa_shard_matches_page_and_oracle(lib):
    for i in range(8):
        assert tp.tp_gqa_shard(64, 8, 128, 8, i) == O.gqa_shard(64, 8, 128, 8, i) == (1024 * i, 1024, 128 * i, 128)
    with pytest.raises(tp.TpError) as e:
        tp.tp_gqa_shard(64, 8, 128, 16, 0)   # 8 KV heads cannot be split over 16 ranks
    assert e.value.status == SHAPE


def test_col_linear_validation(lib):
    f = lib.tp_col_linear
    # bad dtype / act
    assert f(FAKE, FAKE, None, None, FAKE, None, 0, 4, 8, 8, 7, 0, None) == DTYPE
    assert f(FAKE, FAKE, None, None, FAKE, None, 0, 4, 8, 8, 0, 9, None) == ACTE
    # SWIGLU needs w_up; others must not have it; no bias with SWIGLU
    assert f(FAKE, FAKE, None, None, FAKE, None, 0, 4, 8, 8, 0, 3, None) == ACTE
    assert f(FAKE, FAKE, FAKE, None, FAKE, None, 0, 4, 8, 8, 0, 1, None) == ACTE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 8, 8, 0, 3, None) == ACTE
    # negative sizes
    assert f(FAKE, FAKE, None, None, FAKE, None, 0, -1, 8, 8, 0, 1, None) == SHAPE
    # null operands
    assert f(None, FAKE, None, None, FAKE, None, 0, 4, 8, 8, 0, 1, None) == NULL
    assert f(FAKE, FAKE, None, None, None, None, 0, 4, 8, 8, 0, 1, None) == NULL
    # T == 0 is a no-op, even with null pointers
    assert f(None, None, None, None, None, None, 0, 0, 8, 8, 0, 1, None) == OK


def test_col_linear_workspace_too_small(lib):
    need = lib.tp_col_linear_workspace(64, 8192, 3584, 0, 3)
    assert need > 0   # decode-sized calls split K
    # the query is the maximum over operand alignments; half of it is too small for every plan
    assert lib.tp_col_linear(FAKE, FAKE, FAKE, None, FAKE, FAKE, need // 2, 64, 8192, 3584, 0, 3, None) == WS
    assert lib.tp_col_linear_workspace(4096, 8192, 3584, 0, 3) == 0   # large T: no split


def test_act_inplace_validation(lib):
    f = lib.tp_act_inplace
    assert f(FAKE, None, 4, 8, 0, 3, None) == ACTE        # SWIGLU without up
    assert f(FAKE, FAKE, 4, 8, 0, 2, None) == ACTE        # up with GELU
    assert f(None, None, 4, 8, 0, 1, None) == NULL
    assert f(FAKE, None, 4, 8, 5, 1, None) == DTYPE
    assert f(None, None, 4, 8, 0, 0, None) == OK          # NONE: no-op


def test_row_linear_validation(lib):
    f = lib.tp_row_linear_partial
    assert f(FAKE, FAKE, FAKE, None, 0, 4, 8, 8, 1, 0, None) == DTYPE   # f32 in, bf16 out
    assert f(FAKE, None, FAKE, None, 0, 4, 8, 8, 0, 0, None) == NULL
    assert f(FAKE, FAKE, FAKE, None, 0, 4, -8, 8, 0, 0, None) == SHAPE
    assert f(None, None, None, None, 0, 0, 8, 8, 0, 0, None) == OK


def test_mlp_fwd_validation(lib):
    f = lib.tp_mlp_shard_fwd
    need = lib.tp_mlp_shard_fwd_workspace(64, 8192, 3584, 0, 3)
    assert need >= 64 * 3584 * 2
    args = (64, 8192, 3584, 0, 0, 3, None)
    # the query is the maximum over operand alignments; half of it is too small for every plan
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need // 2, *args) == WS
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, *args) == WS
    assert f(FAKE, FAKE, None, FAKE, FAKE, None, FAKE, need, *args) == ACTE    # SWIGLU needs w_up
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need, 64, 8192, 3584, 0, 0, 1, None) == ACTE
    assert f(FAKE, FAKE, None, FAKE, FAKE, None, FAKE, need, 64, 8192, 3584, 1, 0, 1, None) == DTYPE  # f32 -> bf16
    assert f(None, FAKE, FAKE, FAKE, FAKE, None, FAKE, need, *args) == NULL
    assert f(None, None, FAKE, None, None, None, None, 0, 0, 8192, 3584, 0, 0, 3, None) == OK  # T == 0


def test_mlp_bwd_validation(lib):
    f = lib.tp_mlp_shard_bwd
    need = lib.tp_mlp_shard_bwd_workspace(2048, 4096, 1792, 0, 3)
    assert need >= 2048 * 1792 * 2 * 3
    sz = (2048, 4096, 1792, 0, 3, None)
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, *sz) == WS
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need, *sz) == ACTE  # dw_up missing
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, *sz) == NULL  # saved missing


def test_partial_sum_validation(lib):
    f = lib.tp_partial_sum
    arr = (ctypes.c_void_p * 2)(0x1000, None)
    assert f(arr, 2, None, FAKE, 4, 8, 0, 1, None) == NULL          # z[1] null
    assert f(arr, 0, None, FAKE, 4, 8, 0, 1, None) == SHAPE
    assert f(arr, 65, None, FAKE, 4, 8, 0, 1, None) == SHAPE
    assert f(arr, 1, None, FAKE, 4, 8, 3, 1, None) == DTYPE
    assert f(arr, 2, None, FAKE, 0, 8, 0, 1, None) == OK             # T == 0


def test_rs_residual_rmsnorm_validation(lib):
    f = lib.tp_rs_residual_rmsnorm
    arr = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    args = (None, FAKE, FAKE, ctypes.c_float(1e-5), FAKE, FAKE)
    assert f(arr, 2, 0, *args, 8, 64, 7, 0, None) == DTYPE
    assert f(arr, 0, 0, *args, 8, 64, 0, 0, None) == SHAPE          # p = 0
    assert f(arr, 2, 2, *args, 8, 64, 0, 0, None) == SHAPE          # rank out of range
    assert f(arr, 2, -1, *args, 8, 64, 0, 0, None) == SHAPE
    assert f(arr, 2, 0, *args, 7, 64, 0, 0, None) == SHAPE          # 7 rows, 2 shares
    assert f(arr, 2, 0, *args, 8, 40000, 0, 0, None) == 6           # N above the row limit: unsupported
    assert f(arr, 2, 0, None, FAKE, FAKE, ctypes.c_float(-1.0), FAKE, FAKE, 8, 64, 0, 0, None) == SHAPE
    assert f(arr, 2, 0, None, None, FAKE, ctypes.c_float(0.0), FAKE, FAKE, 8, 64, 0, 0, None) == NULL
    bad = (ctypes.c_void_p * 2)(0x1000, None)
    assert f(bad, 2, 0, *args, 8, 64, 0, 0, None) == NULL            # z[1] null
    assert f(arr, 2, 0, *args, 0, 64, 0, 0, None) == OK              # T == 0


def test_linear_shard_bwd_validation(lib):
    f = lib.tp_linear_shard_bwd
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 8, 16, 32, 5, None) == DTYPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, -1, 16, 32, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, None, None, None, 0, 8, 16, 32, 0, None) == NULL      # nothing requested
    assert f(None, FAKE, FAKE, FAKE, None, None, 0, 8, 16, 32, 0, None) == NULL      # dw without x
    assert f(FAKE, None, FAKE, None, FAKE, None, 0, 8, 16, 32, 0, None) == NULL      # dx without w
    assert f(FAKE, FAKE, None, FAKE, FAKE, None, 0, 8, 16, 32, 0, None) == NULL      # no dy
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 8, 0, 32, 0, None) == OK         # K == 0: nothing to do
    assert f(FAKE, FAKE, FAKE, None, FAKE, None, 0, 0, 16, 32, 0, None) == OK        # T == 0, no dw
    assert lib.tp_linear_shard_bwd_workspace(0, 8192, 1280, 0) == 0
    need = lib.tp_linear_shard_bwd_workspace(64, 8192, 1280, 0)   # split-K at T = 64
    assert need > 0
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 64, 8192, 1280, 0, None) == WS
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 64, 8192, 1280, 0, None) == WS


def test_gqa_attention_validation(lib):
    f = lib.tp_gqa_attention_fwd
    sc = ctypes.c_float(0.088)
    assert f(FAKE, FAKE, -1, 8, 1, 128, 1, sc, None) == SHAPE
    assert f(FAKE, FAKE, 64, 8, 3, 128, 1, sc, None) == SHAPE          # 8 query heads over 3 KV heads
    assert f(FAKE, FAKE, 64, 0, 1, 128, 1, sc, None) == SHAPE
    assert f(FAKE, FAKE, 64, 8, 1, 128, 2, sc, None) == SHAPE          # causal flag not 0/1
    assert f(FAKE, FAKE, 64, 8, 1, 128, 1, ctypes.c_float(0.0), None) == SHAPE
    assert f(FAKE, FAKE, 64, 8, 1, 128, 1, ctypes.c_float(float("nan")), None) == SHAPE
    assert f(FAKE, FAKE, 64, 8, 1, 128, 1, ctypes.c_float(float("inf")), None) == SHAPE
    assert f(FAKE, FAKE, 64, 8, 1, 64, 1, sc, None) == 6               # head_dim 64: not built
    assert f(None, FAKE, 64, 8, 1, 128, 1, sc, None) == NULL
    assert f(ctypes.c_void_p(0x1008), FAKE, 64, 8, 1, 128, 1, sc, None) == 6   # unaligned
    assert f(None, None, 0, 8, 1, 128, 1, sc, None) == OK              # T == 0


def test_linear_fp8_validation(lib):
    f = lib.tp_col_linear_fp8
    ws = lib.tp_linear_fp8_workspace(64, 1024, 256, 0)
    assert ws > 0 and lib.tp_linear_fp8_workspace(65, 1024, 256, 0) == 0
    args = (FAKE, ctypes.c_size_t(ws), 64, 1024, 256)
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, *args, 9, None) == ACTE          # unknown act
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, *args, 3, None) == ACTE          # SWIGLU without wq_up
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, *args, 3, None) == ACTE          # bias with SWIGLU
    assert f(FAKE, FAKE, None, None, None, None, FAKE, *args, 0, None) == NULL          # no scale
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, ws, 65, 1024, 256, 0, None) == 6   # T > 64
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, ws, 64, 1024, 272, 0, None) == 6   # N % 64
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, None, 0, 64, 1024, 256, 0, None) == WS
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, ws - 1, 64, 1024, 256, 0, None) == WS
    assert f(None, None, None, None, None, None, None, None, 0, 0, 1024, 256, 0, None) == OK   # T == 0
    g = lib.tp_row_linear_partial_fp8
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, ws, 64, 1024, 256, 7, None) == DTYPE
    assert g(FAKE, FAKE, None, FAKE, FAKE, ws, 64, 1024, 256, 0, None) == NULL
    m = lib.tp_mlp_shard_fwd_fp8
    mws = lib.tp_mlp_shard_fwd_fp8_workspace(64, 8192, 3584, 3)
    assert mws > 0 and lib.tp_mlp_shard_fwd_fp8_workspace(65, 8192, 3584, 3) == 0
    margs = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert m(*margs, ctypes.c_size_t(mws), 64, 8192, 3584, 0, 9, None) == ACTE
    assert m(*margs, ctypes.c_size_t(mws), 65, 8192, 3584, 0, 3, None) == 6      # T > 64
    assert m(*margs, ctypes.c_size_t(mws), 64, 8192, 3600, 0, 3, None) == 6      # ff_i % 64
    assert m(*margs[:8], None, 0, 64, 8192, 3584, 0, 3, None) == WS
    assert m(FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, mws, 64, 8192, 3584, 0, 3, None) == ACTE
    pk = lib.tp_fp8_pack_strips
    assert pk(FAKE, ctypes.c_void_p(0x2000), 16, 100, None) == SHAPE     # N % 64
    assert pk(FAKE, FAKE, 16, 128, None) == SHAPE                         # aliasing
    assert pk(None, FAKE, 16, 128, None) == NULL
    assert pk(None, None, 0, 128, None) == OK


def test_moe_validation(lib):
    r = lib.tp_moe_route
    assert r(FAKE, 8, 4, 5, FAKE, FAKE, None) == SHAPE        # k > E
    assert r(FAKE, 8, 2000, 2, FAKE, FAKE, None) == SHAPE     # E > 1024
    assert r(FAKE, 8, 16, 17, FAKE, FAKE, None) == SHAPE      # k > 16
    assert r(None, 8, 16, 2, FAKE, FAKE, None) == NULL
    assert r(None, 0, 16, 2, None, None, None) == OK
    f = lib.tp_moe_shard_fwd
    ws = lib.tp_moe_shard_fwd_workspace(64, 256, 96, 16, 4)
    assert ws > 0
    a = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert f(*a, FAKE, ctypes.c_size_t(ws), 64, 256, 96, 16, 4, 7, None) == DTYPE
    assert f(*a, FAKE, ctypes.c_size_t(ws), 64, 256, 96, 16, 17, 0, None) == SHAPE
    assert f(*a, FAKE, ctypes.c_size_t(ws), 64, 260, 96, 16, 4, 0, None) == 6       # d % 8
    assert f(*a, None, 0, 64, 256, 96, 16, 4, 0, None) == WS
    assert f(*a, FAKE, ctypes.c_size_t(ws - 1), 64, 256, 96, 16, 4, 0, None) == WS
    assert f(None, None, None, None, None, None, None, None, 0, 0, 256, 96, 16, 4, 0, None) == OK


def test_status_strings(lib):
    for s in range(8):
        assert lib.tp_status_string(s)


def test_binding_rejects_mixed_operand_dtypes():
    """The kernels read raw bytes, so the binding refuses operands whose dtype
    differs from the one the call declares (checked before any device call)."""
    import torch
    f32 = torch.zeros(4, 8, dtype=torch.float32)
    bf = torch.zeros(8, 8, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        B.tp_col_linear(f32, bf, None, None, torch.zeros(4, 8), "none")
    with pytest.raises(TypeError):
        B.tp_row_linear_partial(f32, bf, torch.zeros(4, 8))
    with pytest.raises(TypeError):
        B.tp_gqa_attention_fwd(torch.zeros(4, 3 * 128), torch.zeros(4, 128), 1, 1, 128, True, 0.1)
    with pytest.raises(TypeError):
        B.tp_partial_sum([torch.zeros(4, 8), torch.zeros(4, 8, dtype=torch.bfloat16)], None, torch.zeros(4, 8))


def test_mlp_shard_fwd_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """The allocation-free forward refuses shapes whose scratch exceeds its
    static array, before it touches the device."""
    need = tp.tp_mlp_shard_fwd_workspace(4096, 16384, 8192, tp.TP_BF16, "swiglu")
    assert need > B.NOALLOC_SCRATCH_BYTES
    f = lib.tp_mlp_shard_fwd_noalloc
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, 4096, 16384, 8192, 0, 0, 3, None) == WS
    assert "static scratch" in lib.tp_last_error().decode()
    # the other argument checks come first, as in tp_mlp_shard_fwd
    assert f(FAKE, FAKE, None, FAKE, FAKE, None, 64, 64, 64, 0, 0, 3, None) == ACTE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, 64, 64, 64, 1, 0, 3, None) == DTYPE


def test_packed_entry_points_validation(lib):
    """Packed-weight calls serve T <= 64 and check their arguments first."""
    assert lib.tp_col_linear_packed(FAKE, FAKE, None, None, FAKE, FAKE, 1 << 20, 65, 64, 64, 0, None) == SHAPE
    assert "T <= 64" in lib.tp_last_error().decode()
    assert lib.tp_col_linear_packed(FAKE, FAKE, None, None, FAKE, FAKE, 1 << 20, 4, 64, 64, 3, None) == ACTE
    assert lib.tp_col_linear_packed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 4, 64, 64, 3, None) == ACTE
    assert lib.tp_col_linear_packed(FAKE, FAKE, None, None, FAKE, None, 0, 4, 64, 64, 0, None) == WS
    assert lib.tp_col_linear_packed(FAKE, FAKE, None, None, FAKE, FAKE, 16, 4, 64, 64, 0, None) == WS
    assert lib.tp_row_linear_partial_packed(FAKE, None, FAKE, FAKE, 1 << 20, 4, 64, 64, 0, None) == NULL
    assert lib.tp_row_linear_partial_packed(FAKE, FAKE, FAKE, FAKE, 1 << 20, 4, 64, 64, 9, None) == DTYPE
    assert lib.tp_mlp_shard_fwd_packed(FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 20, 4, 64, 64, 0, 3, None) == ACTE
    assert lib.tp_mlp_shard_fwd_packed(FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 20, 100, 64, 64, 0, 1, None) == SHAPE
    assert lib.tp_pack_weight(None, FAKE, 4, 4, None) == NULL
    assert lib.tp_pack_weight(FAKE, ctypes.c_void_p(0x1008), 4, 4, None) == SHAPE
    assert tp.tp_packed_weight_bytes(8192, 3584) == 224 * 256 * 1024
    assert tp.tp_packed_weight_bytes(33, 17) == 2 * 2 * 1024
    assert tp.tp_linear_packed_workspace(65, 64, 64) == 0
    assert tp.tp_mlp_shard_fwd_packed_workspace(64, 8192, 3584, "swiglu") > 0


def test_packed_fp8_entry_points_validation(lib):
    """Packed fp8 calls: T <= 64, scales required, up weights iff SWIGLU, the
    fused shard needs ff_i % 64 == 0; sizes of the packed codes."""
    f = lib.tp_col_linear_packed_fp8
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, 1 << 20, 65, 64, 64, 0, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, 1 << 20, 4, 64, 64, 3, None) == ACTE   # SWIGLU, no up
    assert f(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1 << 20, 4, 64, 64, 3, None) == ACTE   # up, no scale_up
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 20, 4, 64, 64, 0, None) == ACTE   # up without SWIGLU
    assert f(FAKE, FAKE, None, None, None, None, FAKE, FAKE, 1 << 20, 4, 64, 64, 0, None) == NULL   # no scale
    assert f(FAKE, FAKE, FAKE, None, None, None, FAKE, None, 0, 4, 64, 64, 0, None) == WS
    g = lib.tp_row_linear_partial_packed_fp8
    assert g(FAKE, FAKE, None, FAKE, FAKE, 1 << 20, 4, 64, 64, 0, None) == NULL
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 4, 64, 64, 9, None) == DTYPE
    m = lib.tp_mlp_shard_fwd_packed_fp8
    assert m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 24, 4, 64, 96, 0, 3, None) == 6   # ff_i % 64
    assert m(FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 1 << 24, 4, 64, 64, 0, 3, None) == ACTE
    assert lib.tp_pack_weight_fp8(None, FAKE, 4, 4, None) == NULL
    assert lib.tp_pack_weight_fp8(FAKE, ctypes.c_void_p(0x1008), 4, 4, None) == SHAPE
    assert tp.tp_packed_fp8_weight_bytes(8192, 3584) == 224 * 128 * 1024
    assert tp.tp_packed_fp8_weight_bytes(65, 17) == 2 * 2 * 1024
    assert tp.tp_linear_packed_fp8_workspace(65, 64, 64) == 0
    assert tp.tp_mlp_shard_fwd_packed_fp8_workspace(64, 8192, 3552, "swiglu") == 0
    assert tp.tp_mlp_shard_fwd_packed_fp8_workspace(64, 8192, 3584, "swiglu") > 0
