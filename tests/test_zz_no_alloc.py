"""GPU test of the allocation-free forward shard (tp_mlp_shard_fwd_noalloc):
through the C ABI it must give what tp_mlp_shard_fwd gives with a caller
workspace, bit for bit (the same kernels run), and meet the oracle's
tolerance, over two calls in a row whose second input is smaller (the static
scratch keeps the first call's contents)."""
import pytest
import torch

import oracle as O
import workloads as W
import tensor_sharded_transformer_amd as tp

pytestmark = pytest.mark.gpu


def _shard(T, d, ff, act, seed, out_dtype=torch.bfloat16):
    wl = W.MlpWorkload("noalloc", T=T, d=d, ff=ff, p=1, act=act, dtype="bf16", seed=seed)
    t = W.mlp_unsharded(wl)
    dev = lambda v: None if v is None else v.contiguous().to("cuda")
    x, w1, wup, w2 = dev(t["x"]), dev(t["w1"]), dev(t.get("w_up")), dev(t["w2"])
    y_ref = torch.full((T, d), 3.0, dtype=out_dtype, device="cuda")
    sv_ref = torch.full((T, (2 if act == "swiglu" else 1) * ff), 3.0, dtype=torch.bfloat16, device="cuda")
    ws = tp.new_workspace(tp.tp_mlp_shard_fwd_workspace(T, d, ff, tp.TP_BF16, act))
    tp.tp_mlp_shard_fwd(x, w1, wup, w2, y_ref, act, ws, sv_ref)
    ref, _ = O.mlp_shard_fwd(O.to64(t["x"]), O.to64(t["w1"]), None if wup is None else O.to64(t["w_up"]),
                             O.to64(t["w2"]), act)
    return (x, w1, wup, w2), y_ref, sv_ref, ref


def _noalloc(args, act, T, d, ff, out_dtype=torch.bfloat16):
    y = torch.full((T, d), 5.0, dtype=out_dtype, device="cuda")
    sv = torch.full((T, (2 if act == "swiglu" else 1) * ff), 5.0, dtype=torch.bfloat16, device="cuda")
    tp.tp_mlp_shard_fwd_noalloc(*args, y, act, sv)
    return y, sv


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_noalloc_matches_the_workspace_entry_point_on_two_calls(act):
    # the 70B-class decode shard, then a smaller ragged one on the same scratch
    for (T, d, ff, seed) in ((64, 8192, 3584, 81), (37, 1000, 264, 82)):
        args, y_ref, sv_ref, ref = _shard(T, d, ff, act, seed)
        y, sv = _noalloc(args, act, T, d, ff)
        torch.cuda.synchronize()
        print(f"noalloc {act} T={T} d={d} ff={ff}", flush=True)
        assert torch.equal(y, y_ref), "y differs from tp_mlp_shard_fwd"
        assert torch.equal(sv, sv_ref), "saved pre-activations differ"
        ok, rf, rm = O.within(y, ref)
        assert ok, (rf, rm)


def test_noalloc_prefill_rows_and_fp32_output():
    """A tiled-kernel shape (T=512) that still fits the scratch, fp32 output,
    after the decode shapes have used the array."""
    T, d, ff = 512, 2048, 1024
    args, y_ref, sv_ref, ref = _shard(T, d, ff, "swiglu", 83, torch.float32)
    y, sv = _noalloc(args, "swiglu", T, d, ff, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(sv, sv_ref)
    ok, rf, rm = O.within(y, ref)
    assert ok, (rf, rm)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    T, d, ff = 4096, 16384, 8192
    assert tp.tp_mlp_shard_fwd_workspace(T, d, ff, tp.TP_BF16, "swiglu") > tp.binding.NOALLOC_SCRATCH_BYTES
    x = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(d, ff, dtype=torch.bfloat16, device="cuda")
    w2 = torch.empty(ff, d, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tp.TpError) as e:
        tp.tp_mlp_shard_fwd_noalloc(x, w, w, w2, y, "swiglu")
    assert e.value.status == 5
