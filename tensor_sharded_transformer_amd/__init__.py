"""One tensor-parallel rank's transformer-block shard on AMD MI355X (gfx950).

The compute lives in the C-ABI HIP library ``lib/libtpshard.so`` (declared in
``include/tpshard.h``); ``binding`` is a thin ctypes layer over it that takes
torch tensors for device memory and streams.
"""
from .binding import (  # noqa: F401
    ACT,
    TP_BF16,
    TP_F32,
    TpError,
    load,
    new_workspace,
    tp_abi_version,
    tp_act_inplace,
    tp_col_linear,
    tp_col_linear_fp8,
    tp_col_linear_workspace,
    tp_fp8_pack_strips,
    tp_gqa_attention_fwd,
    tp_gqa_shard,
    tp_linear_shard_bwd,
    tp_linear_fp8_workspace,
    tp_linear_shard_bwd_workspace,
    tp_mlp_shard_bwd,
    tp_mlp_shard_bwd_workspace,
    tp_mlp_shard_fwd,
    tp_mlp_shard_fwd_noalloc,
    tp_moe_route,
    tp_moe_shard_fwd,
    tp_moe_shard_fwd_workspace,
    tp_mlp_shard_fwd_fp8,
    tp_mlp_shard_fwd_fp8_workspace,
    tp_mlp_shard_fwd_workspace,
    tp_partial_sum,
    tp_row_linear_partial,
    tp_row_linear_partial_fp8,
    tp_row_linear_partial_workspace,
    tp_rs_residual_rmsnorm,
    tp_shard_range,
    tp_workspace_init,
)
