"""Routed sparse-MoE layer for AMD Instinct MI355X (gfx950).

The compute lives in ``libmoe.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/moe.h``); this package only marshals arguments to it.
"""
from ._abi import (  # noqa: F401
    ACT, EXPORTS, LIB_PATH, MOE_DT_BF16, MOE_DT_F32, MOE_F_CHECK_FINITE, MOE_F_FUSED_FFN,
    MOE_F_TILED_WEIGHTS,
    MOE_STAGE_DOWN, MOE_STAGE_GATE_UP, MOE_WF_DENSE, MOE_WF_INT2_G32, MOE_WF_INT4_G32, STATUS, WFMT,
    MoEError, load, make_experts, make_perm, make_shape, moe_combine, moe_device_clock_khz,
    moe_experts, moe_ffn_down, moe_ffn_fused, moe_ffn_fused_items, moe_ffn_gate_up, moe_ffn_down_combine, moe_route_permute, moe_grouped_ffn, moe_layer,
    moe_layer_noalloc, MOE_NOALLOC_SCRATCH_BYTES, moe_perm, moe_permute, moe_route,
    moe_route_locality, moe_route_locality_blocks, moe_shape, moe_stage_experts, moe_status_str,
    moe_stream_read, moe_tile_experts, moe_workspace_size,
)
from .layer import MoELayerBuffers  # noqa: F401
