"""Decode-time fine-grained MoE layer with low-bit experts on AMD MI355X (gfx950).

The compute lives in libmoe.so (HIP kernels behind the C ABI in include/moe.h); this package is
its Python binding plus host-side orchestration of a prerouted decode stack.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, MOE_INPUT_RMSNORM, MOE_MAX_D, MOE_MAX_E, MOE_MAX_K, MOE_TOPK_RENORM, Experts, Lora3,
    MoEError, PrerouterWeights, moe_combine, moe_expert_ffn_q4, moe_expert_ffn_workspace_size, moe_prerouter,
    moe_prerouter_workspace_size, moe_route_topk, moe_sort_by_expert, moe_status_string, moe_version,
    moe_decode_step, moe_decode_workspace_size, moe_decode_layer, moe_decode_stack, moe_rmsnorm,
    MOE_DECODE_GIVEN_ROUTING, moe_expert_ffn_sparse, moe_expert_ffn_sparse_workspace_size,
    Pool, moe_pool, moe_stream_in, moe_stream_workspace_size, moe_stream_in_many, moe_stream_job, MOE_POOL_MAX_JOBS,
    moe_read_probe, MOE_READ_PROBE_BLOCKS, moe_exchange_probe, moe_exchange_probe_workspace_size, moe_xchg_cfg,
    MOE_XCHG_ALL, MOE_XCHG_RING, MOE_XCHG_SCOPE_DEVICE, MOE_XCHG_SCOPE_XCD, moe_decode_step_grid,
    moe_decode_step_stamped, moe_expert_ffn_q4_noalloc, MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_TOO_LARGE,
    moe_decode_step_grid_for, moe_expert_ffn_q4_shared, moe_expert_ffn_shared_workspace_size,
)
