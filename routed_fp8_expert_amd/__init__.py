"""MI355X (gfx950) decode-step mixture-of-experts FFN.

The compute path is the HIP library built from csrc/ (libmoe_ffn.so) behind
the C ABI in include/moe.h; this package only marshals arguments to it.
"""
from .binding import (  # noqa: F401
    Ctx, DenseWeights, LayerWeights, MoeError, Routing, moe_abi_version, moe_ctx_create, moe_ctx_destroy,
    moe_ctx_device_errors, moe_ctx_kernel_stats, moe_ctx_set_fault_at, moe_ctx_set_force_arm,
    moe_ctx_set_few_rows, moe_ctx_set_mfma_min_rows, moe_ctx_set_one_row_path, moe_ctx_set_timing,
    moe_ctx_set_wait_limit, moe_ctx_status, moe_debug_decode, moe_debug_set_phase_stamps,
    moe_dense_fp8, moe_expert_ffn, moe_layer_forward, moe_layer_forward_norm, moe_layer_forward_static, moe_route, moe_workspace_bytes,
    strerror, workspace,
    KERNELS, MOE_WFMT_FP8_E4M3_B128, MOE_WFMT_NVFP4, MOE_WFMT_INT8_ROW, MOE_WFMT_INT4_ROW, MOE_WFMT_INT4_G64,
    MOE_WFMT_FP8_E4M3_B128_BF16S,
)
