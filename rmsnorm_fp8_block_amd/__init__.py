"""MI355X (gfx950) library for the MLA decode hot path: fused dual RMSNorm +
per-1x128 FP8 group quantisation of the q/kv latents, its single-input and
norm-less forms, and the block-scaled FP8 GEMM that consumes the quantised
activation.

The computation runs in HIP kernels behind the C ABI of
``include/mi_normquant.h`` (``libmi_normquant.so``); the functions below are
its ctypes binding.  ``workloads`` holds the seeded synthetic inputs.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MiError,
    TiledWeight,
    lib,
    mi_block_scaled_fp8_gemm,
    mi_block_scaled_fp8_gemm_pair,
    mi_fused_dual_rmsnorm_group_quant,
    mi_fused_dual_rmsnorm_group_quant_e8m0,
    mi_fused_normquant_gemm_pair,
    mi_fused_normquant_gemm_pair_launches,
    mi_gemm_capabilities,
    mi_preferred_weight_layout,
    mi_group_quant_1x128,
    mi_rmsnorm_group_quant,
    mi_negotiate_scale_layout,
    mi_status_string,
    mi_init,
    prepare_block_scaled_fp8_gemm,
    prepare_block_scaled_fp8_gemm_pair,
    prepare_fused_dual_rmsnorm_group_quant,
    prepare_fused_dual_rmsnorm_group_quant_e8m0,
    prepare_fused_normquant_gemm_pair,
    prepare_group_quant_1x128,
    prepare_rmsnorm_group_quant,
    relayout_weight,
    scale_is_transposed,
    untile_weight,
    weight_already_tiled,
)
