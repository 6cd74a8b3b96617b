"""Fused weight-gradient GEMM + optimizer step for AMD MI355X (gfx950).

A thin binding over the C ABI in include/forge.h (libforge.so, built in-tree by
``python -m weight_gradient_gemm_amd.build``). Every step of the path runs in
the library's HIP kernels; this module only turns torch tensors into device
pointers and sizes and passes the current HIP stream. There is no CPU path:
if the library is missing, importing the entry points raises.
"""
from ._lib import (  # noqa: F401
    FORGE_TILE_128x128,
    FORGE_TILE_256x128,
    FORGE_TILE_256x256,
    FORGE_TILE_PERSISTENT,
    FORGE_TILE_DEFAULT,
    FORGE_BF16,
    FORGE_F32,
    FORGE_FP8_E4M3,
    FORGE_FP8_E5M2,
    ForgeError,
    STATUS,
    forge_adamw,
    forge_adamw_mixed,
    forge_dgrad,
    forge_dgrad_bf16w,
    forge_grouped_wgrad_adamw,
    forge_grouped_wgrad_sgdm,
    forge_linear_backward_adamw,
    forge_linear_backward_adamw_bf16w,
    forge_linear_backward_sgdm,
    forge_linear_backward_sgdm_bf16w,
    forge_sgdm,
    forge_status_string,
    forge_wgrad,
    forge_wgrad_adamw,
    forge_wgrad_adamw_bf16state,
    forge_wgrad_adamw_bf16w,
    forge_wgrad_adamw_fp8,
    forge_wgrad_bf16,
    forge_wgrad_fp8,
    forge_wgrad_sgdm,
    forge_wgrad_sgdm_bf16w,
    library,
    library_path,
)
