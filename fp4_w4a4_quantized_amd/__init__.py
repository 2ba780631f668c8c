"""fp4q: block-scaled FP4 (NVFP4 / MXFP4) W4A4 linear layers with sparse
residual compensation, for AMD Instinct MI355X (gfx950).

The product is the C-ABI library ``libfp4q.so`` (include/fp4q.h); this
package holds its HIP sources (``csrc/``), the build step (``build``) and a
thin ctypes binding (``binding``).
"""
from .binding import (  # noqa: F401
    BLOCK,
    MXFP4,
    NVFP4,
    OUT_BF16,
    OUT_F32,
    ROWMAJOR,
    TILED,
    Fp4qError,
    comp_weights,
    comp_weights_bytes,
    comp_weights_into,
    error_decompose,
    error_decompose_into,
    error_decompose_workspace_bytes,
    gemm,
    gemm_into,
    gemm_prepared,
    gemm_prepared_into,
    gemm_residual_fp4,
    gemm_residual_fp4_into,
    gemm_residual_fp4_workspace_bytes,
    gemm_workspace_bytes,
    grouped_comp_weights,
    grouped_comp_weights_bytes,
    grouped_gemm,
    grouped_gemm_prepared,
    grouped_gemm_prepared_into,
    grouped_gemm_into,
    grouped_gemm_workspace_bytes,
    lib,
    packed_bytes,
    permute_quantized,
    permute_quantized_into,
    quantize,
    quantize_into,
    quantize_workspace_bytes,
    select_channels,
    select_channels_into,
    select_channels_workspace_bytes,
)
