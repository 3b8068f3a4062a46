"""MXFP8 MoE expert grouped-GEMM hot path for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``libmxfp8moe.so`` (include/mxfp8moe.h); this package is the thin Python
binding over it (torch supplies device memory and streams) plus the seeded
input generators.
"""

from .binding import (  # noqa: F401
    COLWISE, LAYOUT_NN, LAYOUT_NT, LAYOUT_TN, NOALLOC_SCRATCH_BYTES, ROWWISE, MXFP8Tensor,
    convert_sweep, dbias_workspace_bytes, group_quantize, group_quantize_requant,
    group_quantize_requant_noalloc, grouped_dbias, grouped_gemm, grouped_gemm_swiglu_quantize,
    grouped_gemm_wgrad_accumulate,
    grouped_scaled_bias_grad, gemm_workspace_bytes, requant_colwise, swiglu_bwd,
    swiglu_bwd_quantize, swiglu_fwd,
    swiglu_quantize, validate_splits)
from ._native import load as load_library, lib_path  # noqa: F401
