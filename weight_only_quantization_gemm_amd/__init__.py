"""AWQ W4A16 on MI355X: activation-aware scale search, group-wise int4 packing
and the W4A16 GEMV/GEMM, as hand-written HIP kernels for gfx950 behind the C ABI
of libawq.so (include/awq.h).  This package is the thin Python binding: torch
allocates device memory and provides streams; every step runs in the library.
"""
from ._lib import LIB_PATH, AwqError, load  # noqa: F401
from .api import (  # noqa: F401
    ABLATION_ORDER,
    GROUP,
    MAX_ALPHAS,
    awq_ablation_workspace_bytes,
    awq_channel_mean_abs,
    awq_gemm,
    awq_gemm_kernel,
    awq_gemm_scaled,
    awq_gemm_scaled_workspace_bytes,
    awq_gemm_workspace_bytes,
    awq_keep_fp16_ablation,
    awq_last_error,
    awq_pack,
    awq_packed_bytes,
    awq_quantize,
    awq_quantize_workspace_bytes,
    awq_scale_input,
    awq_scales_bytes,
    awq_status_string,
    awq_unpack,
    awq_version,
    awq_zeros_bytes,
    bits_of,
    default_alpha_grid,
    empty_packed,
    packed_words,
)
