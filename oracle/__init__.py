"""The oracle: a plain, slow CPU statement of what the AWQ hot path computes.

TEST INFRASTRUCTURE ONLY.  Import it from tests, from the package's smoke check
and from the bench's CPU-baseline leg; the product path never imports it.

The oracle is the C++ implementation in awq_oracle.cpp (built by
`__graft_entry__.build()` into liboracle.so with g++, IEEE fp32 quantizer, fp64
dequantization, loss and product), reached through cpp_oracle.py.  awq_oracle.py
is a second, independent coding of the same method in numpy (BLAS matmuls as
single steps), exported as `numpy_reference`: the pins run on both, and the two
must agree (tests/test_oracle_cross.py).

Parity status per function (what pins it is in the tests named here):
  channel_mean_abs   pinned: exact sums vs math.fsum, constant columns, sign flips
  scales_for_alpha   pinned: alpha = 0, a = 0, powers of two, monotonicity
  quantize_groups    pinned: brute-force nearest code, error bound, hand-worked groups,
                     power-of-two scale covariance, code ranges; the C++ fp32 -> fp16
                     conversion of the step against the host F16C instruction on all 2^32
                     patterns; numpy's cast against an integer-only round-to-nearest-even
  dequantize / effective_weight / weight_error
                     pinned: lossless on-grid construction, scaling invariance
  output_mse / output_mse_gram
                     pinned: Gram identity = direct form, brute-force loops, zero loss
  search             pinned: alpha = 0 is round-to-nearest, L(alpha*) <= L(0),
                     forced tie, known-answer construction
  gemm               pinned: brute-force loops, one-hot inputs, codes = zeros
  scaled_input       pinned: s = 1 identity, powers of two exact, nearest fp16 to the exact
                     quotient (brute force), product = unscaled layer within the rounding bound
  top_channels / keep_fp16_error / keep_fp16_ablation
                     pinned: hand-built rankings with ties, keeping every channel gives 0,
                     keeping none is the alpha = 0 search loss, brute-force loops with the
                     kept columns removed, Gram form = direct form
"""
import numpy as _np

from . import awq_oracle as numpy_reference  # noqa: F401
from .cpp_oracle import (  # noqa: F401
    alpha_grid,
    channel_mean_abs,
    scales_for_alpha,
    scale_weights,
    quantize_groups,
    dequantize,
    scaled_input,
    effective_weight,
    weight_error,
    output_mse,
    gram,
    output_mse_gram,
    quantize_at,
    search,
    gemm,
    top_channels,
    keep_fp16_error,
    keep_fp16_ablation,
    f32_to_f16_bits,
)

# Smallest normal fp16 value: the floor of a group's step.
SCALE_FLOOR = _np.float32(2.0 ** -14)
