"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This package draws random numbers and shapes them into fp16 tensors of the
workloads' sizes and value laws. It holds none of the quantization method's
arithmetic: no statistics, scales, codes, losses or products.
"""
from .synth import (  # noqa: F401
    rng,
    normal_fp16,
    outlier_channels,
    activations_fp16,
    lognormal_profile,
)
from .workloads import WORKLOADS, Layer, seed_for  # noqa: F401
