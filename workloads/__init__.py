"""Seeded synthetic inputs for the FP4 W4A4 hot path.

This package is shared by the tests (oracle side and GPU side) and by the
benchmark.  It draws random tensors, rounds them to BF16 and picks the
compensated channel set; it holds none of the quantization, GEMM or error
decomposition arithmetic.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    bf16_bits,
    bf16_to_f32,
    dense_case,
    moe_case,
    moe_routing,
    top_variance_channels,
)
