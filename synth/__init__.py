"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package draws random numbers and encodes them; it holds none of the
method's arithmetic (no contraction, no optimizer step).
"""
from .gen import (  # noqa: F401
    CONFIGS,
    DenseCase,
    GroupedCase,
    bf16_bits_from_f32,
    dense_case,
    dense_inputs,
    dense_inputs_f32,
    dense_inputs_fp8,
    fp8_bits_from_f32,
    fp8_inputs,
    fp8_scale,
    dense_state,
    grouped_case,
    grouped_inputs,
    grouped_state,
    lmhead_dy,
    moe_loads,
    moe_routing,
    normal_bf16,
    normal_f32,
)
