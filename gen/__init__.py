"""Seeded synthetic attention layers ("planted-v1") shared by the HIP path and the oracle.

This package only draws inputs: Gaussian Q/K/V, rotary position embedding,
planted vertical-slash / query-aware structure, bf16 rounding and the per-token
int8 quantisation that the W8A8 variant consumes.  It contains none of the
sparse-prefill method's own arithmetic (no softmax, pooling, divergence,
selection or attention).
"""
from .planted import (  # noqa: F401
    CONFIGS,
    LayerConfig,
    Layer,
    make,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    quantize_rows,
    rope_tables,
    projection_inputs,
)
