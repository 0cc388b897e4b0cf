"""Seeded synthetic inputs for the SVDQuant W4A4 + low-rank linear layer.

This module only draws random numbers and stores them in the input
dtypes (bf16 / fp32).  It holds none of the layer's arithmetic: no
smoothing, no decomposition, no quantization and no product.  Both the
HIP path (through its Python binding) and the CPU oracle consume what it
returns; neither is imported here.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    SEEDS,
    LayerSpec,
    bf16_bits_from_f32,
    bf16_bits_to_f32,
    draw_activations,
    draw_layer,
    draw_qkv_extras,
    draw_raw,
    draw_w4a16,
    layer_spec,
)
