"""Seeded synthetic inputs for the RT-Lynx sparse + LoRA linear layer.

This package only draws random numbers and rounds them to bf16.  It holds none
of the layer's arithmetic, so both the CPU oracle's tests and the HIP path's
tests and benchmark may use it without sharing any part of the method.
"""
from .generators import (  # noqa: F401
    BLOCK_LAYER_NAMES,
    CONFIGS,
    LayerInputs,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_layer,
    make_config,
    make_activation,
    make_weights,
)
