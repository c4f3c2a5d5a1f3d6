"""Seeded synthetic inputs for the sparse MoE layer.

This module only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic (no routing, no expert math), so the
oracle and the HIP path can both consume its output without sharing code.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    SEED_BASE,
    MoEInputs,
    bf16_bits_from_f32,
    bf16_bits_to_f32,
    make_config_inputs,
    make_inputs,
)
