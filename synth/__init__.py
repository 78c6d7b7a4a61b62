"""Seeded synthetic MoE-layer workloads.

This package only draws inputs: hidden states, router weights, the per-expert
int4 weight pool and the expert-to-slot table.  It holds none of the layer's
forward arithmetic (routing, regrouping, dequantisation, FFN, combine); both
the CPU oracle and the HIP path consume what it produces.
"""

from .layers import (  # noqa: F401
    CASES,
    Case,
    LayerShape,
    Weights,
    bf16_bits_from_f32,
    case_shape,
    draw_dense_expert,
    make_case,
    make_hidden,
    make_weights,
)
