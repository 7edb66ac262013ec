"""Seeded synthetic inputs for the fused W4A16 MoE layer.

This package is shared by the CPU oracle's tests and by the GPU harness. It holds
no arithmetic of the layer itself: it only draws random numbers (activations,
router scores, fp32 weights, raw FP4/FP8 code bytes) with fixed seeds and the
shapes of the five workloads. Quantisation to FP4 codes is *not* here: tests do
that through the oracle; the GPU benchmark draws raw code bytes directly.
"""

from .configs import CONFIGS, Workload, get_config  # noqa: F401
from .draw import (  # noqa: F401
    draw_routing,
    draw_activations_bf16,
    draw_normal_weights,
    draw_random_codes,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
)
