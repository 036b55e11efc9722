"""Seeded synthetic workloads shared by the oracle-side tests and the HIP path.

Holds shapes, random draws and the synthetic expert stage only.
"""
from .configs import (ALL, BY_NAME, DECODE, FUSED, PARTIALS, PREFILL, SKEWED, TINY,
                      PartialsWorkload, Workload)
from .inputs import (Inputs, bf16_bits_to_f32, draw_routing, draw_softmax_weights,
                     expert_outputs, f32_to_bf16_bits, make_inputs, make_partials,
                     region_messages)

__all__ = [
    "ALL", "BY_NAME", "DECODE", "FUSED", "PARTIALS", "PREFILL", "SKEWED", "TINY",
    "PartialsWorkload", "Workload", "make_partials",
    "Inputs", "bf16_bits_to_f32", "draw_routing", "draw_softmax_weights",
    "expert_outputs", "f32_to_bf16_bits", "make_inputs", "region_messages",
]
