"""Seeded synthetic inputs for the MoE-layer workloads.

This package is the only code shared by the oracle-side tests and the GPU
path: it draws random tensors and encodes them as bf16/fp32 bit patterns.
It holds none of the layer's arithmetic (no routing, counting, permutation,
expert FFN or combine).
"""
from .configs import WORKLOADS, Workload, get_workload
from .gen import (
    Inputs,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_inputs,
    zipf_routing,
)

__all__ = [
    "WORKLOADS",
    "Workload",
    "get_workload",
    "Inputs",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "make_inputs",
    "zipf_routing",
]
