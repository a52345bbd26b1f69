"""Seeded synthetic inputs for the tree-attention + tree-verification path.

This package only draws random numbers and lays them out in the shapes the
library and the oracle consume. It holds none of the method's arithmetic (no
tree construction, no masking, no attention, no verification), so both the
oracle and the GPU path may use it without sharing any of the computation.
"""
from .configs import CONFIGS, WorkloadSpec, get_config
from .synth import Workload, make_workload, bf16_bits_to_f32, f32_to_bf16_bits

__all__ = [
    "CONFIGS",
    "WorkloadSpec",
    "get_config",
    "Workload",
    "make_workload",
    "bf16_bits_to_f32",
    "f32_to_bf16_bits",
]
