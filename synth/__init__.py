"""Seeded synthetic workloads for the HHR decode path.

This package only draws random inputs (keys, values, queries, the per-head
R_h and W_h, sequence lengths); it holds none of the method's arithmetic.
Both the GPU library's tests/benchmark and the CPU oracle consume what it
makes.
"""
from .workloads import (WORKLOADS, Workload, bf16_bits_to_f32, f32_to_bf16_bits, keep_for,
                        make_layer, make_layer_torch)
from .scores import tie_scores

__all__ = ["WORKLOADS", "Workload", "make_layer", "make_layer_torch", "keep_for",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "tie_scores"]
