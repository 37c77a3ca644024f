"""Seeded synthetic inputs for GQLA decode attention.

This package is shared by the fp64 oracle's tests and by the HIP path's tests and
benchmark. It holds no attention arithmetic: it only draws Gaussian numbers, applies
the rotary position embedding to the RoPE slices (input preparation, the decode path
receives post-RoPE values), rounds to the storage dtype, and scatters logical tokens
into a paged cache through a block table.
"""
from .shapes import WORKLOADS, Workload, workload
from .generate import (
    Inputs,
    generate,
    queries_for,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    rope_rotate,
)

__all__ = [
    "WORKLOADS",
    "Workload",
    "workload",
    "Inputs",
    "generate",
    "queries_for",
    "bf16_bits_to_f64",
    "f64_to_bf16_bits",
    "rope_rotate",
]
