"""Seeded synthetic inputs for the FlashAttention forward workloads.

This package is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds input construction only: seeded draws, the fp32 -> bf16
encoding of those draws, and the packing descriptors (sequence lengths,
``cu_seqlens`` offsets, padding masks and ``indices``).  None of the attention
arithmetic lives here.
"""

from .gen import (  # noqa: F401
    Workload,
    bf16_bits_from_f32,
    normal_bf16,
    cu_seqlens_from_lengths,
    build_workload,
    WORKLOADS,
    SEEDS,
)
