"""Seeded synthetic inputs for the FlashNorm norm-then-project workloads.

This module is shared by the CPU oracle and the GPU path as *input* only: it
draws random numbers and stores them in the dtype a workload uses. It holds
none of the method's arithmetic (no normalisation, no folding, no matmul).
"""

from .gen import (  # noqa: F401
    BF16,
    F32,
    Workload,
    bf16_bits_from_f32,
    bf16_bits_to_f64,
    normal,
    splitmix64_mix,
    stored_to_f64,
    uniform01,
    workload,
    WORKLOADS,
)
