"""Seeded synthetic inputs for banded sparse self-attention.

This package is shared by the fp64 oracle's tests, the GPU parity tests and the benchmark.
It holds input preparation only: random draws, bf16 rounding, the partial rotary
pre-rotation that the causal sliding-window workload applies to Q and K before attention, and
the structure of each attention pattern (global positions, key padding, block layout).  None of
the attention arithmetic lives here, and nothing here imports the oracle or the HIP library.
"""

from .configs import WORKLOADS, Workload, workload
from .gen import (
    Inputs,
    bf16_bits_to_f32,
    bigbird_layout,
    draw_dout,
    make_inputs,
    random_case,
    round_to_bf16_bits,
    widen,
)

__all__ = [
    "WORKLOADS",
    "Workload",
    "workload",
    "Inputs",
    "bf16_bits_to_f32",
    "bigbird_layout",
    "draw_dout",
    "make_inputs",
    "random_case",
    "round_to_bf16_bits",
    "widen",
]
