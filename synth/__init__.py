"""Seeded synthetic inputs for the Muon step and the AdamW step.

This module holds only random-number generation and shape bookkeeping: none
of the optimizer's arithmetic.  Both the CPU oracle (through the tests) and
the HIP library (through the tests and the benchmark) consume what it makes.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    MatrixSpec,
    bf16_bits_round,
    gaussian_f32,
    spectral_grad,
    spectral_grad_torch,
    matrix_inputs,
    adamw_inputs,
)
