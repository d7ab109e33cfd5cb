"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package holds random-number generation and data layout only: it draws
activations, weights and router logits with the shapes and value
distributions of the five workloads, and converts fp32 samples to bf16 bit
patterns.  It contains none of the quantization, selection, GEMM or MoE
arithmetic; the oracle (``oracle/``) and the HIP library each implement that
on their own.
"""
from .synthetic import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_activations,
    make_logits,
    make_weight,
    make_moe_weights,
    make_inputs,
    rng_for,
)
