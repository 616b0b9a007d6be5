"""Seeded synthetic workloads for batched draft-block verification.

This package only draws inputs (logits, lengths, temperatures, draft tokens and
uniforms). It contains none of the verification arithmetic, so both the CPU
oracle and the HIP path can take their inputs from it without sharing any of
the method's code.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    workload,
    make_workload,
    bf16_bits_from_f64,
    bf16_bits_to_f32,
)
