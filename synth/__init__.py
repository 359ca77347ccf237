"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This package holds no arithmetic of the ARL2 layer itself: only random draws, the
bf16 round-to-nearest-even used to hand identical values to both sides, and the
workload shapes.
"""
from .arl2_inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_gate_weights,
    make_gates,
    make_hidden,
    make_out_grad,
    make_pass_inputs,
    make_phi,
    make_state_grad,
    round_bf16,
)
