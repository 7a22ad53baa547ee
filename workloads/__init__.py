"""Seeded synthetic inputs for the H2O chunked sparse-attention workloads.

This package is shared by the CPU oracle side (tests, the CPU baseline) and the
GPU side (tests, bench).  It draws random numbers and rounds them to the
storage precision; it holds none of the method's arithmetic.
"""
from .synth import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits,
    bf16_round,
    chunk_inputs,
    decode_initial_state,
    decode_step_inputs,
    heavy_boost,
    rng_for,
    steady_state,
    workload,
)
