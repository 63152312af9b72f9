"""Seeded synthetic inputs for SLA2 sparse-linear attention.

This package holds data generation only (shapes, random draws, bf16 storage rounding).
It contains none of the attention method's arithmetic, so both the CPU oracle and the
GPU library may be fed from it without sharing any part of the computation.
"""
from .generators import (CONFIGS, Problem, Inputs, make_inputs, make_custom,
                         bf16_round_bits, bf16_bits_to_f32, sha256_of)

__all__ = ["CONFIGS", "Problem", "Inputs", "make_inputs", "make_custom",
           "bf16_round_bits", "bf16_bits_to_f32", "sha256_of"]
