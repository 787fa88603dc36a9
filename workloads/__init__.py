"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This package only draws and shapes inputs.  It holds none of the method's own
arithmetic (no block representatives, scores, selection or attention): those live
in ``oracle/`` (CPU reference) and in the HIP library (the product).
"""
from .gen import CONFIGS, Workload, round_bf16, bf16_bits_to_f32, f32_to_bf16_bits

__all__ = ["CONFIGS", "Workload", "round_bf16", "bf16_bits_to_f32", "f32_to_bf16_bits"]
