"""Seeded synthetic inputs shared by the oracle's tests, the GPU parity tests and the bench.

This package only draws random tensors (workload definitions and a gradient stream).
It holds none of the optimizer's arithmetic: no top-k, no projection, no Adam.
"""
from .gen import (WORKLOADS, TINY_F32, F32_32x32x16x16, F16_4x64x64x64x64, C64_64x64x64x33,
                  BF16_64x64x48x48x25, Workload, GradStream, init_weights, to_storage, storage_to_f32)

__all__ = ["WORKLOADS", "TINY_F32", "F32_32x32x16x16", "F16_4x64x64x64x64", "C64_64x64x64x33",
           "BF16_64x64x48x48x25", "Workload", "GradStream", "init_weights", "to_storage", "storage_to_f32"]
