"""Seeded synthetic inputs shared by the oracle's tests, the GPU parity tests and the bench.

This package only draws random tensors (workload definitions and a gradient stream).
It holds none of the optimizer's arithmetic: no top-k, no projection, no Adam.
"""
from .gen import CONFIGS, Workload, GradStream, init_weights, to_storage, storage_to_f32

__all__ = ["CONFIGS", "Workload", "GradStream", "init_weights", "to_storage", "storage_to_f32"]
