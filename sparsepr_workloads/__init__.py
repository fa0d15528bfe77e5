"""Seeded synthetic workloads shared by the GPU path's tests/benchmark and the oracle.

Holds shapes, seeds and random-number recipes only; no attention arithmetic.
"""
from .configs import CONFIGS, Workload, small  # noqa: F401
from .generator import make_inputs, head_inputs, round_to_bf16  # noqa: F401
