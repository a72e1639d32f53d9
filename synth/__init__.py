"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the bench.

Nothing here computes any step of the MoE layer; it only draws inputs.
"""
from . import configs, inputs  # noqa: F401
