"""Seeded synthetic inputs (weights in stored form, activations, router logits).

Used by the tests, the benchmark and the smoke check on both sides of the
parity comparison. Draws numbers only; holds none of the method's arithmetic.
"""
from .configs import WORKLOADS, Workload, small_workload  # noqa: F401
from . import gen  # noqa: F401
