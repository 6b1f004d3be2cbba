"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This package only draws random inputs and lays them out (shapes, host ranges);
it holds none of the method's arithmetic (no scoring, selection or cache logic).
"""
from .configs import WORKLOADS, Workload, get  # noqa: F401
from .gen import Inputs, make_inputs, seed_for  # noqa: F401
