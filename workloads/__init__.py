"""Seeded synthetic decode workloads.

This package is shared by the fp64 oracle tests, the GPU parity tests and the
benchmark.  It only draws random inputs and lays them out in memory; it holds
none of the method's arithmetic (no pooling, no gate score, no selection, no
attention).
"""

from .configs import WORKLOADS, Workload, get_workload
from .gen import Case, GateWeights, make_case, make_gate_weights

__all__ = ["WORKLOADS", "Workload", "get_workload", "Case", "make_case", "GateWeights",
           "make_gate_weights"]
