"""CPU float64 oracle for SLA2 sparse-linear attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py, never by the GPU library. It shares no code with the GPU path; both are
fed from the separate ``workloads`` input generators.
"""
from . import sla_oracle, fp8, pisa, backward
from .sla_oracle import forward, route, route_head, forward_head
from .fp8 import forward_fp8

__all__ = ["sla_oracle", "fp8", "pisa", "backward", "forward", "route", "route_head", "forward_head", "forward_fp8"]
