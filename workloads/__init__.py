"""Seeded synthetic inputs and the named workloads.

This package holds no part of the attention method: only shapes, seeds and
the random draws that both the HIP path and the CPU oracle consume.  Nothing
here pools, scores, selects or attends.
"""
from .configs import WORKLOADS, Workload, get_workload, custom_workload
from .gen import make_inputs, make_embedding, head_gains

__all__ = [
    "WORKLOADS",
    "Workload",
    "get_workload",
    "custom_workload",
    "make_inputs",
    "make_embedding",
    "head_gains",
]
