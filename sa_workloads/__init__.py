"""Seeded synthetic workloads for the sparse-attention path.

This package only draws random inputs and names shapes. It contains none of the method's arithmetic, so both the
CPU oracle (``oracle/``) and the HIP path may take their inputs from it.
"""
from .configs import WORKLOADS, Workload, get_workload
from .gen import make_inputs, to_storage

__all__ = ["WORKLOADS", "Workload", "get_workload", "make_inputs", "to_storage"]
