"""Seeded synthetic inputs for MiniMax Sparse Attention (MSA) workloads.

This package only draws random tensors of the shapes and value distributions
of the workloads; it holds none of the method's arithmetic (no pooling, no
scoring, no selection, no attention).  Both the HIP path and the CPU oracle
consume what it produces.
"""
from .configs import WORKLOADS, Workload, get_workload  # noqa: F401
from .gen import (  # noqa: F401
    decode_inputs,
    grad_output,
    prefill_inputs,
    sample_rows,
    seed_for,
)
