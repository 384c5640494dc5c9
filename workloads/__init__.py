"""Seeded synthetic workloads for the Muon / MONA step.

This package only draws random numbers and lays out shapes: it holds none of
the optimizer's arithmetic.  Both the HIP path and the fp64 oracle consume the
tensors it returns.
"""
from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    make_state,
    make_grads,
    make_sketch,
    seed_for,
    workload_sketch,
)
