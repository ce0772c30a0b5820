"""Seeded synthetic inputs for the Kamera rehydrate operator.

This package only draws random numbers and lays them out. It holds none of the
operator's arithmetic (no rotation, no patch, no output rounding), so both the
fp64 oracle and the HIP path can consume what it produces without sharing any
of the method's code.
"""
from .configs import (  # noqa: F401
    CONFIG_NAMES,
    FactorSpec,
    ChunkSpec,
    LayoutSpec,
    Workload,
    make_workload,
)
