"""Seeded synthetic inputs for the multi-LoRA projection.

This package only draws numbers, rounds them to the storage type and lays them out; it holds
none of the projection's arithmetic.  The HIP path (through its tests and the benchmark) and the
fp64 oracle both take their inputs from here, and from nowhere else.
"""
from .gen import (  # noqa: F401
    CONFIG_NAMES,
    Workload,
    build,
    custom,
    round_to_bf16,
    storage_to_f64,
)
