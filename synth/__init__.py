"""Seeded synthetic inputs for the decode-step weight stream.

This module is shared by the tests, the oracle's callers and the benchmark.  It
holds NONE of the method's arithmetic (no norm, product, epilogue or argmax):
it only draws seeded normal samples, rounds them to the storage type, and
describes the workloads' shapes.  Both the HIP path and the CPU oracle receive
the very same bits.
"""
from .gen import (  # noqa: F401
    normal, seed_of, bf16_bits_to_numpy, f16_bits_to_numpy,
    Workload, WORKLOADS, make_stage_tensors,
)
