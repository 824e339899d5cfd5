"""Seeded synthetic inputs for the selective-scan workloads.

This module is shared by the oracle side and the GPU side of the tests and the
benchmark.  It only draws random numbers and encodes them (float32, bfloat16
bits); it holds no step of the scan itself.  The recipes follow the five
synthetic workloads the method is measured on (shapes, dtypes, distributions);
the seeds (5400 + k for workload k, 5406 for the decode step, 5407 for the Mamba block, numpy PCG64) and the draw order (x, Delta
or u, B, C, then W_x, W_dt, Delta0) are fixed so that every run sees the same
values.
"""
from .synth import (  # noqa: F401
    SCAN_WORKLOADS,
    WORKLOADS,
    Workload,
    bf16_bits_from_float32,
    bf16_bits_to_float32,
    generate,
    generate_block,
    generate_extras,
    generate_step,
    to_float64,
    workload,
)
