"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the bench.

This package only draws random data (NumPy PCG64 on the host, or a seeded
torch generator on the device for the full-size workloads) and rounds it to
the storage precision.  It holds none of the method's arithmetic: no
projection, softmax, acceptance test or sampling.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_round,
    bf16_bits,
    gate_vector,
    gemm_inputs,
    verify_inputs,
    lm_head_inputs,
    layer_shapes,
)
