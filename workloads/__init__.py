"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the bench.

This package only describes shapes and draws random inputs.  It holds none of the
quantize / pack / attention arithmetic: the CPU oracle (``oracle/``) and the HIP
library (``quantized_decode_attention_kv_amd``) each implement that on their own.
"""

from .configs import WORKLOADS, Workload, workload, small_cases
from .synth import (
    SlabInputs,
    f32_to_bf16_bits,
    head_params,
    make_queries,
    make_slab,
    make_all,
)

__all__ = [
    "WORKLOADS",
    "Workload",
    "workload",
    "small_cases",
    "SlabInputs",
    "f32_to_bf16_bits",
    "head_params",
    "make_queries",
    "make_slab",
    "make_all",
]
