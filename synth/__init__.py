"""Seeded synthetic inputs for the QSA forward path.

This package only draws inputs (random tensors, planted needle blocks). It holds
none of the method's arithmetic and is shared by the tests, the benchmark and the
smoke check; neither the oracle nor the HIP library imports it.
"""
from .workloads import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits,
    decode_query_sets,
    generate,
    generate_varlen,
    serving_lengths,
    workload,
)
