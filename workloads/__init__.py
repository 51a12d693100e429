"""Seeded synthetic decode workloads shared by tests and the benchmark.

This package only draws inputs (context lengths, page placement, block tables,
slot mappings, Q/K/V values).  It holds none of the attention arithmetic, so the
CPU oracle and the HIP path can both consume it without sharing any method code.
"""
from .configs import (  # noqa: F401
    CONFIGS,
    DecodeConfig,
    Workload,
    config_by_id,
    make_workload,
    make_custom_workload,
    make_chunk_queries,
    bf16_bits_from_f32,
)
