"""Seeded synthetic inputs for batched paged-KV decode attention.

This package draws page tables, KV page pools, per-page fp8 scales and query
tensors. It holds none of the attention arithmetic: both the float64 oracle
(through the tests) and the HIP path consume what it produces, and neither
one's numbers come from the other.
"""
from .synthetic import (  # noqa: F401
    CONFIGS,
    Workload,
    custom_workload,
    device_case,
    explicit_table,
    host_case,
    page_table,
    query_rows,
    read_mask,
)
