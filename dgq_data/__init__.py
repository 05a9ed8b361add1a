"""Seeded synthetic KV-cache workloads shared by the CPU oracle's tests and the GPU path.

This package only draws random inputs (keys, values, queries, sequence lengths, block tables).
It holds none of the compression or attention arithmetic, so both sides can use it without
sharing any part of the method.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    WorkloadConfig,
    get_config,
    sigma_profile,
    head_kv,
    head_profile,
    batch_kv,
    batch_kv_device,
    queries,
    seq_lens,
    block_tables,
)
