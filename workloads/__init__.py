"""Seeded synthetic inputs for paged-KV append/decode attention.

This module only draws random inputs (queries, raw cache bytes, scales,
lengths and block tables).  It performs none of the attention arithmetic,
so both the CPU oracle and the GPU path can consume its arrays without
sharing any of the method's code.
"""
from .synth import (  # noqa: F401
    Workload,
    CONFIGS,
    make_workload,
    config_workload,
    small_variant,
    kv_write_inputs,
)
