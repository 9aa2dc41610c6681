"""Seeded synthetic inputs for the Block-Union KV Selection hot path.

This package only draws random numbers and lays them out (masks, Q, paged K/V, page maps).
It holds none of the method's arithmetic: no union, no table, no attention.  Both the CPU
oracle (through the tests) and the HIP library (through the tests and the benchmark) consume
what it produces.
"""
from .configs import (  # noqa: F401
    BLOCK,
    Workload,
    CONFIG_NAMES,
    make_config,
    make_workload,
    bf16_round,
    chunked_sequence_chunk,
)
