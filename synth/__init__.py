"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This package draws random tensors, random lengths and random block-id orders.
It holds none of the attention, cache-write, scheduling or allocation
arithmetic: everything here is "what the input is", never "what the method
computes from it".
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    draw_normal,
    free_block_order,
    get_workload,
    prompt_qkv,
    config3_suffix_lengths,
    config4_decode_contexts,
)
