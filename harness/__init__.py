"""Seeded synthetic inputs and named workload shapes.

This package holds no arithmetic of the attention method: it draws random
numbers, rounds them to the storage precision, and names the shapes. Both the
HIP path (through tests and the bench) and the CPU oracle consume what it
produces.
"""
from .configs import MLAConfig, CONFIGS, get_config  # noqa: F401
from .gen import (  # noqa: F401
    round_to,
    to_bf16_bits,
    from_bf16_bits,
    layer_weights,
    query_weights,
    frame_tokens,
    chunk_queries,
)
