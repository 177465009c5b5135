"""Seeded synthetic inputs for paged attention: pools, block tables, lengths, queries.

Holds input construction only (value draws, a minimal block manager, the five
workload recipes). It computes no attention and is imported by the tests, the
bench and the oracle's tests alike.
"""
from .block_manager import BlockManager, PoolExhausted
from .configs import CONFIG_NAMES, Workload, build_decode_workload, make_workload
from .hints import share_prev_hint
from .rng import element_bytes, f32_to_bf16_bits, normal_values

__all__ = ["BlockManager", "PoolExhausted", "CONFIG_NAMES", "Workload",
           "build_decode_workload", "make_workload", "element_bytes",
           "f32_to_bf16_bits", "normal_values", "share_prev_hint"]
