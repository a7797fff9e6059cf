"""Seeded synthetic workloads for paged-KV attention.

This module stands in for the block manager and the request generator of a
serving engine: it draws sequence lengths, hands out physical block ids and
fills the cache pool and the new Q/K/V rows with seeded N(0, 1) data rounded
to bfloat16.  It holds none of the attention arithmetic and does not compute
slot numbers or any other per-token metadata: that is the job of the
metadata step being tested (and of the oracle's own copy of it).

Both the GPU path and the CPU oracle consume what this module produces.
"""
from .configs import CONFIGS, CONFIG_ORDER, config_seed
from .gen import SeqState, Plan, Tensors, make_plan, make_tensors, custom_plan, NAN_BF16_BITS

__all__ = [
    "CONFIGS", "CONFIG_ORDER", "config_seed", "SeqState", "Plan", "Tensors",
    "make_plan", "make_tensors", "custom_plan", "NAN_BF16_BITS",
]
