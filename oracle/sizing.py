"""KV-cache sizing (oracle).

* ``kv_cache_bytes`` is the per-request estimate of "Paged Attention Explained"
  (deepneuralai.in), section "Why Does the KV Cache Consume So Much Memory?":
  two tensors (K and V) x layers x cached tokens x KV heads x head dim x bytes
  per element.  A paged pool of N blocks of bs slots holds T = N*bs token slots.
* ``blocks_required`` is the block count of the same page, section "How Paged
  Attention Improves GPU Memory Utilization": cached tokens divided by tokens
  per block, rounded up; its error rules (negative token count, non-positive
  block size) follow the page's "Practical Example" illustration.
"""
from __future__ import annotations

import math


def kv_cache_bytes(layers: int, tokens: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * layers * tokens * kv_heads * head_dim * elem_bytes


def pool_bytes(layers: int, num_blocks: int, block_size: int, kv_heads: int, head_dim: int,
               elem_bytes: int) -> int:
    return kv_cache_bytes(layers, num_blocks * block_size, kv_heads, head_dim, elem_bytes)


def blocks_required(tokens: int, block_size: int) -> int:
    if tokens < 0:
        raise ValueError("token count cannot be negative")
    if block_size <= 0:
        raise ValueError("block size must be positive")
    return math.ceil(tokens / block_size)


def unused_slots(tokens: int, block_size: int) -> int:
    """Slots of the last block left empty (internal fragmentation)."""
    return blocks_required(tokens, block_size) * block_size - tokens
