"""Closed-form KV-cache sizing from the pages (test infrastructure, part of the oracle).

Each function restates one formula the pages give; the tests pin them against the worked
numbers the pages print (``tests/golden/sizing_examples.json``).
"""
from __future__ import annotations

import math


def kv_bytes(num_layers: int, num_kv_heads: int, head_dim: int, seq_len: int, dtype_bytes: int,
             batch_size: int = 1) -> int:
    """Bytes of K and V for `batch_size` sequences of `seq_len` tokens.

    "KV-Cache Management and PagedAttention" (adversariallm.ai), section "Why the cache exists,
    and why it's so hungry": 2 (K and V) x layers x kv heads x head dim x tokens x element bytes
    x batch. Same product as "PagedAttention and KV Cache Management" (blog.sejan.dev), section
    "The KV Cache Size Equation".
    """
    return 2 * num_layers * num_kv_heads * head_dim * seq_len * dtype_bytes * batch_size


def block_bytes(block_size: int, num_layers: int, num_kv_heads: int, head_dim: int,
                dtype_bytes: int) -> int:
    """Bytes of one physical block across all layers, K and V.

    "PagedAttention and KV Cache Management", section "How Block Paging Operates During
    Generation", item 3: B x 2 x n_layers x n_heads x d_head x dtype_size.
    """
    return block_size * 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """On-demand allocation: blocks for a prompt of num_tokens ("PagedAttention and KV Cache
    Management", section "How Block Paging Operates During Generation", item 1)."""
    return -(-num_tokens // block_size)


def wasted_slots(num_tokens: int, block_size: int) -> int:
    """Unwritten slots of a sequence's last block (item 4 of the same section: at most B-1)."""
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


def capacity_plan(gpu_mem: float, weights: float, activations: float,
                  kv_bytes_per_token: float, avg_tokens_per_request: float):
    """("KV-Cache Management and PagedAttention", section "Planning capacity when context gets
    long") kv_budget = gpu_mem - weights - activations; tokens_max = kv_budget / bytes per token;
    concurrency = tokens_max / average tokens per request."""
    kv_budget = gpu_mem - weights - activations
    tokens_max = kv_budget / kv_bytes_per_token
    concurrency = tokens_max / avg_tokens_per_request
    return kv_budget, tokens_max, concurrency


def reservation_idle_fraction(used_tokens: int, reserved_tokens: int) -> float:
    """Share of a contiguous max-length reservation left empty ("PagedAttention and KV Cache
    Management", section "The Three Forms of Memory Waste", item 1)."""
    return 1.0 - used_tokens / reserved_tokens


def reserved_but_unused(used_tokens: int, reserved_tokens: int) -> int:
    """Slots reserved and never written ("PagedAttention and KV Cache Management", section "The
    Memory Fragmentation Crisis in Traditional Serving", the three-request flowchart)."""
    return reserved_tokens - used_tokens


def truncate(x: float, decimals: int) -> float:
    """Cut (not round) to a number of decimals, as the pages print some figures."""
    f = 10 ** decimals
    return math.floor(x * f) / f
