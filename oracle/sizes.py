"""Oracle: closed-form sizes and waste figures (TEST INFRASTRUCTURE).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.
Each function is the plain definition of a quantity the pages print; the
tests pin them to the printed numbers.
"""

from __future__ import annotations

import math


def block_elements(block_size: int, num_heads: int, head_dim: int) -> int:
    """Elements in one physical block holding K and V of ``block_size`` tokens for
    every head of one layer ([PA] §3.1 "物理块分配器设计": tokens x heads x dim x 2)."""
    return block_size * num_heads * head_dim * 2


def kv_bytes_per_token(num_layers: int, num_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V bytes one token occupies across all layers ([KVM] Part 1
    "内存成本的量化分析": the LLaMA-2-13B fp16 example)."""
    return 2 * num_layers * num_heads * head_dim * elem_bytes


def contiguous_utilization(used_tokens: int, reserved_tokens: int) -> float:
    """Share of a contiguous per-request reservation that holds tokens
    ([PA] §1: mean generation 256 tokens against a 4096-token reservation)."""
    return used_tokens / reserved_tokens


def contiguous_waste(used_tokens: int, reserved_tokens: int) -> float:
    """Share of a contiguous reservation left unused ([KVM] Part 2 "朴素方案的内存碎片噩梦")."""
    return 1.0 - used_tokens / reserved_tokens


def paged_waste_slots(context_len: int, block_size: int) -> int:
    """Unused slots in a sequence's last block under paging ([KVM] Part 2
    "碎片问题的解决": at most B-1 per request)."""
    return math.ceil(context_len / block_size) * block_size - context_len


def contiguous_bytes(num_requests: int, max_len: int, num_heads: int, head_dim: int,
                     elem_bytes: int, num_layers: int = 1) -> int:
    """Memory of the contiguous-preallocation scheme of [PA] §1,
    sum over requests of 2 x L_max x h x d x bytes (times layers; the page's
    formula is per layer)."""
    return num_requests * 2 * max_len * num_heads * head_dim * elem_bytes * num_layers
