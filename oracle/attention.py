"""Oracle: paged single-query decode attention in float64 (TEST INFRASTRUCTURE).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.

What is computed, following the pages:

* [VM] "PagedAttention的注意力计算流程" and [KVM] Part 2 "PagedAttention 的核心
  思想": for each request and head, read the list of physical blocks from the
  request's block table, read the Keys of those blocks and take their dot
  products with the query, normalise with softmax, then weight the Values of
  the same blocks and sum. The kernel reassembles the logical K/V sequence from
  scattered physical blocks, so the oracle does exactly that: it gathers the
  sequence's blocks, in logical order, into one contiguous array and runs
  plain dense attention on it.
* [VM] "Python 演示" note 9: softmax subtracts the maximum before
  exponentiating.
* [PA] §5.1 "分块Softmax算法": the five-step blockwise softmax (local maxima per
  block, global maximum, exponentials shifted by it, global sum, weights).
  ``blockwise_softmax`` follows those steps; ``partitioned_decode_one`` applies
  the same steps at the granularity of context partitions and merges them.

Readings taken where the pages are silent:
  * cache layout ``[num_blocks][num_kv_heads][block_size][head_dim]`` per layer,
    K and V in separate arrays (the pages only say a block is contiguous and is
    reached by base + offset, [PA] §3.2);
  * the scale is passed in (1/sqrt(head_dim) for every workload);
  * query head h reads KV head h // (num_q_heads // num_kv_heads);
  * a context length of 0 gives an all-zero output.
"""

from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np
import torch


def to_f64(x) -> np.ndarray:
    """Exact upcast of an fp32/fp16/bf16 tensor or array to float64."""
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def gather_sequence(cache: np.ndarray, block_table: Sequence[int], context_len: int) -> np.ndarray:
    """The first ``context_len`` token rows of one sequence, in logical order.

    ``cache`` is ``[num_blocks, num_kv_heads, block_size, head_dim]``. Logical
    block j of the sequence lives in physical block ``block_table[j]``
    ([PA] §3.2: logical block j -> table[j] -> physical id -> base + offset).
    Returns ``[context_len, num_kv_heads, head_dim]``.
    """
    _, H, B, d = cache.shape
    n_blocks = -(-context_len // B)
    rows = np.empty((n_blocks * B, H, d), dtype=cache.dtype)
    for j in range(n_blocks):
        phys = int(block_table[j])
        if not 0 <= phys < cache.shape[0]:
            raise IndexError(f"block table entry {j} = {phys} outside the pool")
        # block j holds tokens j*B .. j*B+B-1; inside it, [head][offset][dim]
        rows[j * B:(j + 1) * B] = cache[phys].transpose(1, 0, 2)
    return rows[:context_len]


def dense_decode_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Single-query attention for one sequence over contiguous K/V, float64.

    q ``[Hq, d]``, K and V ``[ctx, Hkv, d]``; returns ``[Hq, d]``.
    s_t = scale * q_h . K_t ; w = softmax(s) (max subtracted) ; out_h = sum_t w_t V_t.
    """
    Hq, d = q.shape
    ctx, Hkv, _ = K.shape
    out = np.zeros((Hq, d), dtype=np.float64)
    if ctx == 0:
        return out
    group = Hq // Hkv
    for h in range(Hq):
        kv = h // group
        s = scale * (K[:, kv, :] @ q[h])
        m = s.max()
        e = np.exp(s - m)
        w = e / e.sum()
        out[h] = w @ V[:, kv, :]
    return out


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float) -> np.ndarray:
    """Oracle of ``pa_decode``: per sequence, gather its blocks through its block
    table, then dense fp64 attention. ``q`` ``[S, Hq, d]``; caches
    ``[N, Hkv, B, d]``; ``block_tables`` a list (or 2-D array) of physical ids
    per sequence; ``context_lens`` ``[S]``. Returns float64 ``[S, Hq, d]``."""
    q64 = to_f64(q)
    kc = to_f64(k_cache) if not isinstance(k_cache, np.ndarray) or k_cache.dtype != np.float64 else k_cache
    vc = to_f64(v_cache) if not isinstance(v_cache, np.ndarray) or v_cache.dtype != np.float64 else v_cache
    S = q64.shape[0]
    out = np.zeros_like(q64)
    for s in range(S):
        ctx = int(context_lens[s])
        K = gather_sequence(kc, block_tables[s], ctx)
        V = gather_sequence(vc, block_tables[s], ctx)
        out[s] = dense_decode_one(q64[s], K, V, scale)
    return out


def blockwise_softmax(scores: np.ndarray, block_size: int) -> np.ndarray:
    """The five steps of [PA] §5.1 over consecutive blocks of ``block_size`` scores:
    (1) local maximum m_j of each block, (2) global maximum as the max of the
    m_j, (3) exp(s - m_global), (4) global sum l as the sum of per-block sums,
    (5) w = exp(s - m_global) / l."""
    n = scores.shape[0]
    starts = range(0, n, block_size)
    local_max = [scores[i:i + block_size].max() for i in starts]          # step 1
    m_global = max(local_max)                                              # step 2
    e = np.exp(scores - m_global)                                          # step 3
    l_global = sum(e[i:i + block_size].sum() for i in starts)              # step 4
    return e / l_global                                                    # step 5


def partition_state(q_h: np.ndarray, K_kv: np.ndarray, V_kv: np.ndarray,
                    scale: float) -> Tuple[float, float, np.ndarray]:
    """Steps 1-4 of [PA] §5.1 restricted to one context partition: the
    partition's max m_p, its sum l_p = sum exp(s - m_p), and its normalised
    partial output o_p = sum exp(s - m_p) V / l_p."""
    s = scale * (K_kv @ q_h)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return m, l, (e @ V_kv) / l


def merge_partitions(states) -> np.ndarray:
    """Steps 2-5 of [PA] §5.1 across partitions: global max m = max_p m_p,
    global sum L = sum_p l_p exp(m_p - m), output = sum_p l_p exp(m_p - m) o_p / L."""
    m = max(st[0] for st in states)
    weights = [st[1] * math.exp(st[0] - m) for st in states]
    L = sum(weights)
    return sum(w * st[2] for w, st in zip(weights, states)) / L


def partitioned_decode_one(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                           partition_size: int) -> np.ndarray:
    """Split-context decode for one sequence: partitions of ``partition_size``
    tokens each produce (m_p, l_p, o_p); the merge combines them."""
    Hq, d = q.shape
    ctx, Hkv, _ = K.shape
    out = np.zeros((Hq, d), dtype=np.float64)
    if ctx == 0:
        return out
    group = Hq // Hkv
    for h in range(Hq):
        kv = h // group
        states = [partition_state(q[h], K[p:p + partition_size, kv], V[p:p + partition_size, kv], scale)
                  for p in range(0, ctx, partition_size)]
        out[h] = merge_partitions(states)
    return out
