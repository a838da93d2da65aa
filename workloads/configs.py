"""The five decode workloads, as seeded synthetic inputs.

Every workload is a list of host operations (``DecodeStep``) on a pool of
fixed-size physical blocks, together with the numbers those operations
carry. Draws use ``numpy.random.default_rng`` streams spawned from one seed
per workload, so that the context lengths, the free-list order and the
K/V/q values each come from their own stream and stay the same when an
unrelated knob (the block size of the long-context sweep) changes.

Values are drawn as float32 N(0, 1) (times a per-workload factor) and then
rounded to the storage dtype with torch's round-to-nearest-even cast. Both
sides read the rounded values.

Nothing here computes a slot, a block table, a softmax or a copy.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np
import torch

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class DecodeStep:
    """One host operation of a workload.

    kind:
      ``add_seq``  - a new sequence ``seq_ids[0]`` holding ``num_tokens``
                     prompt tokens whose K/V rows are ``k``/``v``
                     ``[num_tokens, num_kv_heads, head_dim]`` in position order.
                     With prefix caching, ``tokens`` (int32 token ids) and
                     ``extra_key`` (an adapter id) identify the prompt; a
                     sequence without ``tokens`` is allocated plainly.
      ``fork``     - ``seq_ids = (parent, child)``: the child shares every
                     block of the parent.
      ``append``   - one new token for each sequence of ``seq_ids``, in that
                     order; ``k``/``v`` are ``[len(seq_ids), num_kv_heads,
                     head_dim]``, row i belonging to ``seq_ids[i]``.
      ``decode``   - one single-query attention for each sequence of
                     ``seq_ids``; ``q`` is ``[len(seq_ids), num_q_heads,
                     head_dim]``.
      ``swap_out`` - evict each sequence of ``seq_ids`` (in order) to the
                     swap space; ``swap_in`` brings them back.
      ``free``     - each sequence of ``seq_ids`` has finished.
    """

    kind: str
    seq_ids: Tuple[int, ...]
    num_tokens: int = 0
    k: Optional[torch.Tensor] = None
    v: Optional[torch.Tensor] = None
    q: Optional[torch.Tensor] = None
    tokens: Optional[np.ndarray] = None
    extra_key: int = 0


@dataclass
class Workload:
    name: str
    description: str
    dtype: str                      # "f32" | "f16" | "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    partition_size: int             # split-context partition (tokens); 0 = the library's default
    free_order: np.ndarray          # int32 [num_blocks], initial free-list order
    ops: List[DecodeStep] = field(default_factory=list)
    kv_cache_dtype: str = ""        # "" = the caches hold `dtype`; "fp8" / "int8" = codes + a scale per row
    num_swap_blocks: int = 0        # swap-space blocks (CPU memory) for swap_out / swap_in
    swap_free_order: Optional[np.ndarray] = None   # int32 [num_swap_blocks], initial swap free-list order
    prefix_caching: bool = False    # add_seq ops with tokens reuse indexed prompt blocks

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return {"f32": 4, "f16": 2, "bf16": 2}[self.dtype]

    @property
    def kv_bytes_per_token(self) -> int:
        """K+V bytes the cache holds per token (codes and scales for FP8)."""
        if self.kv_cache_dtype in ("fp8", "int8"):
            return 2 * self.num_kv_heads * (self.head_dim + 4)
        return 2 * self.num_kv_heads * self.head_dim * self.elem_bytes

    def max_context_len(self) -> int:
        """Longest context any decode op of the workload sees (plain bookkeeping
        over the op list: prompt lengths plus appended tokens)."""
        lens = {}
        best = 0
        for op in self.ops:
            if op.kind == "add_seq":
                lens[op.seq_ids[0]] = op.num_tokens
            elif op.kind == "fork":
                lens[op.seq_ids[1]] = lens[op.seq_ids[0]]
            elif op.kind == "append":
                for s in op.seq_ids:
                    lens[s] += 1
            elif op.kind == "decode":
                best = max(best, max(lens[s] for s in op.seq_ids))
        return best


def _streams(seed: int, n: int) -> List[np.random.Generator]:
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal(rng: np.random.Generator, shape, factor: float, dtype: str) -> torch.Tensor:
    x = rng.standard_normal(shape, dtype=np.float32)
    if factor != 1.0:
        x *= np.float32(factor)
    t = torch.from_numpy(x)
    return t if dtype == "f32" else t.to(_TORCH_DTYPES[dtype])


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _prompt_workload(name, description, seed, dtype, ctx, Hq, Hkv, d, B, factor,
                     num_blocks, n_steps=0, partition_size=0) -> Workload:
    """Independent sequences 0..S-1 with the given prompt lengths, one decode,
    then ``n_steps`` rounds of (append one token to every sequence, decode)."""
    r_perm, r_val = _streams(seed, 3)[1:]
    S = len(ctx)
    free_order = r_perm.permutation(num_blocks).astype(np.int32)
    q = _normal(r_val, (S, Hq, d), factor, dtype)
    total = int(sum(ctx))
    k_all = _normal(r_val, (total, Hkv, d), factor, dtype)
    v_all = _normal(r_val, (total, Hkv, d), factor, dtype)
    wl = Workload(name, description, dtype, Hq, Hkv, d, B, num_blocks,
                  1.0 / math.sqrt(d), partition_size, free_order)
    off = 0
    for s, n in enumerate(ctx):
        n = int(n)
        wl.ops.append(DecodeStep("add_seq", (s,), n, k_all[off:off + n], v_all[off:off + n]))
        off += n
    seqs = tuple(range(S))
    wl.ops.append(DecodeStep("decode", seqs, q=q))
    if n_steps:
        k_new = _normal(r_val, (n_steps, S, Hkv, d), factor, dtype)
        v_new = _normal(r_val, (n_steps, S, Hkv, d), factor, dtype)
        q_new = _normal(r_val, (n_steps, S, Hq, d), factor, dtype)
        for i in range(n_steps):
            wl.ops.append(DecodeStep("append", seqs, k=k_new[i], v=v_new[i]))
            wl.ops.append(DecodeStep("decode", seqs, q=q_new[i]))
    return wl


def tiny_paged_decode_f32(seed: int = 1, n_steps: int = 0) -> Workload:
    """Tiny single-layer decode in fp32: 4 sequences of 5, 16, 17 and 100
    tokens, 8 heads of dim 64, blocks of 16, a pool of 64 blocks in seeded
    random order. After the first decode, sequence 2 is forked into sequence
    4 (both of its blocks then have two owners), every sequence appends one
    token, and all five sequences decode again. ``n_steps`` further rounds
    append one token to each of the five and decode them (their values come
    from a stream of their own, so the ops above do not change)."""
    Hq = Hkv = 8
    d, B, N = 64, 16, 64
    ctx = [5, 16, 17, 100]
    wl = _prompt_workload("tiny_paged_decode_f32",
                          "4 seqs ctx {5,16,17,100}, 8 heads, d 64, B 16, 64 blocks, fp32",
                          seed, "f32", ctx, Hq, Hkv, d, B, 1.0, N)
    r_step = _streams(seed, 4)[3]
    k5 = _normal(r_step, (5, Hkv, d), 1.0, "f32")
    v5 = _normal(r_step, (5, Hkv, d), 1.0, "f32")
    q5 = _normal(r_step, (5, Hq, d), 1.0, "f32")
    wl.ops.append(DecodeStep("fork", (2, 4)))
    wl.ops.append(DecodeStep("append", (0, 1, 2, 3, 4), k=k5, v=v5))
    wl.ops.append(DecodeStep("decode", (0, 1, 2, 3, 4), q=q5))
    if n_steps:
        r_more = _streams(seed, 5)[4]
        for _ in range(n_steps):
            wl.ops.append(DecodeStep("append", (0, 1, 2, 3, 4), k=_normal(r_more, (5, Hkv, d), 1.0, "f32"),
                                     v=_normal(r_more, (5, Hkv, d), 1.0, "f32")))
            wl.ops.append(DecodeStep("decode", (0, 1, 2, 3, 4), q=_normal(r_more, (5, Hq, d), 1.0, "f32")))
    return wl


def llama7b_decode_f16(seed: int = 2, num_seqs: int = 64,
                       ctx_range: Tuple[int, int] = (1, 2048), n_steps: int = 0) -> Workload:
    """LLaMA-7B-shaped decode: 32 heads of dim 128, blocks of 16, fp16 KV,
    context lengths uniform in ``ctx_range``, values 0.5 * N(0, 1), pool =
    ceil(1.05 * blocks needed after ``n_steps`` append+decode rounds)."""
    r_ctx = _streams(seed, 3)[0]
    ctx = r_ctx.integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs).astype(np.int64)
    need = sum(_cdiv(int(c) + n_steps, 16) for c in ctx)
    N = int(math.ceil(1.05 * need))
    return _prompt_workload("llama7b_decode_f16",
                            f"{num_seqs} seqs ctx U[{ctx_range[0]},{ctx_range[1]}], 32 heads, d 128, B 16, fp16",
                            seed, "f16", ctx, 32, 32, 128, 16, 0.5, N, n_steps=n_steps)


def lognormal_context_lens(rng: np.random.Generator, n: int, median: float = 256.0,
                           sigma: float = 1.0, lo: int = 1, hi: int = 4096) -> np.ndarray:
    return np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, size=n))), lo, hi).astype(np.int64)


def llama2_13b_decode_f16(seed: int = 3, num_seqs: int = 128, n_steps: int = 16,
                          ctx_cap: int = 4096) -> Workload:
    """LLaMA-2-13B-shaped decode: 40 heads of dim 128, blocks of 16, fp16,
    context lengths log-normal (median 256, sigma 1, clipped to [1, 4096]).
    After the first decode, ``n_steps`` rounds each append one token to every
    sequence and decode again. Pool = ceil(1.05 * blocks needed after the
    last step)."""
    r_ctx = _streams(seed, 3)[0]
    ctx = lognormal_context_lens(r_ctx, num_seqs, hi=ctx_cap)
    need = sum(_cdiv(int(c) + n_steps, 16) for c in ctx)
    N = int(math.ceil(1.05 * need))
    return _prompt_workload("llama2_13b_decode_f16",
                            f"{num_seqs} seqs ctx lognormal(median 256, sigma 1, <= {ctx_cap}), "
                            f"40 heads, d 128, B 16, fp16, {n_steps} append+decode steps",
                            seed, "f16", ctx, 40, 40, 128, 16, 1.0, N, n_steps=n_steps)


def shared_prefix_beam_f16(seed: int = 4, num_groups: int = 32, beam_width: int = 4,
                           prompt_len: int = 2040, max_tail: int = 64, n_steps: int = 0) -> Workload:
    """Beam search / parallel sampling over a shared prompt, fp16, 32 heads of
    dim 128, blocks of 16. Each group's leader (sequence ``g * beam_width``)
    holds the ``prompt_len``-token prompt and is forked ``beam_width - 1``
    times. Each beam then grows a tail of U{0..max_tail} tokens, one append
    step at a time (at step t the beams whose tail is longer than t append, in
    ascending sequence id). A last step appends one token to every beam and
    decodes all of them; ``n_steps`` further rounds do the same."""
    Hq = Hkv = 32
    d, B = 128, 16
    r_ctx, r_perm, r_val = _streams(seed, 3)
    S = num_groups * beam_width
    tails = r_ctx.integers(0, max_tail + 1, size=S)
    # Pool sizing: per group the prompt's full blocks are stored once; every
    # beam owns the blocks past them (its copy of the partial prompt block
    # included) up to its final length.
    full = prompt_len // B
    need = 0
    for gi in range(num_groups):
        need += full
        for b in range(beam_width):
            final = prompt_len + int(tails[gi * beam_width + b]) + 1 + n_steps
            need += _cdiv(final, B) - full
    N = int(math.ceil(1.05 * need))
    free_order = r_perm.permutation(N).astype(np.int32)
    q = _normal(r_val, (S, Hq, d), 1.0, "f16")
    wl = Workload("shared_prefix_beam_f16",
                  f"{num_groups} groups x beam {beam_width}, shared {prompt_len}-token prompt, "
                  f"tails U[0,{max_tail}], 32 heads, d 128, B 16, fp16",
                  "f16", Hq, Hkv, d, B, N, 1.0 / math.sqrt(d), 0, free_order)
    pk = _normal(r_val, (num_groups, prompt_len, Hkv, d), 1.0, "f16")
    pv = _normal(r_val, (num_groups, prompt_len, Hkv, d), 1.0, "f16")
    for gi in range(num_groups):
        lead = gi * beam_width
        wl.ops.append(DecodeStep("add_seq", (lead,), prompt_len, pk[gi], pv[gi]))
        for b in range(1, beam_width):
            wl.ops.append(DecodeStep("fork", (lead, lead + b)))
    for t in range(max_tail):
        seqs = tuple(s for s in range(S) if tails[s] > t)
        if not seqs:
            continue
        k = _normal(r_val, (len(seqs), Hkv, d), 1.0, "f16")
        v = _normal(r_val, (len(seqs), Hkv, d), 1.0, "f16")
        wl.ops.append(DecodeStep("append", seqs, k=k, v=v))
    allseq = tuple(range(S))
    k = _normal(r_val, (S, Hkv, d), 1.0, "f16")
    v = _normal(r_val, (S, Hkv, d), 1.0, "f16")
    wl.ops.append(DecodeStep("append", allseq, k=k, v=v))
    wl.ops.append(DecodeStep("decode", allseq, q=q))
    if n_steps:
        k_new = _normal(r_val, (n_steps, S, Hkv, d), 1.0, "f16")
        v_new = _normal(r_val, (n_steps, S, Hkv, d), 1.0, "f16")
        q_new = _normal(r_val, (n_steps, S, Hq, d), 1.0, "f16")
        for i in range(n_steps):
            wl.ops.append(DecodeStep("append", allseq, k=k_new[i], v=v_new[i]))
            wl.ops.append(DecodeStep("decode", allseq, q=q_new[i]))
    return wl


def long_context_gqa_bf16(seed: int = 5, block_size: int = 16, num_seqs: int = 16,
                          ctx_range: Tuple[int, int] = (16384, 32768),
                          pool_tokens: int = 640_000, n_steps: int = 0) -> Workload:
    """Long-context decode, bf16, a Mistral-7B-like shape: 32 query heads
    sharing 8 KV heads, head dim 128; context lengths uniform in
    ``ctx_range``; split-context partitions of 512 tokens. The pool keeps
    ``pool_tokens`` token slots whatever the block size (40,000 blocks of 16),
    in seeded random order. Context lengths and values do not depend on the
    block size."""
    r_ctx = _streams(seed, 3)[0]
    ctx = r_ctx.integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs).astype(np.int64)
    N = pool_tokens // block_size
    return _prompt_workload(f"long_context_gqa_bf16_B{block_size}",
                            f"{num_seqs} seqs ctx U[{ctx_range[0]},{ctx_range[1]}], 32 q heads / 8 kv heads, "
                            f"d 128, B {block_size}, bf16, {N} blocks",
                            seed, "bf16", ctx, 32, 8, 128, block_size, 1.0, N, n_steps=n_steps,
                            partition_size=512)


def llama2_13b_decode_fp8(seed: int = 3, num_seqs: int = 128, n_steps: int = 16, ctx_cap: int = 4096) -> Workload:
    """The LLaMA-2-13B-shaped decode with an FP8 (E4M3) cache: the same
    sequences, values and steps; K/V rows arrive as fp16 and are stored as
    codes with one float32 scale per (token, head); q and the output are fp16."""
    wl = llama2_13b_decode_f16(seed=seed, num_seqs=num_seqs, n_steps=n_steps, ctx_cap=ctx_cap)
    wl.name = "llama2_13b_decode_fp8"
    wl.description = wl.description.replace("fp16", "fp16 q, FP8 E4M3 KV cache")
    wl.kv_cache_dtype = "fp8"
    return wl


def llama2_13b_decode_int8(seed: int = 3, num_seqs: int = 128, n_steps: int = 16, ctx_cap: int = 4096) -> Workload:
    """The LLaMA-2-13B-shaped decode with an INT8 cache: the same sequences,
    values and steps; K/V rows arrive as fp16 and are stored as int8 codes
    with one float32 scale per (token, head); q and the output are fp16."""
    wl = llama2_13b_decode_f16(seed=seed, num_seqs=num_seqs, n_steps=n_steps, ctx_cap=ctx_cap)
    wl.name = "llama2_13b_decode_int8"
    wl.description = wl.description.replace("fp16", "fp16 q, INT8 KV cache")
    wl.kv_cache_dtype = "int8"
    return wl


def preempt_swap(seed: int = 6, dtype: str = "f16", kv_cache_dtype: str = "", num_seqs: int = 12,
                 ctx_range: Tuple[int, int] = (40, 900), num_kv_heads: int = 8, head_dim: int = 128,
                 block_size: int = 16, n_steps: int = 2) -> Workload:
    """Eviction to CPU memory and back, under a pool sized to run out.

    Sequences 0..S-1 with prompts U[ctx_range]; sequence S is a fork of
    sequence 0 that grows its own tail (so some blocks are shared when it is
    evicted). All decode. Then: the odd sequences and the fork are swapped
    out; two new sequences S+1, S+2 take the freed blocks; the running set
    appends and decodes ``n_steps`` times; S+1 finishes; the swapped set comes
    back; every live sequence appends and decodes ``n_steps`` times; finally
    one sequence is swapped out and freed while out. The GPU pool is sized so
    that every step fits and, at the default sizes, the two new sequences
    would not fit without the eviction (a test checks this); the swap space
    holds every evicted block, in seeded random order."""
    Hq = Hkv = num_kv_heads
    d, B = head_dim, block_size
    r_ctx, r_perm, r_val = _streams(seed, 3)
    S = num_seqs
    ctx = r_ctx.integers(ctx_range[0], ctx_range[1] + 1, size=S).astype(np.int64)
    fork_tail = 3
    out_set = tuple(s for s in range(S) if s % 2 == 1) + (S,)
    run_set = tuple(s for s in range(S) if s % 2 == 0)
    # Plain block counting for the pool size. in_use: blocks held just before
    # the eviction (the fork shares sequence 0's full prompt blocks and owns
    # the rest); reserve: what must stay free then so that the two new
    # sequences, the growth after them and the return of the evicted set
    # (the fork coming back with a whole table of its own) all fit, while the
    # new sequences alone would not fit without the eviction.
    g1, g2 = _cdiv(n_steps, B), _cdiv(n_steps + 1, B)
    fork_own = _cdiv(int(ctx[0]) + fork_tail + n_steps, B) - int(ctx[0]) // B
    in_use = sum(_cdiv(int(c) + n_steps, B) for c in ctx) + fork_own
    out_lower = sum(_cdiv(int(ctx[s]), B) for s in out_set if s < S)
    new_each = max(1, 3 * out_lower // 8)
    new_len = new_each * B - B // 2
    reserve = new_each + 1 + int(ctx[0]) // B + len(run_set) * g1 + (S + 2) * g2 + 2
    N = in_use + reserve
    num_swap = sum(_cdiv(int(ctx[s]) + n_steps, B) for s in out_set if s < S) + \
        _cdiv(int(ctx[0]) + fork_tail + n_steps, B) + 8
    wl = Workload("preempt_swap", f"{S} seqs ctx U{list(ctx_range)} + fork, swap out/in, Hkv {Hkv} d {d} B {B} "
                  f"{dtype}{f' {kv_cache_dtype} cache' if kv_cache_dtype else ''}", dtype, Hq, Hkv, d, B, N,
                  1.0 / math.sqrt(d), 0, r_perm.permutation(N).astype(np.int32), kv_cache_dtype=kv_cache_dtype,
                  num_swap_blocks=num_swap, swap_free_order=r_perm.permutation(num_swap).astype(np.int32))
    def kv(n):
        return _normal(r_val, (n, Hkv, d), 1.0, dtype), _normal(r_val, (n, Hkv, d), 1.0, dtype)
    def q(seqs):
        return _normal(r_val, (len(seqs), Hq, d), 1.0, dtype)
    def steps(seqs, n):
        for _ in range(n):
            k, v = kv(len(seqs))
            wl.ops.append(DecodeStep("append", seqs, k=k, v=v))
            wl.ops.append(DecodeStep("decode", seqs, q=q(seqs)))
    for s in range(S):
        k, v = kv(int(ctx[s]))
        wl.ops.append(DecodeStep("add_seq", (s,), int(ctx[s]), k, v))
    wl.ops.append(DecodeStep("fork", (0, S)))
    for _ in range(fork_tail):
        k, v = kv(1)
        wl.ops.append(DecodeStep("append", (S,), k=k, v=v))
    everyone = tuple(range(S + 1))
    steps(everyone, n_steps)
    wl.ops.append(DecodeStep("swap_out", out_set))
    for s in (S + 1, S + 2):
        k, v = kv(new_len)
        wl.ops.append(DecodeStep("add_seq", (s,), new_len, k, v))
    steps(run_set + (S + 1, S + 2), n_steps)
    wl.ops.append(DecodeStep("free", (S + 1,)))
    wl.ops.append(DecodeStep("swap_in", out_set))
    live_set = tuple(range(S + 1)) + (S + 2,)
    steps(live_set, n_steps)
    wl.ops.append(DecodeStep("swap_out", (1,)))
    wl.ops.append(DecodeStep("free", (1,)))
    rest = tuple(s for s in live_set if s != 1)
    steps(rest, 1)
    return wl


def prefix_cache_requests(seed: int = 10, dtype: str = "f16", kv_cache_dtype: str = "", num_kv_heads: int = 8,
                          head_dim: int = 128, block_size: int = 16, system_len: int = 300,
                          suffix_range: Tuple[int, int] = (1, 120), n_steps: int = 2, num_blocks: int = 140,
                          filler_len: int = 1000, vocab: int = 32000, swap: bool = False) -> Workload:
    """Requests that share a system prompt, served with prefix caching.

    Wave 1: requests 0..5 are the system prompt plus a suffix of
    U[suffix_range] tokens; requests 4 and 5 run under adapter 1 (same
    tokens, other K/V). All decode for ``n_steps`` rounds; 0, 1, 2 finish.
    Wave 2: request 6 continues request 1's conversation (its whole prompt
    plus a new turn); 7 and 8 are the system prompt plus a suffix; 9 is a
    plain sequence of ``filler_len`` tokens (no token ids), which pushes
    finished blocks out of the free queue. All live requests decode for
    ``n_steps`` rounds; 3, 6 and 9 finish. Wave 3: 10 and 11 are the system
    prompt plus a suffix, 12 repeats request 6's prompt and 13 repeats
    request 0's (whose own blocks the filler has evicted). All live requests
    decode for ``n_steps`` rounds.

    K/V rows depend on the token prefix as a model's would: the system
    prompt's rows are drawn once per adapter, a continuation reuses the rows
    of the conversation it extends, and a repeated prompt repeats its rows.
    A CPU test checks that the default pool fits every step, that the
    filler evicts indexed blocks and that request 13 then finds only part of
    its prompt cached.

    With ``swap``, requests 3 and 5 are evicted to a swap space after wave 1
    (their indexed blocks stay indexed in the free queue, where wave 2's
    admissions can claim them) and brought back just before wave 2 decodes."""
    Hq = Hkv = num_kv_heads
    d, B = head_dim, block_size
    r_ctx, r_perm, r_val = _streams(seed, 3)
    wl = Workload("prefix_cache_requests", f"system prompt {system_len} tok, suffixes U{list(suffix_range)}, "
                  f"continuation, repeat, adapter 1, filler {filler_len}; Hkv {Hkv} d {d} B {B} {dtype}"
                  f"{f' {kv_cache_dtype} cache' if kv_cache_dtype else ''}, {num_blocks} blocks", dtype, Hq, Hkv, d, B, num_blocks,
                  1.0 / math.sqrt(d), 0, r_perm.permutation(num_blocks).astype(np.int32),
                  kv_cache_dtype=kv_cache_dtype, prefix_caching=True)
    system = r_ctx.integers(0, vocab, size=system_len).astype(np.int32)
    sys_kv = {a: (_normal(r_val, (system_len, Hkv, d), 1.0, dtype), _normal(r_val, (system_len, Hkv, d), 1.0, dtype))
              for a in (0, 1)}
    prompts = {}

    def kv(n):
        return _normal(r_val, (n, Hkv, d), 1.0, dtype), _normal(r_val, (n, Hkv, d), 1.0, dtype)

    def add(s, tokens, k, v, extra=0):
        prompts[s] = (tokens, k, v, extra)
        wl.ops.append(DecodeStep("add_seq", (s,), len(tokens), k, v, tokens=tokens, extra_key=extra))

    def with_suffix(s, extra=0):
        n = int(r_ctx.integers(suffix_range[0], suffix_range[1] + 1))
        sk, sv = kv(n)
        k0, v0 = sys_kv[extra]
        add(s, np.concatenate([system, r_ctx.integers(0, vocab, size=n).astype(np.int32)]),
            torch.cat([k0, sk]), torch.cat([v0, sv]), extra)

    def rounds(seqs):
        wl.ops.append(DecodeStep("decode", seqs, q=_normal(r_val, (len(seqs), Hq, d), 1.0, dtype)))
        for _ in range(n_steps):
            k, v = kv(len(seqs))
            wl.ops.append(DecodeStep("append", seqs, k=k, v=v))
            wl.ops.append(DecodeStep("decode", seqs, q=_normal(r_val, (len(seqs), Hq, d), 1.0, dtype)))

    for s in range(6):
        with_suffix(s, extra=1 if s >= 4 else 0)
    rounds(tuple(range(6)))
    if swap:
        wl.num_swap_blocks = 64
        wl.swap_free_order = r_perm.permutation(64).astype(np.int32)
        wl.ops.append(DecodeStep("swap_out", (3, 5)))
    wl.ops.append(DecodeStep("free", (0, 1, 2)))
    t1, k1, v1, _ = prompts[1]
    n = int(r_ctx.integers(suffix_range[0], suffix_range[1] + 1))
    nk, nv = kv(n)
    add(6, np.concatenate([t1, r_ctx.integers(0, vocab, size=n).astype(np.int32)]), torch.cat([k1, nk]),
        torch.cat([v1, nv]))
    with_suffix(7)
    with_suffix(8)
    fk, fv = kv(filler_len)
    wl.ops.append(DecodeStep("add_seq", (9,), filler_len, fk, fv))
    if swap:
        wl.ops.append(DecodeStep("swap_in", (3, 5)))
    rounds((3, 4, 5, 6, 7, 8, 9))
    wl.ops.append(DecodeStep("free", (3, 6, 9)))
    with_suffix(10)
    with_suffix(11)
    t6, k6, v6, _ = prompts[6]
    add(12, t6.copy(), k6.clone(), v6.clone())
    t0, k0, v0, _ = prompts[0]
    add(13, t0.copy(), k0.clone(), v0.clone())
    rounds((4, 5, 7, 8, 10, 11, 12, 13))
    return wl


def custom_decode(seed: int, dtype: str, ctx: Sequence[int], num_q_heads: int, num_kv_heads: int,
                  head_dim: int, block_size: int, num_blocks: Optional[int] = None, factor: float = 1.0,
                  n_steps: int = 0, kv_cache_dtype: str = "") -> Workload:
    """Independent sequences with the given prompt lengths (a small test shape
    of any supported geometry); pool = blocks needed + 3, shuffled."""
    need = sum(_cdiv(int(c) + n_steps, block_size) for c in ctx)
    N = need + 3 if num_blocks is None else num_blocks
    wl = _prompt_workload("custom", f"ctx {list(ctx)} Hq {num_q_heads} Hkv {num_kv_heads} d {head_dim} "
                          f"B {block_size} {dtype}{f' {kv_cache_dtype} cache' if kv_cache_dtype else ''}", seed, dtype,
                          [int(c) for c in ctx], num_q_heads, num_kv_heads, head_dim, block_size, factor, N,
                          n_steps=n_steps)
    wl.kv_cache_dtype = kv_cache_dtype
    return wl


ALL_CONFIGS: Sequence[Callable[..., Workload]] = (
    tiny_paged_decode_f32,
    llama7b_decode_f16,
    llama2_13b_decode_f16,
    shared_prefix_beam_f16,
    long_context_gqa_bf16,
)


def make_config(n: int, **kw) -> Workload:
    """Workload number ``n`` (1..5) at its full size."""
    return ALL_CONFIGS[n - 1](**kw)


def scaled_down(n: int) -> Workload:
    """A small variant of workload ``n`` that the oracle finishes in seconds
    while still spanning several blocks, several partitions and ragged tails."""
    if n == 1:
        return tiny_paged_decode_f32()
    if n == 2:
        return llama7b_decode_f16(seed=12, num_seqs=6, ctx_range=(1, 1200))
    if n == 3:
        return llama2_13b_decode_f16(seed=13, num_seqs=8, n_steps=3, ctx_cap=1500)
    if n == 4:
        return shared_prefix_beam_f16(seed=14, num_groups=2, beam_width=4, prompt_len=600, max_tail=20)
    if n == 5:
        return long_context_gqa_bf16(seed=15, block_size=16, num_seqs=3, ctx_range=(900, 2100),
                                     pool_tokens=16384)
    raise ValueError(n)
