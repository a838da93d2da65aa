"""Seeded synthetic inputs for paged decode attention.

This package only draws numbers: context lengths, the initial order of the
free block list, query vectors and per-token K/V values, plus the list of
host operations a workload replays (add a sequence, fork, append a step,
decode). It holds none of the method's arithmetic: it never addresses a
cache, builds a block table, computes a slot, a softmax or a copy. Both the
CPU oracle and the GPU path read the same objects from here and each runs
the method with its own code.

Shapes follow the pages' workloads: LLaMA-7B (32 heads, head dim 128),
LLaMA-2-13B (40 heads, head dim 128), beam search over a shared prompt, and
a Mistral-7B-like grouped-query shape (32 query heads over 8 KV heads).
"""

from .configs import (  # noqa: F401
    Workload,
    DecodeStep,
    ALL_CONFIGS,
    make_config,
    tiny_paged_decode_f32,
    llama7b_decode_f16,
    llama2_13b_decode_f16,
    llama2_13b_decode_fp8,
    llama2_13b_decode_int8,
    shared_prefix_beam_f16,
    long_context_gqa_bf16,
    scaled_down,
    custom_decode,
    preempt_swap,
    prefix_cache_requests,
)
