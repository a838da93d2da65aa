"""Decode-step benchmark of the paged KV-cache library on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one pass of the whole decode hot path over the batch: the host
allocator hands out one slot per sequence (new blocks on 16-token
boundaries, copy-on-write pairs for shared blocks), the slots / pairs /
block tables / context lengths are staged to the GPU, copy_blocks runs the
copies, kv_append writes the 128 new K/V rows, and pa_decode attends over
every sequence's whole context. Inputs (K/V rows and queries of every step)
are resident in HBM before the timed region.

Prints one JSON line (stdout). ``value`` is the K/V bytes the decode
attention reads per step (2 * kv_heads * head_dim * elem bytes per context
token) divided by the wall time of the whole step; ``roofline`` gives the
partition kernel's own rate from HIP events recorded around it on its stream;
``cpu_baseline`` times the CPU oracle on a bounded sample of the same state.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn KV GB/s (% of HBM peak) + context tokens/s, 13B-shape fp16"
HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published
COUNTERS_FILE = os.path.join(ROOT, "profiles", "pa_decode_partition_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_cache_411_amd", "csrc", "pa_decode.hip")
PROBE_LIB = os.path.join(ROOT, "paged_kv_cache_411_amd", "libpagedkv_probe.so")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_workload(name: str, n_steps: int):
    import workloads
    if name == "tiny":
        return workloads.tiny_paged_decode_f32(n_steps=n_steps)
    if name == "llama2_13b":
        return workloads.llama2_13b_decode_f16(n_steps=n_steps)
    if name == "llama2_13b_fp8":
        return workloads.llama2_13b_decode_fp8(n_steps=n_steps)
    if name == "llama2_13b_int8":
        return workloads.llama2_13b_decode_int8(n_steps=n_steps)
    if name == "llama7b":
        return workloads.llama7b_decode_f16(n_steps=n_steps)
    if name == "shared_prefix":
        return workloads.shared_prefix_beam_f16(n_steps=n_steps)
    if name.startswith("long_ctx_B"):
        return workloads.long_context_gqa_bf16(block_size=int(name[len("long_ctx_B"):]), n_steps=n_steps)
    raise SystemExit(f"unknown workload {name}")


def kernel_code_hash() -> str:
    """sha256 of the partition kernel's source with its // comments, trailing
    blanks and empty lines taken out: stored counters stay valid across
    comment edits and lapse with any change to the code."""
    lines = []
    for line in open(KERNEL_SOURCE, encoding="utf-8"):
        code = line.split("//", 1)[0].rstrip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def stored_traffic_ratio(workload: str):
    """Calibrated HBM bytes (fetch + write) of the partition kernel per
    algorithmic byte, from the committed rocprofv3 counter runs of this
    workload on this kernel source; None when absent or taken on another
    source. Multiplied by a launch's algorithmic bytes it gives that launch's
    traffic, for any step count."""
    try:
        c = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    w = c.get("workloads", {}).get(workload)
    if not w or w.get("kernel_code_sha256") != kernel_code_hash():
        return None
    return w.get("hbm_bytes_per_algorithmic_byte")


def calib_gather(mib: int, dev) -> None:
    """The gather probe (libpagedkv_probe.so) over exactly ``mib`` MiB: 4 KiB
    chunks of a buffer twice that size, in a seeded random order, 64 chunks
    per workgroup, with the decode's non-temporal loads - a dispatch of known
    bytes for scaling the byte counters."""
    import ctypes

    import numpy as np
    import torch
    lib = ctypes.CDLL(PROBE_LIB)
    lib.pa_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.pa_probe_gather.restype = ctypes.c_int
    lib.pa_probe_gather_sink_words.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.pa_probe_gather_sink_words.restype = ctypes.c_int64
    n = mib * 256                                        # 4 KiB chunks read
    buf = torch.empty(2 * n * 4096, dtype=torch.uint8, device=dev).fill_(1)
    order = torch.from_numpy(np.random.default_rng(11).permutation(2 * n)[:n].astype(np.int32)).to(dev)
    per_item = 64
    sink = torch.empty(int(lib.pa_probe_gather_sink_words(n, per_item)), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    rc = lib.pa_probe_gather(buf.data_ptr(), 2 * n, order.data_ptr(), n, per_item, sink.data_ptr(),
                             torch.cuda.current_stream(dev).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"pa_probe_gather failed ({rc})")
    torch.cuda.synchronize()
    log(f"[bench] calibration gather probe: {n} chunks of 4 KiB = {n * 4096} bytes read, order {4 * n} bytes")


def cpu_baseline(wl, setup_ops, budget_s: float):
    """The CPU oracle, as it stands, on a bounded sample: decodes of the setup
    state's sequences (all heads), cycling over the batch until ``budget_s``
    seconds have passed and the batch has been covered at least once."""
    import numpy as np
    from oracle.runner import OracleReplay
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:   # threadpoolctl missing: report the affinity count
        threads = len(os.sched_getaffinity(0))
    rep = OracleReplay(wl)
    for op in setup_ops:
        if op.kind != "decode":
            rep.apply(op)
    dec = next(op for op in setup_ops if op.kind == "decode")
    S = len(dec.seq_ids)
    done_ctx = 0
    n = 0
    t0 = time.perf_counter()
    # whole-batch passes, one sequence (all heads) at a time, until the budget is spent
    while True:
        i = n % S
        rep.decode((dec.seq_ids[i],), dec.q[i:i + 1])
        done_ctx += rep.alloc.context_lens[dec.seq_ids[i]]
        n += 1
        if time.perf_counter() - t0 >= budget_s and n >= S:
            break
    el = time.perf_counter() - t0
    bpt = wl.kv_bytes_per_token
    return {"value": round(done_ctx * bpt / el / 1e9, 4), "unit": "GB/s",
            "context_tokens_per_s": round(done_ctx / el, 1), "cores": threads, "kind": "oracle",
            "sample": f"{n} single-sequence fp64 decodes ({n / S:.2f} passes over the {S}-sequence batch of the "
                      f"setup state, all {wl.num_q_heads} heads, {done_ctx} context tokens) in {el:.1f} s",
            "host_cpu_count": os.cpu_count(), "host_affinity": len(os.sched_getaffinity(0))}


PCIE_PEAK_GBPS = 64.0    # MI355X host link, PCIe 5.0 x16, published per direction


def _threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:   # threadpoolctl missing: report the affinity count
        return len(os.sched_getaffinity(0))


def cpu_baseline_swap(H: int, B: int, d: int, budget_s: float) -> dict:
    """The oracle's swap (allocator model + whole-block bit copies between a
    GPU-pool array and a swap-space array, numpy on the host) on a bounded
    sample: round trips of 16 sequences of 1024 tokens of the same shape,
    repeated until ``budget_s`` has passed."""
    import numpy as np
    from oracle import alloc_model, cache_ops
    S, T = 16, 1024
    blocks = S * T // B
    m = alloc_model.BlockAllocatorModel(blocks + blocks // 4, B)
    m.set_swap_space(blocks + 64)
    gk = np.zeros((m.num_blocks, H, B, d), np.uint16)
    gv = np.zeros_like(gk)
    hk = np.zeros((blocks + 64, H, B, d), np.uint16)
    hv = np.zeros_like(hk)
    for s in range(S):
        m.add_seq(s, T)
    moved, n = 0, 0
    t0 = time.perf_counter()
    while True:
        for s in range(S):
            cache_ops.swap_blocks(gk, gv, hk, hv, m.swap_out(s))
        for s in range(S):
            cache_ops.swap_blocks(hk, hv, gk, gv, m.swap_in(s))
        moved += 2 * blocks * 2 * H * B * d * 2
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(moved / el / 1e9, 3), "unit": "GB/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{n} swap round trips of {blocks} blocks (oracle allocator model + numpy block copies) "
                      f"in {el:.1f} s"}


def cpu_baseline_prefix(system, suffixes, lens, H: int, B: int, d: int, budget_s: float) -> dict:
    """The oracle's prefix-cached admission (allocator model with exact
    content keys + numpy row writes of the uncached rows) on a bounded sample
    of the same request stream, one step of 32 prompts at a time until
    ``budget_s`` has passed."""
    import numpy as np
    from oracle import alloc_model, cache_ops
    R = len(lens)
    N = int(2 * np.ceil(lens / B).sum())
    m = alloc_model.BlockAllocatorModel(N, B, np.random.default_rng(7).permutation(N))
    m.enable_prefix_caching()
    kc = np.zeros((N, H, B, d), np.uint16)
    vc = np.zeros_like(kc)
    rows = np.zeros((int(lens.max()), H, d), np.uint16)
    tokens, n = 0, 0
    t0 = time.perf_counter()
    while True:
        i = n % len(suffixes)
        for r in range(R):
            sid = n * R + r
            c = m.add_seq_cached(sid, np.concatenate([system, suffixes[i][r]]))
            slots = m.seq_slots(sid, c, int(lens[r]) - c)
            cache_ops.kv_append(kc, vc, rows[c:int(lens[r])], rows[c:int(lens[r])], slots)
        for r in range(R):
            m.free_seq(n * R + r)
        tokens += int(lens.sum())
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(tokens / el, 1), "unit": "tokens/s", "cores": _threads(), "kind": "oracle",
            "sample": f"{n} admission steps of {R} prompts ({tokens} prompt tokens; oracle allocator model with "
                      f"prefix caching + numpy row writes) in {el:.1f} s"}


def bench_swap(args) -> dict:
    """Eviction round trips on the LLaMA-2-13B cache shape (40 KV heads, head
    dim 128, blocks of 16, fp16): 16 sequences of 1024 tokens (1024 blocks,
    320 MiB of K+V) are swapped out to pinned host memory and back in, a step
    being one swap_out of all of them followed by one swap_in. Timed over the
    whole runtime call (allocator, pair upload, swap_blocks); the swap_blocks
    launches are also bracketed by HIP events on their stream. A plain
    contiguous copy of the same byte count through torch (the DMA engines)
    is measured for reference."""
    import numpy as np
    import torch

    import paged_kv_cache_411_amd as pk
    from paged_kv_cache_411_amd.runtime import PagedKVCache

    pk.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H, d, B, S, T = 40, 128, 16, 16, 1024
    blocks = S * T // B
    N = blocks + blocks // 4
    cache = PagedKVCache(N, H, B, d, torch.float16, dev, np.random.default_rng(7).permutation(N),
                         num_swap_blocks=blocks + 64)
    g = torch.Generator(device=dev).manual_seed(1)
    for t in (cache.k_cache, cache.v_cache):
        t.view(torch.int16).copy_(torch.randint(-2**15, 2**15, t.shape, generator=g, device=dev,
                                                dtype=torch.int32).to(torch.int16))
    for s in range(S):
        cache.alloc.add_seq(s, T)
    seqs = list(range(S))
    block_bytes = 2 * H * B * d * 2
    moved = blocks * block_bytes          # bytes per direction per step
    K, W = args.steps, args.warmup
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(W + K)]
    log(f"[bench] swap round trips of {blocks} blocks ({moved / 2**20:.0f} MiB each way), warmup {W}")

    def step(i):
        e = evs[i]
        e[0].record()
        cache.swap_out(seqs)
        e[1].record()
        cache.swap_in(seqs)
        e[2].record()

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] timing {K} swap round trips")
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    out_ms = float(np.mean([evs[i][0].elapsed_time(evs[i][1]) for i in range(W, W + K)]))
    in_ms = float(np.mean([evs[i][1].elapsed_time(evs[i][2]) for i in range(W, W + K)]))
    # reference: one contiguous copy each way through the DMA engines
    host = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
    devb = torch.empty(moved, dtype=torch.uint8, device=dev)
    a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    for _ in range(2):
        a.record()
        host.copy_(devb, non_blocking=True)
        b.record()
        devb.copy_(host, non_blocking=True)
        c.record()
        torch.cuda.synchronize()
    dma_d2h, dma_h2d = moved / a.elapsed_time(b) / 1e6, moved / b.elapsed_time(c) / 1e6
    step_s = wall / K
    value = 2 * moved / step_s / 1e9
    out_gbps, in_gbps = moved / out_ms / 1e6, moved / in_ms / 1e6
    log(f"[bench] swap step {step_s * 1e3:.2f} ms: out {out_ms:.2f} ms ({out_gbps:.1f} GB/s), in {in_ms:.2f} ms "
        f"({in_gbps:.1f} GB/s); DMA copy d2h {dma_d2h:.1f} GB/s, h2d {dma_h2d:.1f} GB/s")
    return {
        "metric": "KV swap GB/s (device <-> pinned host, out + in), 13B-shape fp16 blocks",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(step_s * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "swap_13b", "description": f"{S} seqs x {T} tokens, 40 KV heads, d 128, B 16, "
                   f"fp16; swap_out of all then swap_in of all per step", "blocks_per_direction": blocks,
                   "block_bytes": block_bytes, "swap_space": "pinned host memory (hipHostMalloc via torch)"},
        "swap_out_ms": round(out_ms, 3), "swap_in_ms": round(in_ms, 3),
        "dma_copy_gbps": {"d2h": round(dma_d2h, 1), "h2d": round(dma_h2d, 1)},
        "roofline": {"bound": "pcie", "kernel": "copy_blocks_kernel (swap_blocks)",
                     "achieved": round(min(out_gbps, in_gbps), 1), "peak": PCIE_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(min(out_gbps, in_gbps) / PCIE_PEAK_GBPS, 4), "traffic": None,
                     "achieved_out": round(out_gbps, 1), "achieved_in": round(in_gbps, 1),
                     "algorithmic_bytes_per_launch": moved,
                     "algorithmic_bytes": "K+V bytes of the moved blocks, one direction"},
        **({} if args.no_cpu_baseline else {"cpu_baseline": cpu_baseline_swap(H, B, d, args.cpu_budget)}),
    }


def bench_prefix(args) -> dict:
    """Prompt admission with prefix caching on the LLaMA-2-13B cache shape
    (40 KV heads, head dim 128, blocks of 16, fp16). A step admits 32
    requests - a shared 1024-token system prompt plus a suffix of U[1, 256]
    fresh random tokens each - with PagedKVCache.add_sequences (the host
    allocator's prefix lookup per request, one pair upload, one kv_append
    launch that skips the cached rows), then frees them, so their blocks go
    back to the free queue still indexed. The same steps run with caching
    off for comparison. ``value`` is prompt tokens admitted per second with
    caching on. The K/V rows of every request (a batched prefill's output)
    are resident in HBM before timing."""
    import numpy as np
    import torch

    import paged_kv_cache_411_amd as pk
    from paged_kv_cache_411_amd.runtime import PagedKVCache

    pk.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H, d, B, R, P = 40, 128, 16, 32, 1024
    rng = np.random.default_rng(21)
    lens = P + rng.integers(1, 257, size=R)
    total = int(lens.sum())
    system = rng.integers(0, 32000, size=P).astype(np.int32)
    K, W = args.steps, args.warmup
    suffixes = [[rng.integers(0, 32000, size=int(n) - P).astype(np.int32) for n in lens] for _ in range(W + K)]
    g = torch.Generator(device=dev).manual_seed(3)
    k = torch.randn((total, H, d), generator=g, device=dev).half()
    v = torch.randn((total, H, d), generator=g, device=dev).half()
    off = np.concatenate([[0], np.cumsum(lens)[:-1]])
    for r in range(1, R):        # the system prompt's rows are the same in every request
        k[off[r]:off[r] + P] = k[:P]
        v[off[r]:off[r] + P] = v[:P]
    N = int(2 * np.ceil(lens / B).sum())
    row_bytes = 2 * H * d * 2          # K + V of one token

    def run(caching: bool):
        cache = PagedKVCache(N, H, B, d, torch.float16, dev, np.random.default_rng(7).permutation(N),
                             prefix_caching=caching)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(W + K)]
        host_s, written, cached_tok = [], 0, 0

        def step(i):
            nonlocal written, cached_tok
            ids = list(range(i * R, (i + 1) * R))
            toks = [np.concatenate([system, suffixes[i][r]]) for r in range(R)] if caching else None
            t0 = time.perf_counter()
            c = cache.add_sequences(ids, k, v, lens, tokens=toks, prof_events=evs[i])
            t1 = time.perf_counter()
            for s in ids:
                cache.free(s)
            if i >= W:
                host_s.append(t1 - t0)
                cached_tok += sum(c)
                written += total - sum(c)

        for i in range(W):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(W, W + K):
            step(i)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / K
        app_ms = float(np.mean([evs[i][0].elapsed_time(evs[i][1]) for i in range(W, W + K)]))
        app_bytes = 2 * row_bytes * written / K        # rows read from k/v and written to the cache
        return {"ms_per_step": wall * 1e3, "prompt_tokens_per_s": total / wall,
                "cached_fraction": cached_tok / (total * K), "rows_written_per_step": written / K,
                "append_us": app_ms * 1e3, "append_gbps": app_bytes / (app_ms / 1e3) / 1e9 if app_ms else 0.0,
                "append_bytes": app_bytes, "host_us_per_request": float(np.mean(host_s)) / R * 1e6}

    log(f"[bench] prefix caching: {R} requests of {P} shared + U[1,256] tokens per step, warmup {W}, {K} timed")
    on = run(True)
    off_ = run(False)
    # reference: a plain device-to-device copy of the uncached run's bytes (read once, written once)
    src = torch.empty(int(off_["append_bytes"]) // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(3):
        a_.record()
        dst.copy_(src)
        b_.record()
        torch.cuda.synchronize()
        best = min(best, a_.elapsed_time(b_))
    copy_gbps = 2 * src.numel() / (best / 1e3) / 1e9
    del src, dst
    log(f"[bench] cached: {on['ms_per_step']:.3f} ms/step, {on['prompt_tokens_per_s'] / 1e6:.2f} M prompt tok/s, "
        f"{100 * on['cached_fraction']:.1f}% cached, append {on['append_us']:.1f} us ({on['append_gbps']:.0f} GB/s), "
        f"host {on['host_us_per_request']:.1f} us/request")
    log(f"[bench] uncached: {off_['ms_per_step']:.3f} ms/step, {off_['prompt_tokens_per_s'] / 1e6:.2f} M prompt "
        f"tok/s, append {off_['append_us']:.1f} us ({off_['append_gbps']:.0f} GB/s), host "
        f"{off_['host_us_per_request']:.1f} us/request; plain device copy of the same bytes {copy_gbps:.0f} GB/s")
    rnd = lambda dct: {a: round(b, 4) for a, b in dct.items()}
    return {
        "metric": "prompt tokens admitted/s with prefix caching, 13B-shape fp16 cache",
        "value": round(on["prompt_tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(on["ms_per_step"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "prefix_13b", "description": f"{R} requests/step: {P}-token shared system prompt + "
                   f"U[1,256] fresh tokens; 40 KV heads, d 128, B 16, fp16; admitted then freed each step",
                   "prompt_tokens_per_step": total, "num_blocks": N},
        "cached": rnd(on), "uncached": rnd(off_),
        "speedup_vs_uncached": round(on["prompt_tokens_per_s"] / off_["prompt_tokens_per_s"], 3),
        "d2d_copy_gbps": round(copy_gbps, 1),
        "roofline": {"bound": "hbm", "kernel": "kv_append_kernel (cached run)",
                     "achieved": round(on["append_gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(on["append_gbps"] / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": int(on["append_bytes"]),
                     "algorithmic_bytes": "uncached prompt rows: K+V read from the batch and written to the cache"},
        **({} if args.no_cpu_baseline else
           {"cpu_baseline": cpu_baseline_prefix(system, suffixes, lens, H, B, d, args.cpu_budget)}),
    }


def fixed_state_decode(cache, seqs, q, wl, part: int, schedule: bool, reps: int = 100, warm: int = 10) -> dict:
    """pa_decode alone (partition + merge) repeated on the final cache state
    of the step loop: one schedule, tables and lengths uploaded once, HIP
    events around every launch on the launching stream, median and minimum.
    GB/s counts the K/V bytes of the state (shared blocks once when the
    launch reads them once)."""
    import numpy as np
    import torch

    import paged_kv_cache_411_amd as pk

    dev = q.device
    tables, ctx = cache.tables(seqs)
    max_ctx = max(1, int(ctx.max()))
    d_tables = torch.from_numpy(np.ascontiguousarray(tables)).to(dev)
    d_ctx = torch.from_numpy(np.ascontiguousarray(ctx)).to(dev)
    kw = {}
    if schedule:
        share = pk.pa_decode_share_width() if (cache.share and q.shape[1] == wl.num_kv_heads) else 1
        sch = pk.pa_decode_schedule(ctx, wl.block_size, part, max_ctx, np.ascontiguousarray(tables), share)
        kw = dict(work=torch.from_numpy(np.ascontiguousarray(sch.work)).to(dev),
                  members=torch.from_numpy(np.ascontiguousarray(sch.members)).to(dev) if len(sch.members) else None,
                  num_slots=torch.from_numpy(np.ascontiguousarray(sch.num_slots)).to(dev), max_slots=sch.max_slots)
    if cache.fp8:
        kw.update(k_scale=cache.k_scale, v_scale=cache.v_scale)
    need = pk.pa_decode_workspace_bytes(q, cache.k_cache, d_tables, max_ctx, part, schedule)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    from paged_kv_cache_411_amd import _hip
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev = [(_hip.Event(), _hip.Event()) for _ in range(reps)]
    for i in range(warm + reps):
        if i >= warm:
            ev[i - warm][0].record(stream)
        pk.pa_decode(q, cache.k_cache, cache.v_cache, d_tables, d_ctx, wl.scale, out, max_context_len=max_ctx,
                     partition_size=part, workspace=ws if need else None, **kw)
        if i >= warm:
            ev[i - warm][1].record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_ms(b) * 1e3 for a, b in ev)
    B = wl.block_size
    fill = {}
    for row, c in zip(tables, ctx):
        for j in range(-(-int(c) // B)):
            fill[int(row[j])] = max(fill.get(int(row[j]), 0), min(B, int(c) - j * B))
    logical = float(ctx.sum()) * wl.kv_bytes_per_token
    shared_once = schedule and cache.share and sum(fill.values()) < 0.999 * float(ctx.sum())
    alg = sum(fill.values()) * wl.kv_bytes_per_token if shared_once else logical
    med = us[len(us) // 2]
    return {"launches": reps, "warmup": warm, "median_us": round(med, 2), "min_us": round(us[0], 2),
            "gbps_at_median": round(alg / med / 1e3, 1), "gbps_at_min": round(alg / us[0] / 1e3, 1),
            "bytes": int(alg), "bytes_counted": "unique K+V bytes (shared blocks once)" if shared_once else "K+V bytes",
            "sum_context_tokens": int(ctx.sum()),
            "timing": "HIP events around each pa_decode call (partition + merge) on the launching stream"}


def unique_tokens_per_step(wl, setup_ops, seqs, W: int, K: int):
    """Distinct context tokens each of the K timed steps reads (a block that
    several sequences hold counted once, with its most-filled holder's rows):
    a host allocator is driven through the workload's setup and its W + K
    append steps exactly as the cache's was, and its tables are read after
    each timed step."""
    import numpy as np

    import paged_kv_cache_411_amd as pk
    a = pk.BlockAllocator(wl.num_blocks, wl.block_size, wl.free_order)
    for op in setup_ops:
        if op.kind == "add_seq":
            a.add_seq(op.seq_ids[0], op.num_tokens)
        elif op.kind == "fork":
            a.fork(*op.seq_ids)
        elif op.kind == "append":
            a.append_slots(np.asarray(op.seq_ids, dtype=np.int64))
    B = wl.block_size
    out = []
    for i in range(W + K):
        a.append_slots(seqs)
        if i < W:
            continue
        tables, ctx = a.block_tables(seqs, max(1, a.table_width(seqs)))
        fill = {}
        for row, c in zip(tables, ctx):
            for j in range(-(-int(c) // B)):
                b = int(row[j])
                fill[b] = max(fill.get(b, 0), min(B, int(c) - j * B))
        out.append(sum(fill.values()))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama2_13b")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="split-context partition in tokens (default: the workload's; 0 = the library's)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-schedule", action="store_true",
                    help="launch every (sequence, partition) instead of the longest-first schedule")
    ap.add_argument("--no-share", action="store_true",
                    help="do not read shared-prompt partitions once per group")
    ap.add_argument("--prof-every", type=int, default=0,
                    help="bracket the partition kernel with HIP events on every N-th timed step after the "
                         "first (0: every step when --steps < 16, else every max(2, steps // 16)-th)")
    ap.add_argument("--fixed-reps", type=int, default=100,
                    help="timed pa_decode launches on the final state after the step loop")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain elementwise copy kernel over this many MiB (counter calibration runs)")
    ap.add_argument("--calib-gather-mib", type=int, default=0,
                    help="also run the gather probe over exactly this many MiB (counter calibration runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): the decode path has no "
              f"multi-GPU mode in this library", file=sys.stderr)
        sys.exit(2)

    if args.workload == "swap_13b":
        print(json.dumps(bench_swap(args)), flush=True)
        return
    if args.workload == "prefix_13b":
        print(json.dumps(bench_prefix(args)), flush=True)
        return

    import numpy as np
    import torch

    import paged_kv_cache_411_amd as pk
    from paged_kv_cache_411_amd.runtime import PagedKVCache

    pk.lib()   # fail loudly if the library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, W = args.steps, args.warmup
    log(f"[bench] generating workload {args.workload} with {W + K} append+decode steps")
    wl = make_workload(args.workload, W + K)
    rounds_start = len(wl.ops) - 2 * (W + K)
    setup, rounds = wl.ops[:rounds_start], wl.ops[rounds_start:]
    seqs = np.ascontiguousarray(np.asarray(rounds[0].seq_ids, dtype=np.int64))

    log("[bench] filling the cache on the GPU")
    cache = PagedKVCache(wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim, wl.torch_dtype, dev,
                         wl.free_order, schedule=not args.no_schedule, share=not args.no_share,
                         kv_cache_dtype=wl.kv_cache_dtype)
    for op in setup:
        if op.kind == "add_seq":
            cache.add_sequence(op.seq_ids[0], op.k, op.v)
        elif op.kind == "fork":
            cache.fork(*op.seq_ids)
        elif op.kind == "append":
            cache.append(op.seq_ids, op.k, op.v)
    # step inputs resident in HBM before timing
    ks = [rounds[2 * i].k.to(dev) for i in range(W + K)]
    vs = [rounds[2 * i].v.to(dev) for i in range(W + K)]
    qs = [rounds[2 * i + 1].q.to(dev) for i in range(W + K)]
    out = torch.empty_like(qs[0])
    from paged_kv_cache_411_amd import _hip
    # kernel timestamps: events without the system-scope release, so that a
    # bracketed launch costs the stream (almost) nothing extra
    ev = [(_hip.Event(), _hip.Event()) for _ in range(W + K)]
    torch.cuda.synchronize()
    bytes_per_tok = wl.kv_bytes_per_token      # K+V bytes the cache holds per token (FP8: codes + scales)

    ctx_per_step = []
    part = wl.partition_size if args.partition_size is None else args.partition_size
    part_eff = part or min(1024, 64 * wl.block_size)    # the library's default when 0

    # The partition kernel's launch is bound to a pair of HIP events (its own
    # start and end on its stream) on every PROF_EVERY-th timed step after the
    # first; those launches give its duration. The events cost the host about
    # 25 us per launch, hidden behind the GPU on every step but the first
    # (whose host time the timed region sees whole), and the stream about
    # 2 us, so at 16 steps or more only every other step (or fewer) carries them.
    prof_every = args.prof_every or (1 if K < 16 else max(2, K // 16))
    prof = set(range(W + 1, W + K, prof_every)) if K > 1 else {W}
    host_us = []

    def step(i):
        t = time.perf_counter()
        cache.step(seqs, ks[i], vs[i], qs[i], out=out, scale=wl.scale, partition_size=part,
                   prof_events=ev[i] if i in prof else None)
        host_us.append((time.perf_counter() - t) * 1e6)
        ctx_per_step.append(int(cache.last_context_lens.sum()))

    log(f"[bench] warmup {W} steps")
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    ctx_per_step.clear()
    host_us.clear()
    log(f"[bench] timing {K} steps")
    # nothing but the steps between the two synchronisations: a timing event
    # recorded there would put a marker packet of its own on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part_ms = [ev[i][0].elapsed_ms(ev[i][1]) for i in sorted(prof)]
    step_s = wall / K
    sum_ctx = float(np.mean(ctx_per_step))
    kv_bytes = sum_ctx * bytes_per_tok
    value = kv_bytes / step_s / 1e9
    part_avg_s = float(np.mean(part_ms)) / 1e3
    prof_ctx = float(np.mean([ctx_per_step[i - W] for i in sorted(prof)]))   # context of the bracketed steps
    prof_bytes = prof_ctx * bytes_per_tok
    achieved = prof_bytes / part_avg_s / 1e9
    log(f"[bench] step {step_s * 1e6:.1f} us; partition kernel "
        f"avg {part_avg_s * 1e6:.1f} us min {min(part_ms) * 1e3:.1f} us; sum ctx {sum_ctx:.0f}; "
        f"{achieved:.0f} GB/s in the kernel")

    if args.calib_gather_mib:
        calib_gather(args.calib_gather_mib, dev)
    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2**20 // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)   # an elementwise kernel: reads and writes exactly n * 4 bytes
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")

    fixed = None
    if args.fixed_reps > 0:
        fixed = fixed_state_decode(cache, seqs, qs[-1], wl, part, not args.no_schedule, args.fixed_reps)
        log(f"[bench] pa_decode on the fixed final state: median {fixed['median_us']} us, min {fixed['min_us']} us "
            f"over {fixed['launches']} launches ({fixed['gbps_at_median']} GB/s at the median)")

    # Bytes the decode must read with shared blocks counted once, step by step:
    # a twin of the host allocator replays the setup and takes the same steps
    # (outside the timed region); per step, each distinct physical block counts
    # its most-filled user's rows.
    unique_tok = unique_tokens_per_step(wl, setup, seqs, W, K)
    unique_ratio = float(np.mean(unique_tok)) / sum_ctx
    unique_bytes = float(np.mean(unique_tok)) * bytes_per_tok
    shared = unique_ratio < 0.999 and not args.no_schedule and cache.share
    alg_bytes = unique_bytes if shared else kv_bytes
    prof_unique = float(np.mean([unique_tok[i - W] for i in sorted(prof)])) * bytes_per_tok
    alg_prof = prof_unique if shared else prof_bytes        # per bracketed launch
    achieved = alg_prof / part_avg_s / 1e9
    ratio = stored_traffic_ratio(wl.name)
    traffic = None if ratio is None else int(round(ratio * alg_prof))
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype if not wl.kv_cache_dtype else f"{wl.dtype} q, {wl.kv_cache_dtype} KV",
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "num_seqs": len(seqs),
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "block_size": wl.block_size, "num_blocks": wl.num_blocks, "accumulate": "f32",
                   "kv_cache": wl.kv_cache_dtype or wl.dtype, "kv_bytes_per_token": bytes_per_tok,
                   "partition_size": part_eff, "schedule": "none" if args.no_schedule else ("longest-first" if args.no_share else "longest-first, shared"), "mean_sum_context_tokens": round(sum_ctx, 1),
                   "step": "pa_decode_step: allocator step, schedule, copy_blocks, staged upload + kv_append, pa_decode"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "context_tokens_per_s": round(sum_ctx / step_s, 1),
        "kv_bytes_per_step": int(kv_bytes),
        "unique_kv_bytes_per_step": int(unique_bytes),
        "host_us_per_step": {"first": round(host_us[0], 1), "median": round(float(np.median(host_us)), 1),
                             "note": "host time of each step call (allocator step, schedule, launches, and "
                                     "once the host is a ring of staging buffers ahead, the wait for one); only "
                                     "the first timed step's is not hidden behind earlier GPU work"},
        "pa_decode_fixed_state": fixed,
        "roofline": {"bound": "hbm", "kernel": "pa_decode_partition_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "traffic_per_algorithmic_byte": ratio,
                     "avg_launch_us": round(part_avg_s * 1e6, 2),
                     "algorithmic_bytes_per_launch": int(alg_prof), "launches_timed": len(part_ms),
                     "algorithmic_bytes": "unique K+V bytes (shared blocks once)" if shared else "K+V bytes"},
    }
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_budget:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(wl, setup, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
