"""Oracle: replay a workload's host operations (TEST INFRASTRUCTURE).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.

Each operation of a ``workloads.Workload`` is carried out with the oracle's
own allocator model, bitwise cache operations and fp64 attention:

* ``add_seq``  - allocate the prompt's blocks, then write every prompt token
                 into its slot ([PA] §3.3 steps 2-4); with prefix caching
                 ([KVM] Part 3) the prompt's indexed leading blocks are
                 reused and only the tokens past them are written;
* ``fork``     - share every block of the parent ([VM] "写时复制与块共享机制");
* ``append``   - one slot per listed sequence; the copy-on-write block copies
                 of the step run before the new tokens are written (a copy
                 must carry the old contents into the new block before the
                 writer modifies it, [PA] §4.1 steps 1-3);
* ``decode``   - gather + fp64 attention for the listed sequences;
* ``swap_out`` / ``swap_in`` - each listed sequence in order: the allocator
                 moves its table between the GPU pool and the swap space and
                 the blocks' bits move with it ([VM] "显存管理与调度策略设计");
* ``free``     - release the listed sequences.

Caches are kept as integer bit patterns so that the GPU caches can be
compared bit for bit. A workload with an FP8 cache (``kv_cache_dtype`` "fp8")
keeps E4M3 codes plus one float32 scale per (token, head) row
(``quant.quantize_rows`` at append time); attention then runs on the
dequantised values code * scale.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import alloc_model, attention, cache_ops, error_bound, quant

_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8, "int8": np.int8}


@dataclass
class OpRecord:
    kind: str
    slots: List[int] = field(default_factory=list)
    copies: List[Tuple[int, int]] = field(default_factory=list)
    out: Optional[np.ndarray] = None          # decode: fp64 [len(seq_ids), Hq, d] (NaN where not sampled)
    bound: Optional[np.ndarray] = None        # decode with bound_partition set: error bound, same shape
    tables: Optional[np.ndarray] = None
    context_lens: Optional[np.ndarray] = None
    cached_tokens: int = 0                    # add_seq with prefix caching: leading tokens already cached


def candidate_tilings(i: int, tables: np.ndarray, ctx: np.ndarray, block_size: int, partition: int) -> list:
    """Range tilings a launch may use for sequence ``i`` of a decode batch:
    the context split into ``partition``-token ranges from token 0, and, for
    every other sequence of the batch whose table starts with the same
    physical blocks, the split at the end of that common run of whole blocks
    (a run read once for several sequences is tiled on its own)."""
    c = int(ctx[i])
    cands = {0}
    full_i = c // block_size
    for j in range(len(ctx)):
        if j == i:
            continue
        lim = min(full_i, int(ctx[j]) // block_size)
        k = 0
        while k < lim and tables[i][k] == tables[j][k]:
            k += 1
        if 0 < k * block_size:
            cands.add(k * block_size)
    return [error_bound.dense_partitions(c, partition) if f == 0 else
            error_bound.split_partitions(c, partition, f) for f in sorted(cands)]


class OracleReplay:
    def __init__(self, wl, bound_partition: Optional[int] = None):
        """``bound_partition``: also bound each decode output's error
        (``error_bound``) for launches with ranges of that many tokens."""
        self.wl = wl
        self.bound_partition = bound_partition
        self.alloc = alloc_model.BlockAllocatorModel(wl.num_blocks, wl.block_size, wl.free_order)
        shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
        # quantised caches (codes + one scale per row): "fp8" or "int8"
        self.qfmt = getattr(wl, "kv_cache_dtype", "") or ""
        self.fp8 = self.qfmt in ("fp8", "int8")
        cache_dt = self.qfmt if self.fp8 else wl.dtype
        self.k_bits = np.zeros(shape, dtype=_BITS[cache_dt])
        self.v_bits = np.zeros(shape, dtype=_BITS[cache_dt])
        if self.fp8:
            self.k_scale = np.zeros(shape[:3], dtype=np.float32)
            self.v_scale = np.zeros(shape[:3], dtype=np.float32)
        self.records: List[OpRecord] = []
        if getattr(wl, "prefix_caching", False):
            self.alloc.enable_prefix_caching()
        n_swap = getattr(wl, "num_swap_blocks", 0)
        if n_swap:
            self.alloc.set_swap_space(n_swap, wl.swap_free_order)
            sshape = (n_swap,) + shape[1:]
            self.swap_k = np.zeros(sshape, dtype=self.k_bits.dtype)
            self.swap_v = np.zeros(sshape, dtype=self.v_bits.dtype)
            if self.fp8:
                self.swap_k_scale = np.zeros(sshape[:3], dtype=np.float32)
                self.swap_v_scale = np.zeros(sshape[:3], dtype=np.float32)

    def _values(self, b: np.ndarray) -> np.ndarray:
        return cache_ops.decode_bits(b, self.wl.dtype)

    def _write(self, k, v, slots) -> None:
        """Store new rows at their slots: bit copies, or FP8 / INT8 quantisation."""
        if self.fp8:
            cache_ops.kv_append_fp8(self.k_bits, self.v_bits, self.k_scale, self.v_scale,
                                    attention.to_f64(k).astype(np.float32), attention.to_f64(v).astype(np.float32),
                                    slots, self.qfmt)
        else:
            cache_ops.kv_append(self.k_bits, self.v_bits, cache_ops.bits(k), cache_ops.bits(v), slots)

    def _copy(self, copies) -> None:
        cache_ops.copy_blocks(self.k_bits, self.v_bits, copies)
        if self.fp8:
            cache_ops.copy_blocks(self.k_scale, self.v_scale, copies)

    def _swap(self, pairs, out: bool) -> None:
        """Whole-block moves GPU cache -> swap space (``out``) or back."""
        gpu = [(self.k_bits, self.v_bits)]
        host = [(self.swap_k, self.swap_v)]
        if self.fp8:
            gpu.append((self.k_scale, self.v_scale))
            host.append((self.swap_k_scale, self.swap_v_scale))
        for (gk, gv), (hk, hv) in zip(gpu, host):
            if out:
                cache_ops.swap_blocks(gk, gv, hk, hv, pairs)
            else:
                cache_ops.swap_blocks(hk, hv, gk, gv, pairs)

    def _gather_values(self, bits, scales, table, ctx) -> np.ndarray:
        rows = attention.gather_sequence(bits, table, ctx)
        if not self.fp8:
            return self._values(rows)
        sc = attention.gather_sequence(scales[..., None], table, ctx)[..., 0]
        return quant.dequantize(rows, sc) if self.qfmt == "fp8" else quant.dequantize_int8(rows, sc)

    def decode(self, seq_ids: Sequence[int], q, sample: Optional[Dict[int, Sequence[int]]] = None) -> OpRecord:
        """fp64 attention for ``seq_ids``; with ``sample`` = {row: [heads]} only
        those (row, head) outputs are computed, the rest stay NaN."""
        wl = self.wl
        max_blocks = max(len(self.alloc.tables[s]) for s in seq_ids)
        tables, ctx = self.alloc.block_tables(seq_ids, max(max_blocks, 1))
        q64 = attention.to_f64(q)
        out = np.full((len(seq_ids), wl.num_q_heads, wl.head_dim), np.nan)
        bound = None if self.bound_partition is None else np.full_like(out, np.nan)
        rows = range(len(seq_ids)) if sample is None else sorted(sample)
        group = wl.num_q_heads // wl.num_kv_heads
        for i in rows:
            c = int(ctx[i])
            K = self._gather_values(self.k_bits, getattr(self, "k_scale", None), tables[i], c)
            V = self._gather_values(self.v_bits, getattr(self, "v_scale", None), tables[i], c)
            heads = list(range(wl.num_q_heads)) if sample is None else list(sample[i])
            if sample is None:
                out[i] = attention.dense_decode_one(q64[i], K, V, wl.scale)
            else:
                for h in heads:
                    kv = h // group
                    one = attention.dense_decode_one(q64[i, h:h + 1], K[:, kv:kv + 1], V[:, kv:kv + 1], wl.scale)
                    out[i, h] = one[0]
            if bound is not None:
                tilings = candidate_tilings(i, tables, ctx, wl.block_size, self.bound_partition)
                for h in heads:
                    kv = h // group
                    bound[i, h] = error_bound.decode_error_bound(q64[i, h:h + 1], K[:, kv:kv + 1], V[:, kv:kv + 1],
                                                                 wl.scale, tilings, wl.dtype)[0]
        return OpRecord("decode", out=out, bound=bound, tables=tables, context_lens=ctx)

    def apply(self, op, sample=None) -> OpRecord:
        wl = self.wl
        if op.kind == "add_seq":
            s = op.seq_ids[0]
            cached = 0
            if self.alloc.prefix_caching and getattr(op, "tokens", None) is not None:
                cached = self.alloc.add_seq_cached(s, op.tokens, op.extra_key)
            else:
                self.alloc.add_seq(s, op.num_tokens)
            slots = self.alloc.seq_slots(s, 0, op.num_tokens)
            self._write(op.k[cached:], op.v[cached:], slots[cached:])
            rec = OpRecord("add_seq", slots=slots, cached_tokens=cached)
        elif op.kind == "fork":
            self.alloc.fork(*op.seq_ids)
            rec = OpRecord("fork")
        elif op.kind == "append":
            slots, copies = self.alloc.append_slots(op.seq_ids)
            self._copy(copies)
            self._write(op.k, op.v, slots)
            rec = OpRecord("append", slots=slots, copies=copies)
        elif op.kind == "decode":
            rec = self.decode(op.seq_ids, op.q, sample)
        elif op.kind in ("swap_out", "swap_in"):
            pairs: List[Tuple[int, int]] = []
            for s in op.seq_ids:
                pairs += self.alloc.swap_out(s) if op.kind == "swap_out" else self.alloc.swap_in(s)
            self._swap(pairs, op.kind == "swap_out")
            rec = OpRecord(op.kind, copies=pairs)
        elif op.kind == "free":
            for s in op.seq_ids:
                self.alloc.free_seq(s)
            rec = OpRecord("free")
        else:
            raise ValueError(op.kind)
        self.records.append(rec)
        return rec

    def run(self, decode_sample=None, skip_decode: bool = False) -> List[OpRecord]:
        """Replay every op. ``decode_sample(op_index, op)`` may return a sample
        dict for a decode op (None = all outputs)."""
        for i, op in enumerate(self.wl.ops):
            if op.kind == "decode" and skip_decode:
                self.records.append(OpRecord("decode"))
                continue
            sample = decode_sample(i, op) if (decode_sample and op.kind == "decode") else None
            self.apply(op, sample)
        return self.records
