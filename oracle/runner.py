"""Oracle: replay a workload's host operations (TEST INFRASTRUCTURE).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.

Each operation of a ``workloads.Workload`` is carried out with the oracle's
own allocator model, bitwise cache operations and fp64 attention:

* ``add_seq``  - allocate the prompt's blocks, then write every prompt token
                 into its slot ([PA] §3.3 steps 2-4);
* ``fork``     - share every block of the parent ([VM] "写时复制与块共享机制");
* ``append``   - one slot per listed sequence; the copy-on-write block copies
                 of the step run before the new tokens are written (a copy
                 must carry the old contents into the new block before the
                 writer modifies it, [PA] §4.1 steps 1-3);
* ``decode``   - gather + fp64 attention for the listed sequences.

Caches are kept as integer bit patterns so that the GPU caches can be
compared bit for bit.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import alloc_model, attention, cache_ops

_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


@dataclass
class OpRecord:
    kind: str
    slots: List[int] = field(default_factory=list)
    copies: List[Tuple[int, int]] = field(default_factory=list)
    out: Optional[np.ndarray] = None          # decode: fp64 [len(seq_ids), Hq, d] (NaN where not sampled)
    tables: Optional[np.ndarray] = None
    context_lens: Optional[np.ndarray] = None


class OracleReplay:
    def __init__(self, wl):
        self.wl = wl
        self.alloc = alloc_model.BlockAllocatorModel(wl.num_blocks, wl.block_size, wl.free_order)
        shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
        self.k_bits = np.zeros(shape, dtype=_BITS[wl.dtype])
        self.v_bits = np.zeros(shape, dtype=_BITS[wl.dtype])
        self.records: List[OpRecord] = []

    def _values(self, b: np.ndarray) -> np.ndarray:
        return cache_ops.decode_bits(b, self.wl.dtype)

    def decode(self, seq_ids: Sequence[int], q, sample: Optional[Dict[int, Sequence[int]]] = None) -> OpRecord:
        """fp64 attention for ``seq_ids``; with ``sample`` = {row: [heads]} only
        those (row, head) outputs are computed, the rest stay NaN."""
        wl = self.wl
        max_blocks = max(len(self.alloc.tables[s]) for s in seq_ids)
        tables, ctx = self.alloc.block_tables(seq_ids, max(max_blocks, 1))
        q64 = attention.to_f64(q)
        out = np.full((len(seq_ids), wl.num_q_heads, wl.head_dim), np.nan)
        rows = range(len(seq_ids)) if sample is None else sorted(sample)
        group = wl.num_q_heads // wl.num_kv_heads
        for i in rows:
            c = int(ctx[i])
            K = self._values(attention.gather_sequence(self.k_bits, tables[i], c))
            V = self._values(attention.gather_sequence(self.v_bits, tables[i], c))
            heads = range(wl.num_q_heads) if sample is None else sample[i]
            if sample is None:
                out[i] = attention.dense_decode_one(q64[i], K, V, wl.scale)
            else:
                for h in heads:
                    kv = h // group
                    one = attention.dense_decode_one(q64[i, h:h + 1], K[:, kv:kv + 1], V[:, kv:kv + 1], wl.scale)
                    out[i, h] = one[0]
        return OpRecord("decode", out=out, tables=tables, context_lens=ctx)

    def apply(self, op, sample=None) -> OpRecord:
        wl = self.wl
        if op.kind == "add_seq":
            s = op.seq_ids[0]
            self.alloc.add_seq(s, op.num_tokens)
            slots = self.alloc.seq_slots(s, 0, op.num_tokens)
            cache_ops.kv_append(self.k_bits, self.v_bits, cache_ops.bits(op.k), cache_ops.bits(op.v), slots)
            rec = OpRecord("add_seq", slots=slots)
        elif op.kind == "fork":
            self.alloc.fork(*op.seq_ids)
            rec = OpRecord("fork")
        elif op.kind == "append":
            slots, copies = self.alloc.append_slots(op.seq_ids)
            cache_ops.copy_blocks(self.k_bits, self.v_bits, copies)
            cache_ops.kv_append(self.k_bits, self.v_bits, cache_ops.bits(op.k), cache_ops.bits(op.v), slots)
            rec = OpRecord("append", slots=slots, copies=copies)
        elif op.kind == "decode":
            rec = self.decode(op.seq_ids, op.q, sample)
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
