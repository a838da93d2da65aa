"""One layer's paged KV cache on the GPU, driven by the host block allocator.

``PagedKVCache`` strings the library's calls together the way a decode step
uses them; it computes nothing itself:

* ``add_sequence``  - pa_alloc_add_seq + pa_alloc_seq_slots, then kv_append of
                      the prompt's K/V rows;
* ``fork``          - pa_alloc_fork (blocks shared, counts + 1);
* ``append``        - pa_alloc_append_slots for one token per sequence; the
                      copy-on-write pairs it returns go to copy_blocks, then
                      kv_append writes the new rows (copies first, so that a
                      copied block carries the old contents before the writer
                      adds to it);
* ``decode``        - pa_alloc_block_tables, upload, pa_decode;
* ``free``          - pa_alloc_free_seq.

Host-to-device uploads go through pinned staging memory with asynchronous
copies on the current stream.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
import torch

from . import BlockAllocator, copy_blocks, kv_append, pa_decode, pa_decode_workspace_bytes


def _upload(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).pin_memory().to(device, non_blocking=True)


class PagedKVCache:
    def __init__(self, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                 dtype: torch.dtype, device="cuda", free_order: Optional[Sequence[int]] = None):
        self.device = torch.device(device)
        self.alloc = BlockAllocator(num_blocks, block_size, free_order)
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.k_cache = torch.zeros(shape, dtype=dtype, device=self.device)
        self.v_cache = torch.zeros(shape, dtype=dtype, device=self.device)
        self.block_size = block_size
        self.head_dim = head_dim
        self.dtype = dtype
        self._workspace: Optional[torch.Tensor] = None
        self.last_context_lens: Optional[np.ndarray] = None   # host copy of the last decode's lengths

    def _dev(self, t: torch.Tensor) -> torch.Tensor:
        return t.to(self.device, non_blocking=True)

    def add_sequence(self, seq_id: int, k: torch.Tensor, v: torch.Tensor) -> np.ndarray:
        n = k.shape[0]
        self.alloc.add_seq(seq_id, n)
        slots = self.alloc.seq_slots(seq_id, 0, n)
        if n:
            kv_append(self._dev(k), self._dev(v), _upload(slots, self.device), self.k_cache, self.v_cache)
        return slots

    def fork(self, parent: int, child: int) -> None:
        self.alloc.fork(parent, child)

    def append(self, seq_ids: Sequence[int], k: torch.Tensor, v: torch.Tensor):
        slots, pairs = self.alloc.append_slots(seq_ids)
        if len(pairs):
            copy_blocks(self.k_cache, self.v_cache, _upload(pairs, self.device))
        kv_append(self._dev(k), self._dev(v), _upload(slots, self.device), self.k_cache, self.v_cache)
        return slots, pairs

    def free(self, seq_id: int) -> None:
        self.alloc.free_seq(seq_id)

    def tables(self, seq_ids: Sequence[int]):
        mb = max(1, max(self.alloc.num_table_blocks(s) for s in seq_ids))
        return self.alloc.block_tables(seq_ids, mb)

    def decode(self, seq_ids: Sequence[int], q: torch.Tensor, out: Optional[torch.Tensor] = None,
               scale: Optional[float] = None, partition_size: int = 0, prof_events=None) -> torch.Tensor:
        tables, ctx = self.tables(seq_ids)
        self.last_context_lens = ctx
        q = self._dev(q)
        if out is None:
            out = torch.empty_like(q)
        if scale is None:
            scale = 1.0 / math.sqrt(self.head_dim)
        d_tables = _upload(tables, self.device)
        d_ctx = _upload(ctx, self.device)
        max_ctx = max(1, int(ctx.max()))
        need = pa_decode_workspace_bytes(q, self.k_cache, d_tables, max_ctx, partition_size)
        if need and (self._workspace is None or self._workspace.numel() < need):
            self._workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        pa_decode(q, self.k_cache, self.v_cache, d_tables, d_ctx, scale, out, max_context_len=max_ctx,
                  partition_size=partition_size, workspace=self._workspace if need else None,
                  prof_events=prof_events)
        return out
