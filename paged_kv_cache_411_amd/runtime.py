"""One layer's paged KV cache on the GPU, driven by the host block allocator.

``PagedKVCache`` strings the library's calls together the way a decode step
uses them; it computes nothing itself:

* ``add_sequence``  - pa_alloc_add_seq + pa_alloc_seq_slots, then kv_append of
                      the prompt's K/V rows; with prefix caching and the
                      prompt's token ids, pa_alloc_add_seq_cached instead, and
                      kv_append only of the rows past the cached prefix;
* ``fork``          - pa_alloc_fork (blocks shared, counts + 1);
* ``append``        - pa_alloc_append_slots for one token per sequence; the
                      copy-on-write pairs it returns go to copy_blocks, then
                      kv_append writes the new rows (copies first, so that a
                      copied block carries the old contents before the writer
                      adds to it);
* ``decode``        - pa_alloc_block_tables, upload, pa_decode;
* ``free``          - pa_alloc_free_seq;
* ``swap_out`` / ``swap_in`` - pa_alloc_swap_out / pa_alloc_swap_in for each
                      listed sequence, then one swap_blocks launch that moves
                      the blocks between the device caches and the pinned
                      host swap space (eviction under memory pressure);
* ``step``          - one whole decode step (append one token to each listed
                      sequence, then decode them all) in one library call,
                      pa_decode_step: the allocator step writes the slots, copy
                      pairs, block tables and context lengths straight into a
                      pinned host buffer, the longest-first launch schedule
                      is added to it and the tables are packed behind the
                      schedule; copy_blocks reads its pairs there,
                      kv_append_staged moves the used part of the buffer to
                      the device and writes the new K/V rows (slots read from
                      the pinned buffer) in one launch on the same stream, and
                      pa_decode reads its packed tables, lengths and schedule
                      from the device copy. Python keeps only the ring of
                      pinned buffers.

Host-to-device uploads go through pinned staging memory with asynchronous
copies on the current stream.
"""

from __future__ import annotations

import math
import time
from typing import Optional, Sequence

import numpy as np
import torch

from . import _hip
from . import (DTYPE_CODES, PA_SWAP_IN, PA_SWAP_OUT, BlockAllocator, PagedKVError, StepDesc, cache_desc,
               copy_blocks, copy_blocks_fp8, decode_step, default_partition_size, kv_append, kv_append_fp8,
               kv_append_staged, pa_decode, pa_decode_share_width, pa_decode_workspace_bytes, step_layout,
               swap_blocks)


def _upload(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).pin_memory().to(device, non_blocking=True)


def _event_handle(ev) -> int:
    """hipEvent_t of a torch event or a ``_hip.Event``."""
    return ev.handle if isinstance(ev, _hip.Event) else ev.cuda_event


def _align(x: int, a: int = 256) -> int:
    return -(-x // a) * a


class _StagingRing:
    """The bookkeeping of a ring of ``depth`` host buffers released through a
    progress word: each step stamps the buffer it takes with the next
    sequence number; a buffer in use is handed out again only once
    ``word()`` has reached its stamp. Polling that has not seen it after
    ``spin_s`` seconds calls ``sync()`` (after which nothing reads any buffer)
    instead. Plain Python, no device calls of its own."""

    def __init__(self, depth: int, word, sync, spin_s: float):
        self.depth, self.word, self.sync, self.spin_s = depth, word, sync, spin_s
        self.stamp = [0] * depth
        self.in_use = [False] * depth
        self.serial = 0
        self.turn = 0
        self.waits = 0             # times a step waited for a buffer's last reader
        self.syncs = 0             # ... of which ended in a synchronise

    def next_free(self) -> int:
        """Index of the next buffer in turn, once nothing reads it."""
        i = self.turn
        if self.in_use[i]:
            if self.word() < self.stamp[i]:
                self.waits += 1
                end = time.perf_counter() + self.spin_s
                while self.word() < self.stamp[i]:
                    if time.perf_counter() > end:
                        # much work queued ahead, no later step yet, or a failed
                        # call: once the device is idle, nothing reads the buffer
                        self.syncs += 1
                        self.sync()
                        break
            self.in_use[i] = False
        return i

    def stamp_next(self, i: int) -> int:
        """Stamp buffer i for the next step; returns the number that step's
        first launch stores into the word: the previous step's stamp (every
        launch of the earlier steps has completed by then)."""
        self.serial += 1
        self.stamp[i] = self.serial
        return self.serial - 1

    def release(self, i: int) -> None:
        """Buffer i was handed to a step."""
        self.in_use[i] = True
        self.turn = (i + 1) % self.depth

    def drain(self) -> None:
        """Return once no enqueued work reads any buffer."""
        if any(u and self.word() < t for u, t in zip(self.in_use, self.stamp)):
            self.sync()
        self.in_use = [False] * self.depth


class _StepStaging:
    """A decode step's small inputs in one buffer laid out by the library
    (``pa_step_layout``): a ring of pinned host copies, each reused only after
    the launches that read it have run, and one device copy (stream order
    keeps it from being overwritten while a step still reads it).

    Each step stamps its host buffer with a sequence number and hands the
    library one pinned progress word (``done_flag``) with the previous
    step's number: the step's staging launch stores it there as it starts,
    when every launch of the earlier steps - all that read their buffers -
    has completed. A buffer is reused once the word has reached its stamp
    (``_StagingRing``), so the ring puts no event and no marker on the stream
    (either holds the next kernel back by microseconds), and the decode
    kernels carry nothing for it."""

    DEPTH = 8
    SPIN_S = 0.005   # polling the word longer than this falls back to a device synchronise

    def __init__(self, layout, device):
        self.layout = layout
        self.device = device
        self.n, self.width, self.part = layout.num_seqs, layout.width, layout.partition_size
        self.host = [torch.empty(layout.total, dtype=torch.uint8, pin_memory=True) for _ in range(self.DEPTH)]
        for h in self.host:
            h.zero_()   # the host's first touch of each page faults: take it here, not in a step
        self.host_ptr = [h.data_ptr() for h in self.host]
        n, o = self.n, layout.context_lens
        self.host_ctx = [h.numpy()[o:o + 4 * n].view(np.int32) for h in self.host]
        self.flag = torch.zeros(8, dtype=torch.int64, pin_memory=True)   # word 0; 64 bytes of their own
        self.flag_ptr = self.flag.data_ptr()
        self.word = self.flag.numpy()
        self.ring = _StagingRing(self.DEPTH, lambda: int(self.word[0]), lambda: torch.cuda.synchronize(device),
                                 self.SPIN_S)
        self.dev = torch.empty(layout.total, dtype=torch.uint8, device=device)
        t = layout.tables
        self.d_tables = self.dev[t:t + 4 * n * self.width].view(torch.int32).view(n, self.width)


class PagedKVCache:
    def __init__(self, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                 dtype: torch.dtype, device="cuda", free_order: Optional[Sequence[int]] = None,
                 schedule: bool = True, share: bool = True, kv_cache_dtype: str = "",
                 num_swap_blocks: int = 0, swap_free_order: Optional[Sequence[int]] = None,
                 prefix_caching: bool = False):
        self.device = torch.device(device)
        self.alloc = BlockAllocator(num_blocks, block_size, free_order)
        if prefix_caching:
            self.alloc.enable_prefix_caching()
        self.last_cached_tokens = 0    # leading prompt tokens the last add_sequence found cached
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        # "fp8" / "int8": the caches hold E4M3 / int8 codes with one float32
        # scale per (block, head, token) row
        if kv_cache_dtype not in ("", "fp8", "int8"):
            raise ValueError(f"kv_cache_dtype {kv_cache_dtype!r}: '', 'fp8' or 'int8'")
        self.fp8 = kv_cache_dtype in ("fp8", "int8")
        cache_dtype = (torch.int8 if kv_cache_dtype == "int8" else torch.uint8) if self.fp8 else dtype
        self.k_cache = torch.zeros(shape, dtype=cache_dtype, device=self.device)
        self.v_cache = torch.zeros(shape, dtype=cache_dtype, device=self.device)
        self.k_scale = torch.zeros(shape[:3], dtype=torch.float32, device=self.device) if self.fp8 else None
        self.v_scale = torch.zeros(shape[:3], dtype=torch.float32, device=self.device) if self.fp8 else None
        self.block_size = block_size
        self.head_dim = head_dim
        self.dtype = dtype
        self._workspace: Optional[torch.Tensor] = None
        self._staging: Optional[_StepStaging] = None
        self._step_desc: Optional[StepDesc] = None
        self._step_ws_need = 0
        self.schedule = schedule       # step() launches pa_decode with a longest-first schedule
        self.share = share             # ... whose shared-prompt partitions are read once per group
        self.last_context_lens: Optional[np.ndarray] = None   # host copy of the last decode's lengths
        # swap space: blocks of evicted sequences, in pinned host memory
        self.swap_k = self.swap_v = self.swap_k_scale = self.swap_v_scale = None
        if num_swap_blocks:
            self.alloc.set_swap_space(num_swap_blocks, swap_free_order)
            sshape = (num_swap_blocks,) + shape[1:]
            self.swap_k = torch.zeros(sshape, dtype=cache_dtype, pin_memory=True)
            self.swap_v = torch.zeros(sshape, dtype=cache_dtype, pin_memory=True)
            if self.fp8:
                self.swap_k_scale = torch.zeros(sshape[:3], dtype=torch.float32, pin_memory=True)
                self.swap_v_scale = torch.zeros(sshape[:3], dtype=torch.float32, pin_memory=True)

    def _dev(self, t: torch.Tensor) -> torch.Tensor:
        return t if t.device == self.k_cache.device else t.to(self.device, non_blocking=True)

    def _write(self, k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor, stage=None) -> None:
        """New rows into their slots: bit copies, or FP8 quantisation. ``stage``
        = (device dst, pinned src) is copied in the same launch."""
        if self.fp8:
            kv_append_fp8(k, v, slots, self.k_cache, self.v_cache, self.k_scale, self.v_scale,
                          *(stage if stage else (None, None)))
        elif stage:
            kv_append_staged(k, v, slots, self.k_cache, self.v_cache, *stage)
        else:
            kv_append(k, v, slots, self.k_cache, self.v_cache)

    def _copy(self, pairs: torch.Tensor) -> None:
        if self.fp8:
            copy_blocks_fp8(self.k_cache, self.v_cache, self.k_scale, self.v_scale, pairs)
        else:
            copy_blocks(self.k_cache, self.v_cache, pairs)

    def _scales(self) -> dict:
        return {"k_scale": self.k_scale, "v_scale": self.v_scale} if self.fp8 else {}

    def add_sequence(self, seq_id: int, k: torch.Tensor, v: torch.Tensor, tokens=None,
                     extra_key: int = 0) -> np.ndarray:
        """A new sequence holding the prompt rows ``k``/``v`` ``[n, Hkv, d]``.
        Given the prompt's token ids (and prefix caching is on), its cached
        leading blocks are reused and only the rows past them are written;
        ``last_cached_tokens`` says how many were skipped. Returns the slots of
        all n positions."""
        n = k.shape[0]
        cached = 0
        if tokens is not None:
            cached = self.alloc.add_seq_cached(seq_id, tokens, extra_key)
        else:
            self.alloc.add_seq(seq_id, n)
        self.last_cached_tokens = cached
        slots = self.alloc.seq_slots(seq_id, 0, n)
        if n > cached:
            self._write(self._dev(k[cached:]), self._dev(v[cached:]), _upload(slots[cached:], self.device))
        return slots

    def add_sequences(self, seq_ids: Sequence[int], k: torch.Tensor, v: torch.Tensor, lengths: Sequence[int],
                      tokens: Optional[Sequence] = None, extra_keys: Optional[Sequence[int]] = None,
                      prof_events=None) -> list:
        """Admit several prompts whose K/V rows lie back to back in ``k``/``v``
        ``[sum(lengths), Hkv, d]`` (a batched prefill's output): one
        pa_alloc_admit call for the batch (with the prompts' token ids, when
        given, through the prefix cache), then one kv_append launch in which
        the rows of each prompt's cached prefix carry slot -1 and are skipped.
        Returns each prompt's cached-prefix length. If the pool runs out part
        way, the prompts admitted so far are written and the error is raised.
        ``prof_events`` = (start, end) torch events recorded around the append
        launch."""
        flat = None if tokens is None else np.concatenate([np.asarray(t, dtype=np.int32) for t in tokens])
        err = None
        try:
            slots, cached = self.alloc.admit(seq_ids, lengths, flat, extra_keys)
        except Exception as e:   # the prompts before the failing one are admitted
            err = e
            slots, cached = getattr(e, "slots", np.empty(0, np.int64)), []
        if len(slots):
            d_slots = _upload(slots, self.device)
            if prof_events is not None:
                prof_events[0].record()
            self._write(self._dev(k), self._dev(v), d_slots)
            if prof_events is not None:
                prof_events[1].record()
        if err is not None:
            raise err
        self.last_cached_tokens = cached[-1] if cached else 0
        return cached

    def fork(self, parent: int, child: int) -> None:
        self.alloc.fork(parent, child)

    def append(self, seq_ids: Sequence[int], k: torch.Tensor, v: torch.Tensor):
        slots, pairs = self.alloc.append_slots(seq_ids)
        if len(pairs):
            self._copy(_upload(pairs, self.device))
        self._write(self._dev(k), self._dev(v), _upload(slots, self.device))
        return slots, pairs

    def free(self, seq_id: int) -> None:
        self.alloc.free_seq(seq_id)

    def _swap(self, seq_ids: Sequence[int], out: bool) -> np.ndarray:
        """Allocator moves for each listed sequence in order, then one launch
        for all their blocks. If the allocator refuses a sequence, the blocks
        of the ones before it are still moved, and the error is raised."""
        if self.swap_k is None:
            raise RuntimeError("this cache has no swap space")
        fn = self.alloc.swap_out if out else self.alloc.swap_in
        parts, err = [], None
        for s in seq_ids:
            try:
                parts.append(fn(int(s)))
            except Exception as e:   # earlier sequences have already moved in the allocator
                err = e
                break
        pairs = np.concatenate(parts) if parts else np.empty((0, 2), np.int64)
        if len(pairs):
            swap_blocks(self.k_cache, self.v_cache, self.swap_k, self.swap_v, _upload(pairs, self.device),
                        PA_SWAP_OUT if out else PA_SWAP_IN, k_scale=self.k_scale, v_scale=self.v_scale,
                        swap_k_scale=self.swap_k_scale, swap_v_scale=self.swap_v_scale)
        if err is not None:
            raise err
        return pairs

    def swap_out(self, seq_ids: Sequence[int]) -> np.ndarray:
        """Evict the listed sequences to the host swap space; returns the
        (device block, swap block) pairs moved. The host copies are complete
        once the current stream has been synchronised."""
        return self._swap(seq_ids, True)

    def swap_in(self, seq_ids: Sequence[int]) -> np.ndarray:
        """Bring the listed sequences back; returns the (swap block, device block) pairs."""
        return self._swap(seq_ids, False)

    def tables(self, seq_ids: Sequence[int]):
        mb = max(1, self.alloc.table_width(seq_ids))
        return self.alloc.block_tables(seq_ids, mb)

    def _ensure_workspace(self, q: torch.Tensor, tables: torch.Tensor, max_ctx: int, partition_size: int,
                          scheduled: bool = False) -> int:
        need = pa_decode_workspace_bytes(q, self.k_cache, tables, max_ctx, partition_size, scheduled)
        if need and (self._workspace is None or self._workspace.numel() < need):
            self._workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        return need

    def step(self, seq_ids: Sequence[int], k: Optional[torch.Tensor], v: Optional[torch.Tensor], q: torch.Tensor,
             out: Optional[torch.Tensor] = None, scale: Optional[float] = None, partition_size: int = 0,
             prof_events=None, append: bool = True) -> torch.Tensor:
        """One decode step: (if ``append``) one new token per listed sequence,
        whose K/V rows ``k``/``v`` ``[n, Hkv, d]`` go to the slots the
        allocator picks, after the copy-on-write copies it asks for; then
        attention of ``q`` ``[n, Hq, d]`` over every listed sequence. One
        library call (``pa_decode_step``) does the allocator step, the launch
        schedule and every launch; ``k``, ``v`` and ``q`` should already be on
        the device."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = ids.shape[0]
        Hkv, d = self.k_cache.shape[1], self.head_dim
        q = self._dev(q)
        if q.dim() != 3 or q.shape[0] != n or q.shape[2] != d or not q.is_contiguous():
            raise ValueError("q must be contiguous [n, Hq, d]")
        if append:
            k, v = self._dev(k), self._dev(v)
            for t in (k, v):
                if tuple(t.shape) != (n, Hkv, d) or t.dtype != q.dtype or not t.is_contiguous():
                    raise ValueError("k / v must be contiguous [n, Hkv, d] of q's dtype")
        if out is None:
            out = torch.empty_like(q)
        elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
            raise ValueError("out must be like q")
        if scale is None:
            scale = 1.0 / math.sqrt(self.head_dim)
        part = partition_size or default_partition_size(self.block_size)
        st = self._staging
        if st is None or st.n != n or st.part != part:
            st = self._new_staging(ids, append, n, part)
        try:
            return self._step(st, ids, append, k, v, q, out, scale, part, prof_events)
        except PagedKVError:
            # the staging's tables too narrow? (refused before anything moved)
            if self.alloc.table_width(ids, append) <= st.width:
                raise
            st = self._new_staging(ids, append, n, part)
            return self._step(st, ids, append, k, v, q, out, scale, part, prof_events)

    def _new_staging(self, ids, append, n, part) -> "_StepStaging":
        """Staging for n sequences whose tables fit, with room to grow by 64
        blocks each before the next one is needed."""
        width = max(1, self.alloc.table_width(ids, append))
        if self._staging is not None:
            self._staging.ring.drain()
        self._staging = _StepStaging(step_layout(n, _align(width + 64, 16), self.block_size, part), self.device)
        self._step_desc = None
        return self._staging

    def _step(self, st, ids, append, k, v, q, out, scale, part, prof_events):
        Hkv = self.k_cache.shape[1]
        desc = self._step_desc
        share = pa_decode_share_width() if (self.share and q.shape[1] == Hkv) else 1
        if desc is None or desc.num_q_heads != q.shape[1] or desc.q_dtype != DTYPE_CODES[q.dtype] \
                or desc.share_width != share:
            desc = self._step_desc = StepDesc()
            desc.cache = cache_desc(self.k_cache)
            desc.num_q_heads = q.shape[1]
            desc.q_dtype = DTYPE_CODES[q.dtype]
            desc.share_width = share
            desc.schedule = int(bool(self.schedule))
            desc.layout = st.layout
            if self.fp8:
                desc.k_scale, desc.v_scale = self.k_scale.data_ptr(), self.v_scale.data_ptr()
            # workspace bound: the table capacity of the layout (any context this staging can hold)
            self._step_ws_need = pa_decode_workspace_bytes(q, self.k_cache, st.d_tables, 0, part, bool(self.schedule))
            desc.dev_stage = st.dev.data_ptr()
        need = self._step_ws_need
        if need and (self._workspace is None or self._workspace.numel() < need):
            self._workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        desc.workspace = self._workspace.data_ptr() if need else None   # decode() may have replaced it
        desc.workspace_bytes = self._workspace.numel() if need else 0
        desc.scale = scale
        desc.prof_events[0] = _event_handle(prof_events[0]) if prof_events is not None else None
        desc.prof_events[1] = _event_handle(prof_events[1]) if prof_events is not None else None
        i = st.ring.next_free()
        desc.host_stage = st.host_ptr[i]
        desc.done_flag = st.flag_ptr
        desc.done_value = st.ring.stamp_next(i)
        try:
            decode_step(self.alloc, ids, append, k, v, q, out, self.k_cache, self.v_cache, desc)
        finally:
            # also after an error: a launch that reads the buffer may already be
            # enqueued (a stamp that never arrives ends in a device synchronise)
            st.ring.release(i)
        self.last_context_lens = st.host_ctx[i].copy()
        return out

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
        need = self._ensure_workspace(q, d_tables, max_ctx, partition_size)
        pa_decode(q, self.k_cache, self.v_cache, d_tables, d_ctx, scale, out, max_context_len=max_ctx,
                  partition_size=partition_size, workspace=self._workspace if need else None,
                  prof_events=prof_events, **self._scales())
        return out
