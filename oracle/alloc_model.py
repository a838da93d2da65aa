"""Oracle: the physical block allocator, in plain Python (TEST INFRASTRUCTURE).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.

Rules, and where the pages state them:

* Free pool as a FIFO queue: a new block is taken from the head and a freed
  block goes back to the tail ([VM] "Python 演示": ``free_blocks.pop(0)`` and
  ``free_blocks.append``; [KVM] Part 4 "BlockPool": ``allocate()`` pops from the
  head of the free queue). The initial order is given (default 0..N-1).
* An empty pool is an error and changes nothing ([VM] "Python 演示" raises
  MemoryError; [KVM] Part 4 ``allocate_slots()`` checks the free capacity first
  and either commits or returns None). A request for several blocks is
  all-or-nothing.
* On-demand growth ([PA] §3.3 "按需分配策略"; [VM] "虚拟内存分页机制到KV Cache的映射"):
  to append a token, check whether the current logical block has room; if not,
  take a new physical block and add it to the block table; then the token's
  K/V is written to its slot.
* Sharing ([VM] "写时复制与块共享机制"): sequences that share KV point their table
  entries at the same physical block, whose reference count goes up by one.
* Copy-on-write (same section, and [PA] §4.1): before a sequence modifies a
  shared block it checks the count; at 1 it writes in place; above 1 it copies
  the block to a new physical block, writes there, remaps its table entry and
  decrements the old block's count.
* Free ([VM] "写时复制与块共享机制", last paragraph): when a sequence finishes, each
  block it references loses one count, and a block at 0 returns to the pool.
* Automatic prefix caching ([KVM] Part 3 and Part 4): optional. A full block
  is indexed by a chained content key - block N's key covers the tokens of
  blocks 0..N (block N's own tokens plus block N-1's key) and extra keys such
  as an adapter id - so two requests share block N only when everything up
  to and including it matches. A finished request's blocks return to the
  free queue still indexed. A new request walks its prompt's chain from the
  first block and takes every leading block that is indexed (get computed
  blocks): an indexed block that sits in the free queue is pulled out of it
  (the page's reason for a doubly-linked queue: removal from any position),
  one in use gains a count. Taking a block from the head of the queue drops
  its index entry first (lazy eviction).
* Swap ([VM] "显存管理与调度策略设计", last paragraph): under memory pressure
  the blocks of a waiting request can be evicted - their KV moved to CPU
  memory - to make room, and moved back to GPU memory when that request is
  scheduled again.

Readings where the pages are silent:
  * blocks of a finished sequence are released in ascending logical order;
  * when several sequences of one append call write into the same shared
    block, they are handled in the order given (ascending sequence id in every
    workload), so the first ones copy and the last one writes in place;
  * a slot is ``physical_block * block_size + offset``; -1 pads a block table;
  * the watermark (a reserve of free blocks, [VM] "显存管理与调度策略设计") is a
    query ``can_allocate``; it does not refuse allocations by itself;
  * swap space is a second pool of CPU-side block ids with the same FIFO
    rules. Swapping a sequence out gives each of its table entries, in
    logical order, a swap block from the head of that pool and releases the
    GPU block as a finished sequence would (count - 1, to the tail at 0), so
    a block shared with another sequence stays on the GPU for the others and
    the swapped sequence keeps its own copy. Swapping in takes GPU blocks
    from the head, in logical order, each with count 1, and returns the swap
    blocks to the swap pool's tail. Both need the whole table's worth of free
    blocks or change nothing. A swapped-out sequence cannot grow, fork or be
    decoded; freeing it returns its swap blocks;
  * prefix caching indexes the full blocks of a prompt only (a partial block
    and blocks filled later by decoding are not indexed); the chain walk stops
    at the first block that is not indexed; the caller writes K/V only for the
    positions past the cached prefix; a key that is already indexed keeps its
    block (a second block with the same content stays unindexed); blocks that
    come back from swap space are not re-indexed. Content keys here are exact
    (an interned tuple per block), so a lookup never hits a block with
    different content.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


class NoFreeBlocks(MemoryError):
    """The pool cannot supply the blocks a call needs; nothing was changed."""


class InvalidOperation(ValueError):
    """Unknown / duplicate sequence id or an argument out of range."""


class BlockAllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        if num_blocks < 0 or block_size <= 0:
            raise InvalidOperation("bad pool geometry")
        self.num_blocks = num_blocks
        self.block_size = block_size
        if free_order is None:
            self.free_blocks: List[int] = list(range(num_blocks))
        else:
            self.free_blocks = [int(b) for b in free_order]
            if sorted(self.free_blocks) != list(range(num_blocks)):
                raise InvalidOperation("initial free order must be a permutation of 0..N-1")
        self.ref_counts: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.context_lens: Dict[int, int] = {}
        self.watermark = 0.0
        self.swap_free: List[int] = []      # FIFO of free swap-space block ids
        self.swapped: set = set()           # sequences whose table lists swap blocks
        self.prefix_caching = False
        self._keys: Dict[tuple, int] = {}   # (parent key, block tokens, extra) -> content key
        self.cached: Dict[int, int] = {}    # content key -> block
        self.block_key: Dict[int, int] = {} # block -> content key

    # -- pool ------------------------------------------------------------
    def _take(self) -> int:
        phys = self.free_blocks.pop(0)      # head of the FIFO
        if phys in self.block_key:          # lazy eviction of a cached block
            del self.cached[self.block_key.pop(phys)]
        self.ref_counts[phys] = 1
        return phys

    def _release(self, phys: int) -> None:
        self.ref_counts[phys] -= 1
        if self.ref_counts[phys] == 0:
            self.free_blocks.append(phys)   # tail of the FIFO

    def num_free(self) -> int:
        return len(self.free_blocks)

    def set_watermark(self, fraction: float) -> None:
        if not 0.0 <= fraction < 1.0:
            raise InvalidOperation("watermark must be in [0, 1)")
        self.watermark = fraction

    def can_allocate(self, n: int) -> bool:
        """True when taking ``n`` blocks leaves at least watermark * N free."""
        return len(self.free_blocks) - n >= self.watermark * self.num_blocks

    # -- sequences -------------------------------------------------------
    def add_seq(self, seq_id: int, num_tokens: int) -> None:
        if seq_id in self.tables or num_tokens < 0:
            raise InvalidOperation(f"add_seq({seq_id}, {num_tokens})")
        n = -(-num_tokens // self.block_size)
        if n > len(self.free_blocks):
            raise NoFreeBlocks(f"need {n} blocks, {len(self.free_blocks)} free")
        self.tables[seq_id] = [self._take() for _ in range(n)]
        self.context_lens[seq_id] = num_tokens

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables or child in self.tables or parent in self.swapped:
            raise InvalidOperation(f"fork({parent}, {child})")
        table = list(self.tables[parent])
        for phys in table:
            self.ref_counts[phys] += 1
        self.tables[child] = table
        self.context_lens[child] = self.context_lens[parent]

    def append_slots(self, seq_ids: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One new token for each listed sequence, in order. Returns the slot of
        each new token and the (src, dst) block copies copy-on-write needs.
        All-or-nothing: if the pool cannot cover every new block, nothing
        changes and NoFreeBlocks is raised."""
        if len(set(seq_ids)) != len(seq_ids) or any(s not in self.tables or s in self.swapped for s in seq_ids):
            raise InvalidOperation("append_slots: unknown, repeated or swapped-out sequence id")
        B = self.block_size
        # dry run: count the blocks this call takes, with the counts as they
        # evolve along the list
        refs = {}
        need = 0
        for s in seq_ids:
            pos = self.context_lens[s]
            if pos % B == 0:
                need += 1
            else:
                last = self.tables[s][-1]
                r = refs.get(last, self.ref_counts[last])
                if r > 1:
                    need += 1
                    refs[last] = r - 1
        if need > len(self.free_blocks):
            raise NoFreeBlocks(f"need {need} blocks, {len(self.free_blocks)} free")
        slots: List[int] = []
        copies: List[Tuple[int, int]] = []
        for s in seq_ids:
            table = self.tables[s]
            pos = self.context_lens[s]
            if pos % B == 0:
                table.append(self._take())
            else:
                last = table[-1]
                if self.ref_counts[last] > 1:
                    new = self._take()
                    copies.append((last, new))
                    self.ref_counts[last] -= 1
                    table[-1] = new
            slots.append(table[pos // B] * B + pos % B)
            self.context_lens[s] = pos + 1
        return slots, copies

    def free_seq(self, seq_id: int) -> None:
        if seq_id not in self.tables:
            raise InvalidOperation(f"free_seq({seq_id})")
        table = self.tables.pop(seq_id)
        if seq_id in self.swapped:
            self.swapped.discard(seq_id)
            self.swap_free.extend(table)    # swap blocks back to the swap pool's tail
        else:
            for phys in table:
                self._release(phys)
        del self.context_lens[seq_id]

    # -- prefix caching --------------------------------------------------
    def enable_prefix_caching(self) -> None:
        if self.tables:
            raise InvalidOperation("enable prefix caching before any sequence exists")
        self.prefix_caching = True

    def _chain(self, tokens: Sequence[int], extra: int, create: bool) -> List[Optional[int]]:
        """Content keys of the prompt's full blocks, first block first; None
        for a block (and every block after it) whose content was never seen,
        unless ``create``."""
        B = self.block_size
        keys: List[Optional[int]] = []
        parent = -1
        for j in range(len(tokens) // B):
            ident = (parent, tuple(int(t) for t in tokens[j * B:(j + 1) * B]), int(extra))
            if ident not in self._keys:
                if not create:
                    keys += [None] * (len(tokens) // B - j)
                    return keys
                self._keys[ident] = len(self._keys)
            parent = self._keys[ident]
            keys.append(parent)
        return keys

    def prefix_hits(self, tokens: Sequence[int], extra: int = 0) -> List[int]:
        """Blocks holding the longest indexed run of the prompt's leading full blocks."""
        hits = []
        for k in self._chain(tokens, extra, create=False):
            if k is None or k not in self.cached:
                break
            hits.append(self.cached[k])
        return hits

    def add_seq_cached(self, seq_id: int, tokens: Sequence[int], extra: int = 0) -> int:
        """A new sequence for a prompt with prefix caching: reuse the indexed
        leading blocks, take the rest from the queue head, index the prompt's
        full blocks. Returns the number of leading tokens whose K/V is already
        in the cache. All-or-nothing."""
        if not self.prefix_caching or seq_id in self.tables:
            raise InvalidOperation(f"add_seq_cached({seq_id})")
        B = self.block_size
        n = len(tokens)
        hits = self.prefix_hits(tokens, extra)
        need = -(-n // B) - len(hits)
        idle = sum(1 for b in hits if self.ref_counts[b] == 0)   # hits that sit in the free queue
        if need > len(self.free_blocks) - idle:
            raise NoFreeBlocks(f"need {need} blocks, {len(self.free_blocks) - idle} free")
        for b in hits:
            if self.ref_counts[b] == 0:
                self.free_blocks.remove(b)  # out of the queue, from wherever it sits
            self.ref_counts[b] += 1
        table = hits + [self._take() for _ in range(need)]
        for j, k in enumerate(self._chain(tokens, extra, create=True)):
            if j >= len(hits) and k not in self.cached:
                self.cached[k] = table[j]
                self.block_key[table[j]] = k
        self.tables[seq_id] = table
        self.context_lens[seq_id] = n
        return len(hits) * B

    def cached_blocks(self) -> List[int]:
        return sorted(self.block_key)

    # -- swap space ------------------------------------------------------
    def set_swap_space(self, num_blocks: int, free_order: Optional[Sequence[int]] = None) -> None:
        if self.swapped or num_blocks < 0:
            raise InvalidOperation("set_swap_space")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidOperation("swap free order must be a permutation of 0..S-1")
        self.swap_free = order

    def swap_out(self, seq_id: int) -> List[Tuple[int, int]]:
        """Evict a sequence to swap space; returns the (GPU block, swap block)
        copies that must run before its GPU blocks are reused."""
        if seq_id not in self.tables or seq_id in self.swapped:
            raise InvalidOperation(f"swap_out({seq_id})")
        table = self.tables[seq_id]
        if len(table) > len(self.swap_free):
            raise NoFreeBlocks(f"need {len(table)} swap blocks, {len(self.swap_free)} free")
        host = [self.swap_free.pop(0) for _ in table]
        pairs = list(zip(table, host))
        for phys in table:
            self._release(phys)
        self.tables[seq_id] = host
        self.swapped.add(seq_id)
        return pairs

    def swap_in(self, seq_id: int) -> List[Tuple[int, int]]:
        """Bring a swapped-out sequence back; returns the (swap block, GPU block) copies."""
        if seq_id not in self.swapped:
            raise InvalidOperation(f"swap_in({seq_id})")
        host = self.tables[seq_id]
        if len(host) > len(self.free_blocks):
            raise NoFreeBlocks(f"need {len(host)} blocks, {len(self.free_blocks)} free")
        gpu = [self._take() for _ in host]
        self.swap_free.extend(host)
        self.tables[seq_id] = gpu
        self.swapped.discard(seq_id)
        return list(zip(host, gpu))

    # -- views -----------------------------------------------------------
    def seq_slots(self, seq_id: int, start: int, count: int) -> List[int]:
        """Slots of positions start .. start+count-1 of a sequence."""
        if seq_id in self.swapped:
            raise InvalidOperation(f"sequence {seq_id} is swapped out")
        table = self.tables[seq_id]
        B = self.block_size
        if start < 0 or start + count > len(table) * B:
            raise InvalidOperation("positions outside the sequence's blocks")
        return [table[p // B] * B + p % B for p in range(start, start + count)]

    def block_tables(self, seq_ids: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
        out = np.full((len(seq_ids), max_blocks), -1, dtype=np.int32)
        ctx = np.zeros(len(seq_ids), dtype=np.int32)
        for i, s in enumerate(seq_ids):
            if s in self.swapped:
                raise InvalidOperation(f"sequence {s} is swapped out")
            table = self.tables[s]
            if len(table) > max_blocks:
                raise InvalidOperation(f"sequence {s} has {len(table)} blocks > {max_blocks}")
            out[i, :len(table)] = table
            ctx[i] = self.context_lens[s]
        return out, ctx
