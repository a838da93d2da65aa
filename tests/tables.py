"""Test helper: the compact block-table form pa_decode accepts with a schedule."""

from __future__ import annotations

from typing import Tuple

import numpy as np


def compact_block_tables(block_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
                         work: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Pack padded tables ``[S, max_blocks]`` into one int32 array, each row
    cut to its ceil(ctx / block_size) entries and placed after the rows before
    it, and return it with a copy of the schedule ``work`` whose ints 6 and 7
    give each item's row (start, length)."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    nb = (ctx + block_size - 1) // block_size
    starts = np.concatenate([[0], np.cumsum(nb)[:-1]]).astype(np.int32)
    flat = np.concatenate([block_tables[i, :nb[i]] for i in range(len(nb))] + [np.zeros(0, np.int32)])
    w = np.array(work, dtype=np.int32, copy=True)
    w[:, 6] = starts[w[:, 0]]
    w[:, 7] = nb[w[:, 0]]
    return np.ascontiguousarray(flat, dtype=np.int32), w
