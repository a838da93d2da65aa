"""The one-call decode step's host side, on the CPU (no launch is reached):
the staging layout, and the refusals that must leave the allocator exactly
as it was - too narrow a layout, too small a workspace, an exhausted pool,
bad arguments."""

import ctypes

import numpy as np
import pytest

import paged_kv_cache_411_amd as pk
from tests.tables import compact_block_tables


def test_layout_offsets_and_capacity():
    L = pk.step_layout(128, 272, 16, 0)
    offs = [L.slots, L.pairs, L.context_lens, L.num_slots, L.members, L.work, L.tables, L.total]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    assert L.pairs - L.slots >= 8 * 128 and L.context_lens - L.pairs >= 16 * 128
    assert L.total - L.tables >= 4 * 128 * 272 and L.tables - L.work >= 32 * L.work_capacity
    assert L.partition_size == 1024
    # ranges per sequence: ceil(272 * 16 / 1024) + 1 = 6
    assert L.work_capacity == 128 * 6
    assert pk.step_layout(4, 8, 8, 0).partition_size == 512
    with pytest.raises(pk.PagedKVError):
        pk.step_layout(4, 8, 16, 100)        # not a multiple of the block size
    with pytest.raises(pk.PagedKVError):
        pk.step_layout(4, 0, 16, 0)


def _state(a: pk.BlockAllocator, ids):
    return (a.free_list(), a.ref_counts(), [a.seq_table(s) for s in ids], [a.context_len(s) for s in ids])


def _desc(n, width, workspace_bytes, dtype=1):
    d = pk.StepDesc()
    d.cache = pk.CacheDesc(32, 2, 16, 64, dtype)
    d.num_q_heads = 2
    d.q_dtype = dtype
    d.share_width = 1
    d.schedule = 1
    d.scale = 0.125
    d.workspace = 4096 if workspace_bytes else None     # never dereferenced on these paths
    d.workspace_bytes = workspace_bytes
    d.layout = pk.step_layout(n, width, 16, 0)
    d.host_stage = 4096
    d.dev_stage = 4096
    return d


def _call(a, ids, d, append=1):
    L = pk.lib()
    arr = np.ascontiguousarray(ids, dtype=np.int64)
    fake = ctypes.c_void_p(4096)   # device pointers; the refusals return before any launch
    mc = ctypes.c_int32(0)
    return L.pa_decode_step(a._h, arr.ctypes.data, arr.shape[0], append, fake, fake, fake, fake, fake, fake,
                            ctypes.byref(d), None, ctypes.byref(mc))


def test_refusals_leave_the_allocator_unchanged():
    a = pk.BlockAllocator(32, 16)
    a.add_seq(0, 16)      # next append opens a new block
    a.add_seq(1, 5)
    ids = [0, 1]
    before = _state(a, ids)
    big_ws = 1 << 30
    # too narrow: sequence 0 needs 2 columns after the append
    assert _call(a, ids, _desc(2, 1, big_ws)) == pk.PA_ERR_INVALID
    assert "blocks >" in pk.lib().pa_last_error().decode()
    assert _state(a, ids) == before
    # too small a workspace for a scheduled launch
    assert _call(a, ids, _desc(2, 16, 0)) == pk.PA_ERR_INVALID
    assert "workspace" in pk.lib().pa_last_error().decode()
    assert _state(a, ids) == before
    # layout for another batch size
    assert _call(a, ids, _desc(3, 16, big_ws)) == pk.PA_ERR_INVALID
    assert _state(a, ids) == before
    # unknown sequence
    assert _call(a, [0, 7], _desc(2, 16, big_ws)) == pk.PA_ERR_INVALID
    assert _state(a, ids) == before
    # q / out / new rows of another dtype than the cache (f32 rows on an f16 cache)
    d = _desc(2, 16, big_ws)
    d.q_dtype = 0
    assert _call(a, ids, d) == pk.PA_ERR_INVALID
    assert "q_dtype" in pk.lib().pa_last_error().decode()
    assert _state(a, ids) == before
    # a progress word that is not 8-byte aligned
    d = _desc(2, 16, big_ws)
    d.done_flag = 4096 + 4
    assert _call(a, ids, d) == pk.PA_ERR_INVALID
    assert "done_flag" in pk.lib().pa_last_error().decode()
    assert _state(a, ids) == before
    # FP8 caches take f16 / bf16 rows only
    d = _desc(2, 16, big_ws, dtype=3)
    d.k_scale = d.v_scale = 4096
    d.q_dtype = 0
    assert _call(a, ids, d) == pk.PA_ERR_INVALID
    assert _state(a, ids) == before
    # a misaligned new K row, q, or stage buffer: refused before the allocator moves
    for which in range(3):
        L = pk.lib()
        arr = np.ascontiguousarray(ids, dtype=np.int64)
        ptrs = [ctypes.c_void_p(4096) for _ in range(6)]
        d = _desc(2, 16, big_ws)
        if which < 2:
            ptrs[2 * which] = ctypes.c_void_p(4096 + 8)       # k_new, then q
        else:
            d.dev_stage = 4096 + 4
        mc = ctypes.c_int32(0)
        rc = L.pa_decode_step(a._h, arr.ctypes.data, 2, 1, *ptrs, ctypes.byref(d), None, ctypes.byref(mc))
        assert rc == pk.PA_ERR_INVALID and "aligned" in L.pa_last_error().decode()
        assert _state(a, ids) == before
    # a scale that is not finite
    d = _desc(2, 16, big_ws)
    d.scale = float("nan")
    assert _call(a, ids, d) == pk.PA_ERR_INVALID
    assert _state(a, ids) == before
    # an exhausted pool: all-or-nothing
    b = pk.BlockAllocator(2, 16)
    b.add_seq(0, 16)
    b.add_seq(1, 16)
    ids_b = [0, 1]
    before_b = _state(b, ids_b)
    assert _call(b, ids_b, _desc(2, 16, big_ws)) == pk.PA_ERR_NO_BLOCKS
    assert _state(b, ids_b) == before_b


@pytest.mark.parametrize("share", [1, 4])
def test_step_packs_tables_behind_the_schedule(share):
    """The staging buffer a scheduled step uploads, inspected on the host
    after the step's host half (pa_decode_step_plan: the allocator step, the
    schedule and the packing; nothing launched). The lengths are the appended ones; the items are
    pa_decode_schedule's over the padded tables, each naming its sequence's
    row; the rows follow the items back to back, each the sequence's whole
    table."""
    B = 16
    a = pk.BlockAllocator(96, B, np.random.default_rng(2).permutation(96).astype(np.int32))
    ctxs = [5, 40, 0, 33, 100, 16, 704]
    for i, c in enumerate(ctxs):
        a.add_seq(i, c)
    a.fork(6, 7)                                     # a shared prompt: shared items when share > 1
    ids = np.arange(8, dtype=np.int64)
    width = a.table_width(ids, True)
    L = pk.step_layout(len(ids), width, B, 256)
    host = np.zeros(L.total + 16, np.uint8)
    off = (-host.ctypes.data) % 16                  # the host half needs a 16-byte aligned buffer
    host = host[off:off + L.total]
    d = _desc(len(ids), width, 1 << 30)
    d.cache = pk.CacheDesc(96, 2, B, 64, 1)
    d.share_width = share
    d.layout = L
    d.host_stage = host.ctypes.data
    plan = pk.StepPlan()
    rc = pk.lib().pa_decode_step_plan(a._h, ids.ctypes.data, len(ids), 1, ctypes.byref(d), ctypes.byref(plan))
    assert rc == pk.PA_OK, pk.lib().pa_last_error()
    assert plan.num_cow == 0 and plan.max_context == 705
    ctx = host[L.context_lens:L.context_lens + 4 * len(ids)].view(np.int32)
    assert ctx.tolist() == [c + 1 for c in ctxs] + [705]
    tables, want_ctx = a.block_tables(ids, width)
    assert np.array_equal(ctx, want_ctx)
    sched = pk.pa_decode_schedule(ctx.copy(), B, 256, int(ctx.max()), tables, share)
    nw = len(sched.work)
    if share > 1:
        assert len(sched.members) > 0
    work = host[L.work:L.work + 32 * nw].view(np.int32).reshape(nw, 8)
    assert np.array_equal(work[:, :6], sched.work[:, :6])
    nb = (ctx + B - 1) // B
    starts = np.concatenate([[0], np.cumsum(nb)[:-1]])
    assert work[:, 6].tolist() == starts[work[:, 0]].tolist()
    assert work[:, 7].tolist() == nb[work[:, 0]].tolist()
    at = L.work + -(-32 * nw // 16) * 16
    packed = host[at:at + 4 * int(nb.sum())].view(np.int32)
    assert packed.tolist() == [b for s in ids for b in a.seq_table(int(s))]
    flat, w2 = compact_block_tables(tables, ctx, B, sched.work)   # the test helper agrees
    assert np.array_equal(flat, packed) and np.array_equal(w2, work)
