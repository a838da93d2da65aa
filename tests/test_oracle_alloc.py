"""Pins for the oracle's block allocator model (CPU only).

* a trace worked out by hand from the pages' rules (tests/golden/alloc_trace.json);
* invariants under random operation sequences (hypothesis): every block is
  either free or referenced, reference counts equal table occurrences,
  internal fragmentation is at most B-1 slots per sequence, and freeing every
  sequence returns every block;
* closed counts on the workloads: 16 appends give each sequence exactly one
  new block; a shared partial block shared by k beams is copied k-1 times.
"""

import json
import os
from collections import Counter

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads
from oracle import alloc_model, runner
from oracle.alloc_model import BlockAllocatorModel, InvalidOperation, NoFreeBlocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _state(a: BlockAllocatorModel):
    return {
        "free": list(a.free_blocks),
        "tables": {str(k): list(v) for k, v in a.tables.items()},
        "ctx": {str(k): v for k, v in a.context_lens.items()},
        "refs": list(a.ref_counts),
    }


def run_trace_step(a, step):
    """Apply one golden trace step; returns (result dict, error kind or None)."""
    op = step["op"]
    try:
        if op == "add_seq":
            a.add_seq(step["seq"], step["tokens"])
            return {}, None
        if op == "fork":
            a.fork(step["parent"], step["child"])
            return {}, None
        if op == "append":
            slots, copies = a.append_slots(step["seqs"])
            return {"slots": slots, "copies": [list(c) for c in copies]}, None
        if op == "free_seq":
            a.free_seq(step["seq"])
            return {}, None
        if op == "block_tables":
            t, c = a.block_tables(step["seqs"], step["max_blocks"])
            return {"tables": t.tolist(), "ctx": c.tolist()}, None
    except NoFreeBlocks:
        return {}, "no_blocks"
    except InvalidOperation:
        return {}, "invalid"
    raise ValueError(op)


def test_hand_worked_trace():
    trace = json.load(open(os.path.join(GOLDEN, "alloc_trace.json")))
    a = BlockAllocatorModel(trace["num_blocks"], trace["block_size"])
    for i, step in enumerate(trace["steps"]):
        res, err = run_trace_step(a, step)
        assert err == step.get("error"), (i, step)
        exp = step["expect"]
        if step["op"] == "block_tables":
            assert res == exp, i
            continue
        for key in ("slots", "copies"):
            if key in exp:
                assert res[key] == exp[key], (i, key)
        st_ = _state(a)
        for key in ("free", "tables", "ctx", "refs"):
            assert st_[key] == exp[key], (i, key, st_[key], exp[key])


def test_fresh_pool_order_and_empty_error():
    """[VM] Python 演示: blocks come out 0, 1, 2, ... on a fresh pool; a freed block
    goes to the end of the list; an empty pool is an error."""
    a = BlockAllocatorModel(3, 16)
    a.add_seq(0, 16)
    a.add_seq(1, 17)
    assert a.tables == {0: [0], 1: [1, 2]}
    with pytest.raises(MemoryError):
        a.add_seq(2, 1)
    a.free_seq(0)
    assert a.free_blocks == [0]
    a.add_seq(2, 1)
    assert a.tables[2] == [0]


def test_invalid_ops():
    a = BlockAllocatorModel(4, 4)
    with pytest.raises(InvalidOperation):
        a.free_seq(5)
    a.add_seq(1, 2)
    with pytest.raises(InvalidOperation):
        a.add_seq(1, 2)
    with pytest.raises(InvalidOperation):
        a.fork(2, 3)
    with pytest.raises(InvalidOperation):
        a.append_slots([1, 1])
    with pytest.raises(InvalidOperation):
        BlockAllocatorModel(3, 4, free_order=[0, 0, 1])


def check_invariants(a: BlockAllocatorModel):
    N, B = a.num_blocks, a.block_size
    free = a.free_blocks
    assert len(set(free)) == len(free)
    used = {b for b in range(N) if a.ref_counts[b] > 0}
    assert not (used & set(free))
    assert len(free) + len(used) == N
    occ = Counter(b for t in a.tables.values() for b in t)
    for b in range(N):
        assert a.ref_counts[b] == occ.get(b, 0)
    for s, t in a.tables.items():
        waste = len(t) * B - a.context_lens[s]
        assert 0 <= waste <= B - 1 or (a.context_lens[s] == 0 and len(t) == 0)


ops_strategy = st.lists(
    st.tuples(st.sampled_from(["add", "fork", "append", "free"]),
              st.integers(0, 7), st.integers(0, 7), st.integers(0, 40)),
    min_size=1, max_size=60)


@settings(max_examples=300, deadline=None)
@given(ops=ops_strategy, B=st.sampled_from([1, 2, 4, 16]), N=st.integers(0, 24))
def test_random_ops_keep_invariants(ops, B, N):
    a = BlockAllocatorModel(N, B)
    for kind, x, y, n in ops:
        before = (list(a.free_blocks), list(a.ref_counts), {k: list(v) for k, v in a.tables.items()},
                  dict(a.context_lens))
        try:
            if kind == "add":
                a.add_seq(x, n)
            elif kind == "fork":
                a.fork(x, y)
            elif kind == "append":
                seqs = sorted({x, y} & set(a.tables))
                if seqs:
                    a.append_slots(seqs)
            else:
                a.free_seq(x)
        except (NoFreeBlocks, InvalidOperation):
            after = (list(a.free_blocks), list(a.ref_counts), {k: list(v) for k, v in a.tables.items()},
                     dict(a.context_lens))
            assert after == before          # failed calls change nothing
        check_invariants(a)
    for s in sorted(a.tables):
        a.free_seq(s)
    assert sorted(a.free_blocks) == list(range(N))
    assert all(r == 0 for r in a.ref_counts)


def test_sixteen_appends_give_one_block_per_sequence():
    wl = workloads.llama2_13b_decode_f16(seed=3, num_seqs=128, n_steps=16)
    a = BlockAllocatorModel(wl.num_blocks, wl.block_size, wl.free_order)
    for op in wl.ops:
        if op.kind == "add_seq":
            a.add_seq(op.seq_ids[0], op.num_tokens)
    before = {s: len(t) for s, t in a.tables.items()}
    new_free = a.num_free()
    copies = []
    for op in wl.ops:
        if op.kind == "append":
            copies += a.append_slots(op.seq_ids)[1]
    assert copies == []
    assert all(len(a.tables[s]) == before[s] + 1 for s in before)
    assert new_free - a.num_free() == 128


def test_shared_prefix_copy_counts():
    """A block shared by k beams is copied k-1 times; the last writer keeps it."""
    wl = workloads.shared_prefix_beam_f16(seed=4)
    rep = runner.OracleReplay(wl)
    rep.run(skip_decode=True)
    copies = [c for r in rep.records for c in r.copies]
    assert len(copies) == 32 * 3
    srcs = Counter(src for src, _ in copies)
    assert set(srcs.values()) == {3}
    a = rep.alloc
    check_invariants(a)
    for g in range(32):
        lead = 4 * g
        shared = a.tables[lead][:2040 // 16]
        for b in range(1, 4):
            assert a.tables[lead + b][:2040 // 16] == shared
        assert all(a.ref_counts[x] == 4 for x in shared)
        partial = {a.tables[lead + b][2040 // 16] for b in range(4)}
        assert len(partial) == 4


def test_tiny_script_counts():
    """The tiny workload's append step after forking seq 2: seq 1 (16 tokens)
    takes a new block, seq 2 copies its shared partial block, seq 4 then
    writes in place."""
    wl = workloads.tiny_paged_decode_f32()
    rep = runner.OracleReplay(wl)
    rep.run(skip_decode=True)
    app = [r for r in rep.records if r.kind == "append"][0]
    assert len(app.copies) == 1
    a = rep.alloc
    assert [a.context_lens[s] for s in range(5)] == [6, 17, 18, 101, 18]
    assert len(a.tables[1]) == 2
    assert a.tables[4][1] == app.copies[0][0] and a.tables[2][1] == app.copies[0][1]
    check_invariants(a)


def test_watermark_query():
    a = BlockAllocatorModel(100, 16)
    a.set_watermark(0.05)
    assert a.can_allocate(95) and not a.can_allocate(96)
