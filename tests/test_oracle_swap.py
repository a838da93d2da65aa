"""Pins for the oracle's swap space (eviction to CPU memory and back), CPU only.

* a trace worked out by hand (tests/golden/swap_trace.json);
* invariants under random operation sequences with swaps (hypothesis): every
  GPU block is free or referenced by resident tables only, every swap block is
  free or in exactly one swapped-out table, failed calls change nothing, and
  swapping a sequence out and back in keeps its context length and gives it a
  table of the same length;
* the whole-block copy between pools against brute force;
* the preemption workload needs its evictions: at the default sizes the new
  sequences do not fit in the GPU pool before the first swap-out;
* an oracle replay with its evictions taken out gives the same attention
  output after the swap-in, bit for bit.
"""

import json
import os
from collections import Counter

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads
from oracle import cache_ops
from oracle.alloc_model import BlockAllocatorModel, InvalidOperation, NoFreeBlocks
from oracle.runner import OracleReplay

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class _ModelSide:
    """The oracle model behind the trace's vocabulary."""

    def __init__(self, N, B, S, order=None, swap_order=None):
        self.a = BlockAllocatorModel(N, B, order)
        self.a.set_swap_space(S, swap_order)

    def call(self, op, **kw):
        a = self.a
        try:
            if op == "add_seq":
                a.add_seq(kw["seq"], kw["tokens"])
            elif op == "fork":
                a.fork(kw["parent"], kw["child"])
            elif op == "append":
                s, c = a.append_slots(kw["seqs"])
                return {"slots": list(s), "copies": [list(p) for p in c]}, None
            elif op == "free_seq":
                a.free_seq(kw["seq"])
            elif op == "swap_out":
                return {"pairs": [list(p) for p in a.swap_out(kw["seq"])]}, None
            elif op == "swap_in":
                return {"pairs": [list(p) for p in a.swap_in(kw["seq"])]}, None
            elif op == "block_tables":
                t, c = a.block_tables(kw["seqs"], kw["max_blocks"])
                return {"tables": t.tolist(), "ctx": c.tolist()}, None
            return {}, None
        except NoFreeBlocks:
            return {}, "no_blocks"
        except InvalidOperation:
            return {}, "invalid"

    def state(self):
        a = self.a
        return {"free": list(a.free_blocks), "tables": {str(k): list(v) for k, v in a.tables.items()},
                "ctx": {str(k): v for k, v in a.context_lens.items()}, "refs": list(a.ref_counts),
                "swap_free": list(a.swap_free), "swapped": sorted(a.swapped)}


def _trace_args(step):
    return {k: v for k, v in step.items() if k not in ("op", "expect", "error")}


def run_swap_trace(side):
    """Replay the golden swap trace on ``side`` and check every expectation."""
    tr = json.load(open(os.path.join(GOLDEN, "swap_trace.json")))
    a = side(tr["num_blocks"], tr["block_size"], tr["num_swap_blocks"])
    for i, step in enumerate(tr["steps"]):
        res, err = a.call(step["op"], **_trace_args(step))
        assert err == step.get("error"), (i, step["op"], err)
        exp = step["expect"]
        if step["op"] == "block_tables":
            assert res == exp, i
            continue
        for key in ("slots", "copies", "pairs"):
            if key in exp:
                assert res[key] == exp[key], (i, key, res[key], exp[key])
        st_ = a.state()
        for key in ("free", "tables", "ctx", "refs", "swap_free", "swapped"):
            assert st_[key] == exp[key], (i, key, st_[key], exp[key])


def test_hand_worked_swap_trace():
    run_swap_trace(_ModelSide)


def check_swap_invariants(a: BlockAllocatorModel, S: int):
    N = a.num_blocks
    resident = {s: t for s, t in a.tables.items() if s not in a.swapped}
    occ = Counter(b for t in resident.values() for b in t)
    for b in range(N):
        assert a.ref_counts[b] == occ.get(b, 0)
    assert len(set(a.free_blocks)) == len(a.free_blocks)
    assert len(a.free_blocks) + sum(1 for b in range(N) if a.ref_counts[b] > 0) == N
    held = [b for s in a.swapped for b in a.tables[s]]
    assert len(set(held)) == len(held)            # a swap block belongs to one sequence
    assert not set(held) & set(a.swap_free)
    assert sorted(held + a.swap_free) == list(range(S))


ops_strategy = st.lists(
    st.tuples(st.sampled_from(["add", "fork", "append", "free", "out", "in"]),
              st.integers(0, 5), st.integers(0, 5), st.integers(0, 30)),
    min_size=1, max_size=60)


def _snapshot(a):
    return (list(a.free_blocks), list(a.ref_counts), {k: list(v) for k, v in a.tables.items()},
            dict(a.context_lens), list(a.swap_free), set(a.swapped))


@settings(max_examples=300, deadline=None)
@given(ops=ops_strategy, B=st.sampled_from([1, 2, 4, 16]), N=st.integers(0, 20), S=st.integers(0, 20))
def test_random_swaps_keep_invariants(ops, B, N, S):
    a = BlockAllocatorModel(N, B)
    a.set_swap_space(S)
    for kind, x, y, n in ops:
        before = _snapshot(a)
        try:
            if kind == "add":
                a.add_seq(x, n)
            elif kind == "fork":
                a.fork(x, y)
            elif kind == "append":
                seqs = sorted(({x, y} & set(a.tables)) - a.swapped)
                if seqs:
                    a.append_slots(seqs)
            elif kind == "free":
                a.free_seq(x)
            elif kind == "out":
                ctx, length = a.context_lens.get(x), len(a.tables.get(x, []))
                pairs = a.swap_out(x)
                assert [p[0] for p in pairs] == before[2][x]       # every GPU block, in logical order
                assert a.context_lens[x] == ctx and len(a.tables[x]) == length
            else:
                ctx, length = a.context_lens.get(x), len(a.tables.get(x, []))
                pairs = a.swap_in(x)
                assert [p[0] for p in pairs] == before[2][x]
                assert a.context_lens[x] == ctx and len(a.tables[x]) == length
                assert all(a.ref_counts[b] == 1 for b in a.tables[x])
        except (NoFreeBlocks, InvalidOperation):
            assert _snapshot(a) == before            # failed calls change nothing
        check_swap_invariants(a, S)
    for s in sorted(a.tables):
        a.free_seq(s)
    assert sorted(a.free_blocks) == list(range(N)) and sorted(a.swap_free) == list(range(S))


def test_oracle_swap_blocks_brute_force():
    """Whole blocks between two pools: each destination block equals its
    source block, every other destination block is untouched, and a round trip
    through a second pool restores the original."""
    rng = np.random.default_rng(0)
    src_k = rng.integers(0, 2**16, size=(5, 2, 4, 8), dtype=np.uint16)
    src_v = rng.integers(0, 2**16, size=(5, 2, 4, 8), dtype=np.uint16)
    dst_k = np.zeros((7, 2, 4, 8), np.uint16)
    dst_v = np.zeros((7, 2, 4, 8), np.uint16)
    pairs = [(4, 0), (0, 6), (2, 3)]
    cache_ops.swap_blocks(src_k, src_v, dst_k, dst_v, pairs)
    for s, d in pairs:
        for h in range(2):
            for t in range(4):
                for e in range(8):
                    assert dst_k[d, h, t, e] == src_k[s, h, t, e] and dst_v[d, h, t, e] == src_v[s, h, t, e]
    for d in set(range(7)) - {0, 6, 3}:
        assert not dst_k[d].any() and not dst_v[d].any()
    back_k, back_v = np.zeros_like(src_k), np.zeros_like(src_v)
    cache_ops.swap_blocks(dst_k, dst_v, back_k, back_v, [(d, s) for s, d in pairs])
    for s, _ in pairs:
        assert np.array_equal(back_k[s], src_k[s]) and np.array_equal(back_v[s], src_v[s])


def test_preempt_workload_needs_its_evictions():
    """Replaying the allocator side: the pool is short before the first
    swap-out (the two new sequences would not fit), every op then succeeds,
    and the swap space ends empty-handed (all its blocks free)."""
    wl = workloads.preempt_swap()
    rep = OracleReplay(wl)
    new_blocks = None
    for i, op in enumerate(wl.ops):
        if op.kind == "swap_out" and new_blocks is None:
            adds = [o for o in wl.ops[i:] if o.kind == "add_seq"][:2]
            new_blocks = sum(-(-o.num_tokens // wl.block_size) for o in adds)
            assert new_blocks > rep.alloc.num_free()
        if op.kind != "decode":
            rep.apply(op)
    assert sorted(rep.alloc.swap_free) == list(range(wl.num_swap_blocks))


@pytest.mark.parametrize("kv", ["", "fp8"])
def test_preempt_replay_keeps_values(kv):
    """Oracle replay of a small preemption workload: after a sequence's round
    trip through the swap space, its gathered K/V values equal those of the
    same workload with the evictions taken out (the first decode after the
    swap-in is compared)."""
    wl = workloads.preempt_swap(seed=9, num_seqs=5, ctx_range=(5, 120), num_kv_heads=2, head_dim=64,
                                block_size=8, n_steps=1, kv_cache_dtype=kv)
    plain = workloads.preempt_swap(seed=9, num_seqs=5, ctx_range=(5, 120), num_kv_heads=2, head_dim=64,
                                   block_size=8, n_steps=1, kv_cache_dtype=kv)
    plain.ops = [o for o in plain.ops if o.kind not in ("swap_out", "swap_in")]
    plain.num_blocks *= 2
    plain.free_order = np.arange(plain.num_blocks, dtype=np.int32)
    a, b = OracleReplay(wl), OracleReplay(plain)
    idx_in = next(i for i, o in enumerate(wl.ops) if o.kind == "swap_in")
    k = sum(1 for o in wl.ops[:idx_in] if o.kind == "decode")    # decodes before the swap-in
    def run_to_decode(rep, ops):
        seen = 0
        for op in ops:
            if op.kind == "decode":
                if seen == k:
                    return op
                seen += 1
            rep.apply(op)
    first_dec = run_to_decode(a, wl.ops)
    plain_dec = run_to_decode(b, plain.ops)
    assert first_dec.seq_ids == plain_dec.seq_ids
    ra, rb = a.decode(first_dec.seq_ids, first_dec.q), b.decode(first_dec.seq_ids, first_dec.q)
    assert np.array_equal(ra.context_lens, rb.context_lens)
    assert np.array_equal(ra.out, rb.out)


# -- planted mistakes in the model: each must be caught by a pin above -------

def _trace_fails():
    try:
        run_swap_trace(_ModelSide)
    except AssertionError:
        return True
    return False


def test_planted_swap_out_keeps_gpu_blocks_is_caught(monkeypatch):
    """A swap-out that forgets to release the GPU blocks."""
    def bad(self, seq_id):
        if seq_id not in self.tables or seq_id in self.swapped:
            raise InvalidOperation("swap_out")
        table = self.tables[seq_id]
        if len(table) > len(self.swap_free):
            raise NoFreeBlocks("swap")
        host = [self.swap_free.pop(0) for _ in table]
        pairs = list(zip(table, host))
        self.tables[seq_id] = host
        self.swapped.add(seq_id)
        return pairs
    monkeypatch.setattr(BlockAllocatorModel, "swap_out", bad)
    assert _trace_fails()


def test_planted_swap_in_lifo_swap_pool_is_caught(monkeypatch):
    """Swap blocks returned to the head instead of the tail."""
    orig = BlockAllocatorModel.swap_in
    def bad(self, seq_id):
        host = list(self.tables.get(seq_id, []))
        pairs = orig(self, seq_id)
        for b in host:
            self.swap_free.remove(b)
        self.swap_free[:0] = host
        return pairs
    monkeypatch.setattr(BlockAllocatorModel, "swap_in", bad)
    assert _trace_fails()


def test_planted_free_of_swapped_sequence_is_caught(monkeypatch):
    """Freeing a swapped-out sequence releases GPU ids instead of swap ids."""
    orig = BlockAllocatorModel.free_seq
    def bad(self, seq_id):
        self.swapped.discard(seq_id)
        return orig(self, seq_id)
    monkeypatch.setattr(BlockAllocatorModel, "free_seq", bad)
    assert _trace_fails()
