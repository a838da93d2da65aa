"""Pins for the oracle's prefix caching (CPU only).

* a trace worked out by hand (tests/golden/apc_trace.json): hits on blocks in
  use and on blocks in the free queue, adapter isolation, lazy eviction, a
  chain broken by eviction, all-or-nothing refusals;
* invariants under random operation sequences (hypothesis): counts equal
  table occurrences, the index is a one-to-one map between keys and blocks,
  and every indexed block in a sequence's table at prompt position j carries
  exactly the key of that sequence's first j + 1 prompt blocks - no block is
  ever shared between different contents;
* the replay pin: the prefix-cache workload replayed with caching gives the
  same decode outputs, bit for bit, as the same ops replayed without it
  (every prompt row written), at fp16 and with an FP8 cache;
* closed counts on the workload: every same-adapter request after the first
  finds floor(system_len / B) blocks cached, the other adapter finds none
  at first, and the filler's evictions cut request 13's hit short.
"""

import json
import os
from collections import Counter

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads
from oracle.alloc_model import BlockAllocatorModel, InvalidOperation, NoFreeBlocks
from oracle.runner import OracleReplay

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class ApcModelSide:
    """The oracle model behind the trace's vocabulary."""

    def __init__(self, N, B, order=None):
        self.a = BlockAllocatorModel(N, B, order)
        self.a.enable_prefix_caching()

    def call(self, op, **kw):
        a = self.a
        try:
            if op == "add_seq_cached":
                return {"cached_tokens": a.add_seq_cached(kw["seq"], kw["tokens"], kw["extra"])}, None
            if op == "add_seq":
                a.add_seq(kw["seq"], kw["tokens"])
            elif op == "free_seq":
                a.free_seq(kw["seq"])
            elif op == "fork":
                a.fork(kw["parent"], kw["child"])
            elif op == "append":
                s, c = a.append_slots(kw["seqs"])
                return {"slots": list(s), "copies": [list(p) for p in c]}, None
            elif op == "prefix_hits":
                return {"hits": a.prefix_hits(kw["tokens"], kw["extra"])}, None
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
                "cached": a.cached_blocks()}


def run_apc_trace(side):
    """Replay the golden prefix-caching trace on ``side`` and check every expectation."""
    tr = json.load(open(os.path.join(GOLDEN, "apc_trace.json")))
    a = side(tr["num_blocks"], tr["block_size"])
    for i, step in enumerate(tr["steps"]):
        args = {k: v for k, v in step.items() if k not in ("op", "expect", "error")}
        res, err = a.call(step["op"], **args)
        assert err == step.get("error"), (i, step["op"], err)
        exp = step["expect"]
        if step["op"] == "block_tables":
            assert res == exp, i
            continue
        for key in ("cached_tokens", "hits", "slots", "copies"):
            if key in exp:
                assert res[key] == exp[key], (i, key, res[key], exp[key])
        st_ = a.state()
        for key in ("free", "tables", "ctx", "refs", "cached"):
            assert st_[key] == exp[key], (i, key, st_[key], exp[key])


def test_hand_worked_apc_trace():
    run_apc_trace(ApcModelSide)


def _chain_keys(a: BlockAllocatorModel, tokens, extra):
    """Keys of the prompt's full blocks, recomputed from the tokens alone."""
    B, parent, keys = a.block_size, -1, []
    for j in range(len(tokens) // B):
        parent = a._keys.get((parent, tuple(int(t) for t in tokens[j * B:(j + 1) * B]), int(extra)))
        keys.append(parent)
    return keys


def check_apc_invariants(a: BlockAllocatorModel, prompts):
    N = a.num_blocks
    occ = Counter(b for t in a.tables.values() for b in t)
    for b in range(N):
        assert a.ref_counts[b] == occ.get(b, 0)
    assert len(a.free_blocks) + sum(1 for b in range(N) if a.ref_counts[b] > 0) == N
    assert len(set(a.free_blocks)) == len(a.free_blocks)
    assert {b: k for k, b in a.cached.items()} == a.block_key     # one-to-one
    for s, (tokens, extra) in prompts.items():
        if s not in a.tables:
            continue
        for j, k in enumerate(_chain_keys(a, tokens, extra)):
            b = a.tables[s][j]
            if b in a.block_key:
                assert a.block_key[b] == k, (s, j)    # an indexed block holds this prompt's content


apc_ops = st.lists(
    st.tuples(st.sampled_from(["cached", "cached", "plain", "free", "fork", "append"]),
              st.integers(0, 6), st.integers(0, 6), st.integers(0, 3), st.integers(0, 12), st.integers(0, 1)),
    min_size=1, max_size=50)


@settings(max_examples=300, deadline=None)
@given(ops=apc_ops, B=st.sampled_from([1, 2, 4]), N=st.integers(0, 24))
def test_random_apc_ops_keep_invariants(ops, B, N):
    """Prompts are a template (one of four short token runs) plus a random
    tail, so leading blocks repeat across requests."""
    a = BlockAllocatorModel(N, B)
    a.enable_prefix_caching()
    templates = [[1, 2, 3, 4, 5, 6], [1, 2, 3, 4, 7, 7], [9, 9, 9, 9], []]
    rng = np.random.default_rng(len(ops) * 31 + B * 7 + N)
    prompts = {}
    for kind, x, y, tpl, tail, extra in ops:
        before = (list(a.free_blocks), list(a.ref_counts), {k: list(v) for k, v in a.tables.items()},
                  dict(a.cached))
        try:
            if kind == "cached":
                tokens = templates[tpl] + rng.integers(0, 3, size=tail).tolist()
                c = a.add_seq_cached(x, tokens, extra)
                prompts[x] = (tokens, extra)
                assert c % B == 0 and c <= len(tokens)
            elif kind == "plain":
                a.add_seq(x, tail)
                prompts.pop(x, None)
            elif kind == "free":
                a.free_seq(x)
                prompts.pop(x, None)
            elif kind == "fork":
                a.fork(x, y)
                if x in prompts:
                    prompts[y] = prompts[x]
                else:
                    prompts.pop(y, None)
            else:
                seqs = sorted({x, y} & set(a.tables))
                if seqs:
                    a.append_slots(seqs)
        except (NoFreeBlocks, InvalidOperation):
            after = (list(a.free_blocks), list(a.ref_counts), {k: list(v) for k, v in a.tables.items()},
                     dict(a.cached))
            assert after == before
        check_apc_invariants(a, prompts)
    for s in sorted(a.tables):
        a.free_seq(s)
    assert sorted(a.free_blocks) == list(range(N))


@pytest.mark.parametrize("kv,swap", [("", False), ("fp8", False), ("", True)])
def test_cached_replay_equals_plain_replay(kv, swap):
    """Prefix caching changes which rows are written, never what attention
    sees - also when evicted requests leave indexed blocks in the free queue
    and come back in fresh ones."""
    kw = dict(system_len=40, suffix_range=(1, 30), num_kv_heads=2, head_dim=64, block_size=8,
              num_blocks=80 if swap else 60, filler_len=150, kv_cache_dtype=kv, swap=swap)
    cached, plain = workloads.prefix_cache_requests(**kw), workloads.prefix_cache_requests(**kw)
    plain.prefix_caching = False
    plain.num_blocks = 4 * plain.num_blocks            # no sharing: room for every row
    plain.free_order = np.arange(plain.num_blocks, dtype=np.int32)
    a, b = OracleReplay(cached), OracleReplay(plain)
    ra, rb = a.run(), b.run()
    hit = sum(r.cached_tokens for r in ra if r.kind == "add_seq")
    assert hit > 0
    n_dec = 0
    for x, y in zip(ra, rb):
        if x.kind == "decode":
            assert np.array_equal(x.context_lens, y.context_lens)
            assert np.array_equal(x.out, y.out)
            n_dec += 1
    assert n_dec == 9


def test_prefix_workload_counts():
    wl = workloads.prefix_cache_requests()
    rep = OracleReplay(wl)
    cached, evicted = {}, 0
    for op in wl.ops:
        if op.kind == "decode":
            continue
        before = len(rep.alloc.cached)
        rec = rep.apply(op)
        if op.kind == "add_seq":
            cached[op.seq_ids[0]] = rec.cached_tokens
            if op.tokens is None:
                evicted = before - len(rep.alloc.cached)
    full = (300 // 16) * 16
    assert cached[0] == 0 and cached[4] == 0          # first request of each adapter
    assert all(cached[s] == full for s in (1, 2, 3, 5, 7, 8, 10, 11))
    assert cached[6] >= (316 // 16) * 16              # a continuation finds its whole earlier prompt
    assert cached[12] == (len(wl.ops[[o.seq_ids for o in wl.ops].index((12,))].tokens) // 16) * 16
    assert evicted > 0                                # the filler pushed indexed blocks out
    assert full <= cached[13] < (339 // 16) * 16      # ... and request 13 pays for it


def test_chain_needs_the_whole_prefix():
    """The same block tokens after a different earlier block, or under
    another adapter, are different content: no hit ([KVM] Part 3, the chained
    hash and its extra keys)."""
    a = BlockAllocatorModel(16, 2)
    a.enable_prefix_caching()
    assert a.add_seq_cached(0, [5, 5, 1, 2, 3]) == 0
    assert a.add_seq_cached(1, [6, 6, 1, 2, 3]) == 0          # block [1, 2] follows [6, 6] here
    assert a.tables[1][1] != a.tables[0][1]
    assert a.prefix_hits([5, 5, 1, 2], extra=1) == []
    assert a.prefix_hits([5, 5, 1, 2]) == a.tables[0][:2]
    assert a.prefix_hits([5, 5, 1, 9]) == a.tables[0][:1]
    # [9, 9] is cached after [7, 7]; after [5, 5] it is new content, so only
    # [5, 5] is reused
    assert a.add_seq_cached(2, [7, 7, 9, 9]) == 0
    assert a.add_seq_cached(3, [5, 5, 9, 9]) == 2
    assert a.tables[3][1] != a.tables[2][1]


# -- planted mistakes in the model: each must be caught by a pin above -------

def _apc_trace_fails():
    try:
        run_apc_trace(ApcModelSide)
    except AssertionError:
        return True
    return False


def test_planted_no_lazy_eviction_is_caught(monkeypatch):
    """Popping an indexed block without dropping its index entry."""
    def bad_take(self):
        phys = self.free_blocks.pop(0)
        self.ref_counts[phys] = 1
        return phys
    monkeypatch.setattr(BlockAllocatorModel, "_take", bad_take)
    assert _apc_trace_fails()


def test_planted_chain_without_parent_is_caught(monkeypatch):
    """Keys that ignore the earlier blocks (block tokens and extra key only)."""
    def bad_chain(self, tokens, extra, create):
        B = self.block_size
        keys = []
        for j in range(len(tokens) // B):
            ident = (-1, tuple(int(t) for t in tokens[j * B:(j + 1) * B]), int(extra))
            if ident not in self._keys:
                if not create:
                    keys += [None] * (len(tokens) // B - j)
                    return keys
                self._keys[ident] = len(self._keys)
            keys.append(self._keys[ident])
        return keys
    monkeypatch.setattr(BlockAllocatorModel, "_chain", bad_chain)
    with pytest.raises(AssertionError):
        test_chain_needs_the_whole_prefix()


def test_planted_ignored_extra_key_is_caught(monkeypatch):
    orig = BlockAllocatorModel._chain
    monkeypatch.setattr(BlockAllocatorModel, "_chain", lambda self, t, e, create: orig(self, t, 0, create))
    assert _apc_trace_fails()


def test_planted_hits_not_pulled_from_queue_is_caught(monkeypatch):
    """A hit on a free block that leaves it in the free queue."""
    orig_remove = list.remove
    class Q(list):
        def remove(self, x):
            pass
    orig_init = BlockAllocatorModel.__init__
    def init(self, *a, **k):
        orig_init(self, *a, **k)
        self.free_blocks = Q(self.free_blocks)
    monkeypatch.setattr(BlockAllocatorModel, "__init__", init)
    assert _apc_trace_fails()
    del orig_remove
