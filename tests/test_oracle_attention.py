"""Pins for the oracle's attention (CPU only).

Each check ties the oracle to something other than itself:
  * a library routine: torch scaled_dot_product_attention in fp64 over the
    logical (unpaged) K/V rows of each sequence;
  * brute force with Python loops and math.fsum on the tiny workload;
  * closed-form special cases;
  * invariance under a different physical block permutation;
  * the five-step blockwise softmax and the partition merge against a plain
    global softmax;
  * planted mistakes in the oracle that these pins must catch.
"""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, runner
from tests.logical import logical_decodes, sdpa_reference

pytestmark = pytest.mark.timeout(300)


def _replay(wl):
    rep = runner.OracleReplay(wl)
    recs = rep.run()
    return rep, [r for r in recs if r.kind == "decode"]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_paged_equals_contiguous_sdpa(n):
    """Paged oracle output == torch SDPA (fp64) over the logical K/V, for every
    decode of the scaled-down workloads (config 1 at full size)."""
    wl = workloads.scaled_down(n)
    _, decs = _replay(wl)
    logical = logical_decodes(wl)
    assert len(decs) == len(logical)
    for rec, (seqs, q, rows) in zip(decs, logical):
        for i, s in enumerate(seqs):
            K, V = rows[s]
            ref = sdpa_reference(q[i], K, V, wl.scale).numpy()
            assert np.max(np.abs(rec.out[i] - ref)) <= 1e-12, (n, s)


def _brute_force_one(q, K, V, scale, group):
    Hq, d = len(q), len(q[0])
    out = []
    for h in range(Hq):
        kv = h // group
        scores = [scale * math.fsum(q[h][c] * K[t][kv][c] for c in range(d)) for t in range(len(K))]
        m = max(scores)
        e = [math.exp(x - m) for x in scores]
        z = math.fsum(e)
        out.append([math.fsum(e[t] * V[t][kv][c] for t in range(len(K))) / z for c in range(d)])
    return out


def test_brute_force_tiny():
    wl = workloads.tiny_paged_decode_f32()
    _, decs = _replay(wl)
    for rec, (seqs, q, rows) in zip(decs, logical_decodes(wl)):
        for i, s in enumerate(seqs):
            K, V = rows[s]
            bf = _brute_force_one(q[i].double().tolist(), K.double().tolist(), V.double().tolist(), wl.scale, 1)
            assert np.max(np.abs(rec.out[i] - np.array(bf))) <= 1e-12


def _one_seq_pool(K, V, B, perm_seed):
    """Scatter contiguous K/V [ctx, H, d] into a shuffled pool by hand."""
    ctx, H, d = K.shape
    nb = -(-ctx // B)
    rng = np.random.default_rng(perm_seed)
    N = nb + 3
    phys = rng.permutation(N)[:nb]
    kc = np.full((N, H, B, d), np.nan)
    vc = np.full((N, H, B, d), np.nan)
    for t in range(ctx):
        kc[phys[t // B], :, t % B, :] = K[t]
        vc[phys[t // B], :, t % B, :] = V[t]
    return kc, vc, phys


@pytest.mark.parametrize("ctx", [1, 7, 16, 33])
def test_special_cases(ctx):
    rng = np.random.default_rng(ctx)
    H, d, B = 4, 16, 8
    K = rng.standard_normal((ctx, H, d))
    V = rng.standard_normal((ctx, H, d))
    q = rng.standard_normal((1, H, d))
    kc, vc, phys = _one_seq_pool(K, V, B, 7)
    # q = 0 -> uniform weights -> mean of the V rows
    out = attention.paged_decode(np.zeros((1, H, d)), kc, vc, [phys], [ctx], 0.25)
    np.testing.assert_allclose(out[0], V.mean(axis=0), rtol=0, atol=1e-13)
    # all K rows equal -> mean of V
    kc2, _, _ = _one_seq_pool(np.broadcast_to(K[:1], K.shape).copy(), V, B, 7)
    out = attention.paged_decode(q, kc2, vc, [phys], [ctx], 0.25)
    np.testing.assert_allclose(out[0], V.mean(axis=0), rtol=0, atol=1e-13)
    # V constant -> that constant
    _, vc3, _ = _one_seq_pool(K, np.full(V.shape, 2.5), B, 7)
    out = attention.paged_decode(q, kc, vc3, [phys], [ctx], 0.25)
    np.testing.assert_allclose(out[0], 2.5, rtol=0, atol=1e-13)
    if ctx == 1:
        out = attention.paged_decode(q, kc, vc, [phys], [1], 0.25)
        assert np.array_equal(out[0], V[0])


def test_context_zero_gives_zero():
    kc = np.ones((2, 1, 4, 3))
    out = attention.paged_decode(np.ones((1, 1, 3)), kc, kc, [[-1]], [0], 1.0)
    assert np.array_equal(out, np.zeros((1, 1, 3)))


def test_permutation_invariance_bitwise():
    """Two different physical permutations of the same logical data give the
    same oracle output bit for bit (the gather is identical)."""
    rng = np.random.default_rng(0)
    ctx, H, d, B = 45, 2, 8, 16
    K = rng.standard_normal((ctx, H, d))
    V = rng.standard_normal((ctx, H, d))
    q = rng.standard_normal((1, H, d))
    a = attention.paged_decode(q, *_one_seq_pool(K, V, B, 1)[:2], [_one_seq_pool(K, V, B, 1)[2]], [ctx], 0.3)
    b = attention.paged_decode(q, *_one_seq_pool(K, V, B, 2)[:2], [_one_seq_pool(K, V, B, 2)[2]], [ctx], 0.3)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("B", [8, 16, 32])
@pytest.mark.parametrize("n", [1, 15, 16, 17, 100, 513])
def test_blockwise_softmax_equals_global(B, n):
    s = np.random.default_rng(n * B).standard_normal(n) * 4
    ref = torch.softmax(torch.from_numpy(s), dim=0).numpy()
    assert np.max(np.abs(attention.blockwise_softmax(s, B) - ref)) <= 1e-12


@pytest.mark.parametrize("ctx", [1, 511, 512, 513, 1500, 2049])
def test_partition_merge_equals_dense(ctx):
    rng = np.random.default_rng(ctx)
    Hq, Hkv, d = 4, 2, 8
    K = rng.standard_normal((ctx, Hkv, d)) * 2
    V = rng.standard_normal((ctx, Hkv, d))
    q = rng.standard_normal((Hq, d)) * 2
    ref = sdpa_reference(torch.from_numpy(q), torch.from_numpy(K), torch.from_numpy(V), 0.5).numpy()
    got = attention.partitioned_decode_one(q, K, V, 0.5, 512)
    assert np.max(np.abs(got - ref)) <= 1e-12


# -- planted mistakes: each must be caught by one of the pins above ------------

def _sdpa_check(wl):
    _, decs = _replay(wl)
    worst = 0.0
    for rec, (seqs, q, rows) in zip(decs, logical_decodes(wl)):
        for i, s in enumerate(seqs):
            K, V = rows[s]
            worst = max(worst, float(np.max(np.abs(rec.out[i] - sdpa_reference(q[i], K, V, wl.scale).numpy()))))
    return worst


def test_planted_transposed_block_layout_is_caught(monkeypatch):
    def bad_gather(cache, block_table, context_len):
        _, H, B, d = cache.shape
        nb = -(-context_len // B)
        rows = np.concatenate([cache[int(block_table[j])].reshape(B, H, d) for j in range(nb)])
        return rows[:context_len]
    monkeypatch.setattr(attention, "gather_sequence", bad_gather)
    assert _sdpa_check(workloads.tiny_paged_decode_f32()) > 1e-3


def test_planted_wrong_gqa_mapping_is_caught(monkeypatch):
    orig = attention.dense_decode_one

    def bad(q, K, V, scale):
        Hq = q.shape[0]
        Hkv = K.shape[1]
        if Hq == Hkv:
            return orig(q, K, V, scale)
        out = np.zeros_like(q)
        for h in range(Hq):
            out[h] = orig(q[h:h + 1], K[:, h % Hkv:h % Hkv + 1], V[:, h % Hkv:h % Hkv + 1], scale)[0]
        return out
    monkeypatch.setattr(attention, "dense_decode_one", bad)
    assert _sdpa_check(workloads.scaled_down(5)) > 1e-3


def test_planted_dropped_scale_is_caught(monkeypatch):
    orig = attention.dense_decode_one
    monkeypatch.setattr(attention, "dense_decode_one", lambda q, K, V, scale: orig(q, K, V, 1.0))
    assert _sdpa_check(workloads.tiny_paged_decode_f32()) > 1e-3


def test_planted_off_by_one_block_is_caught(monkeypatch):
    orig = attention.gather_sequence

    def bad(cache, block_table, context_len):
        B = cache.shape[2]
        return orig(cache, block_table, -(-context_len // B) * B)[1:context_len + 1] \
            if -(-context_len // B) * B > context_len else orig(cache, block_table, context_len)
    monkeypatch.setattr(attention, "gather_sequence", bad)
    assert _sdpa_check(workloads.tiny_paged_decode_f32()) > 1e-3


def test_planted_blockwise_step_mistake_is_caught():
    s = np.random.default_rng(3).standard_normal(40) * 4
    ref = torch.softmax(torch.from_numpy(s), dim=0).numpy()
    # using the last block's local max instead of the global one (steps 2-3)
    starts = range(0, 40, 16)
    e = np.exp(s - s[32:].max())
    wrong = e / sum(np.exp(s[i:i + 16] - s[i:i + 16].max()).sum() for i in starts)
    assert np.max(np.abs(wrong - ref)) > 1e-3
