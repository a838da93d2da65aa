"""Pins for the oracle's derived error bound (CPU only).

* a faithful float32 evaluation of the split softmax (partial outputs and the
  result rounded to the output type) stays inside the bound, for float32,
  float16 and bfloat16, one range and many, grouped query heads, and contexts
  of one token up to the long-context shape;
* for float16 and bfloat16 the bound is tighter than the fixed tolerance the
  workloads state (for float32 the two are of the same size, and the tests
  apply both);
* at the long-context shape (one sequence of about 24.6 K tokens, 512-token
  ranges, four query heads on one KV head, head_dim 128, bfloat16), the
  oracle's split decode with any one range left out of the merge, or with
  one range's weight doubled or halved, breaks the bound while staying within
  2e-2 + 1e-2 |y| - the fixed tolerance cannot see such a mistake, the bound
  can.
"""

import numpy as np
import pytest
import torch

from oracle import attention, error_bound

TOL = {"f32": (1e-4, 0.0), "f16": (2e-2, 1e-2), "bf16": (2e-2, 1e-2)}
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _round(x: np.ndarray, dt: str) -> np.ndarray:
    """Round to the type (round to nearest even) and back to float64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(TORCH[dt]).double().numpy()


def _data(rng, ctx, Hq, Hkv, d, dt, amp=1.0):
    q = _round(rng.standard_normal((Hq, d)) * amp, dt)
    K = _round(rng.standard_normal((ctx, Hkv, d)) * amp, dt)
    V = _round(rng.standard_normal((ctx, Hkv, d)) * amp, dt)
    return q, K, V


def _emulate_fp32(q_h, K, V, scale, ranges, dt):
    """The split softmax evaluated in float32, with the partial outputs (more
    than one range) and the result rounded to ``dt``."""
    q32 = q_h.astype(np.float32)
    states = []
    for t0, n in ranges:
        s = (K[t0:t0 + n].astype(np.float32) @ q32) * np.float32(scale)
        m = s.max()
        e = np.exp(s - m, dtype=np.float32)
        l = e.sum(dtype=np.float32)
        o = (e @ V[t0:t0 + n].astype(np.float32)) / l
        if len(ranges) > 1:
            o = _round(o, dt).astype(np.float32)
        states.append((m, l, o))
    m = max(st[0] for st in states)
    W = [np.float32(st[1] * np.exp(np.float32(st[0] - m), dtype=np.float32)) for st in states]
    num = np.zeros_like(states[0][2])
    for w, st in zip(W, states):
        num = num + w * st[2]
    return _round(num / np.float32(sum(W, np.float32(0))), dt)


CASES = [
    # dt, ctx, Hq, Hkv, d, partition
    ("f32", 5, 8, 8, 64, 512), ("f32", 100, 8, 8, 64, 16), ("f32", 2100, 4, 2, 128, 512),
    ("f16", 1, 4, 4, 128, 512), ("f16", 17, 4, 4, 128, 512), ("f16", 700, 4, 4, 128, 128),
    ("f16", 4097, 2, 2, 128, 1024),
    ("bf16", 3, 8, 2, 128, 512), ("bf16", 1500, 8, 2, 128, 512), ("bf16", 9000, 4, 1, 128, 512),
]


@pytest.mark.parametrize("dt,ctx,Hq,Hkv,d,part", CASES)
def test_faithful_fp32_evaluation_stays_inside_the_bound(dt, ctx, Hq, Hkv, d, part):
    rng = np.random.default_rng(ctx * 7 + Hq)
    q, K, V = _data(rng, ctx, Hq, Hkv, d, dt)
    scale = 1.0 / np.sqrt(d)
    ranges = error_bound.dense_partitions(ctx, part)
    bound = error_bound.decode_error_bound(q, K, V, scale, [ranges], dt)
    y = attention.dense_decode_one(q, K, V, scale)
    atol, rtol = TOL[dt]
    if dt != "f32":   # float32 caches: worst-case float32 score sums can exceed 1e-4 on short contexts
        assert np.all(bound < atol + rtol * np.abs(y)), "the bound must be tighter than the fixed tolerance"
    g = Hq // Hkv
    for h in range(Hq):
        got = _emulate_fp32(q[h], K[:, h // g], V[:, h // g], scale, ranges, dt)
        assert np.all(np.abs(got - y[h]) <= bound[h]), (h, float(np.max(np.abs(got - y[h]) / bound[h])))


def test_single_token_bound_is_one_rounding():
    """One token: the exact output is V_0; with a value that the type holds
    exactly the only error left is float32 noise, and the bound is a few
    units in the last place of the output type."""
    rng = np.random.default_rng(3)
    q, K, V = _data(rng, 1, 2, 2, 128, "f16")
    b = error_bound.decode_error_bound(q, K, V, 1 / np.sqrt(128), [[(0, 1)]], "f16")
    y = V[0]
    assert np.all(b <= 4 * 2.0 ** -11 * np.abs(y) + 1e-5)


def _long_context(seed=5):
    rng = np.random.default_rng(seed)
    ctx = 24577                                 # 48 full 512-token ranges and a 1-token tail
    q, K, V = _data(rng, ctx, 4, 1, 128, "bf16")
    return q, K[:, 0], V[:, 0], 1.0 / np.sqrt(128)


def test_long_context_bound_catches_one_bad_range_the_fixed_tolerance_does_not():
    q, K, V, scale = _long_context()
    ctx = K.shape[0]
    ranges = error_bound.dense_partitions(ctx, 512)
    atol, rtol = TOL["bf16"]
    for h in range(q.shape[0]):
        y = attention.dense_decode_one(q[h:h + 1], K[:, None], V[:, None], scale)[0]
        bound = error_bound.decode_error_bound_one(q[h], K, V, scale, ranges, "bf16")
        # the faithful evaluation passes
        good = _emulate_fp32(q[h], K, V, scale, ranges, "bf16")
        assert np.all(np.abs(good - y) <= bound)
        states = [attention.partition_state(q[h], K[t0:t0 + n], V[t0:t0 + n], scale) for t0, n in ranges]
        full = attention.merge_partitions(states)
        assert np.max(np.abs(full - y)) < 1e-12
        caught = {"dropped": 0, "doubled": 0, "halved": 0}
        for p in range(len(ranges) - 1):        # every full range (the 1-token tail weighs ~1/24577)
            variants = {
                "dropped": states[:p] + states[p + 1:],
                "doubled": states[:p] + [(states[p][0], 2 * states[p][1], states[p][2])] + states[p + 1:],
                "halved": states[:p] + [(states[p][0], 0.5 * states[p][1], states[p][2])] + states[p + 1:],
            }
            for name, st in variants.items():
                bad = _round(attention.merge_partitions(st), "bf16")
                err = np.abs(bad - y)
                assert np.all(err <= atol + rtol * np.abs(y)), "the fixed tolerance passes the mistake"
                caught[name] += bool(np.any(err > bound))
        n = len(ranges) - 1
        assert caught == {"dropped": n, "doubled": n, "halved": n}, (h, caught)


def test_split_partitions_tile_the_context():
    for ctx, size, first in [(2041, 512, 2032), (100, 16, 48), (5, 512, 0), (600, 128, 600)]:
        r = error_bound.split_partitions(ctx, size, first)
        covered = [t for t0, n in r for t in range(t0, t0 + n)]
        assert covered == list(range(ctx)) and all(0 < n <= size for _, n in r)
