"""Pins for the oracle's FP8 (E4M3) quantiser (CPU only).

* the encoder against torch's float8_e4m3fn conversion (a library routine) on
  random values, every exactly representable value, every tie between
  neighbouring codes, signed zero and subnormals;
* the decoder against torch for all 256 codes;
* closed forms: a row's largest magnitude maps to the code of +-448; the
  all-zero row gives scale 0 and zero codes; the round-trip error stays within
  half a code step (relative 2^-4 in the normal range, absolute scale * 2^-10 in
  the subnormal range);
* a planted mistake (a wrong exponent bias) fails the torch pin, and the tie
  cases tell ties-to-even from ties-up.
"""

import numpy as np
import pytest
import torch

from oracle import quant


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _representable():
    v = quant.decode_e4m3(np.arange(256, dtype=np.uint8))
    return np.unique(v[~np.isnan(v)])


def _sweep():
    rng = np.random.default_rng(0)
    pos = _representable()
    pos = pos[pos >= 0]
    mids = (pos[1:] + pos[:-1]) / 2
    return np.concatenate([rng.uniform(-448, 448, 50000), rng.standard_normal(20000) * 0.01,
                           rng.standard_normal(5000) * 1e-3, pos, -pos, mids, -mids,
                           np.nextafter(mids, 0), np.nextafter(mids, 1000), [0.0, -0.0, 448.0, -448.0]]
                          ).astype(np.float32)


def test_encoder_matches_torch():
    x = _sweep()
    assert np.array_equal(quant.encode_e4m3(x), _torch_codes(x))


def test_decoder_matches_torch():
    mine = quant.decode_e4m3(np.arange(256, dtype=np.uint8))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(mine, ref, equal_nan=True)
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and np.nanmax(mine) == 448.0


def test_quantize_rows_closed_forms():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 128)) * rng.uniform(1e-3, 50, (64, 1))).astype(np.float32)
    x[3] = 0.0
    codes, scale = quant.quantize_rows(x)
    assert scale[3] == 0.0 and not codes[3].any()
    rows = [i for i in range(64) if i != 3]
    amax_at = np.argmax(np.abs(x[rows]), axis=1)
    top = codes[rows, amax_at]
    assert np.all((top == 0x7E) | (top == 0xFE))                         # +-448
    back = quant.dequantize(codes, scale)
    y = np.abs(x.astype(np.float64)) / np.where(scale > 0, scale, 1)[:, None]
    bound = np.where(y >= 2.0 ** -6, y * 2.0 ** -4, 2.0 ** -10) * scale[:, None]
    assert np.all(np.abs(back - x) <= bound + 1e-30)


def test_quantize_rows_scale_maps_the_row_maximum_to_448():
    """The scale is fixed by what it is for, not by restating its formula: a
    row's largest magnitude divided by its scale lands on 448, the largest
    E4M3 value, within one float32 rounding (relative 2^-24 for each of the
    two roundings, scale and quotient, so |amax / scale - 448| <= 448 * 2^-23),
    and no element of the row divided by the scale exceeds 448 by more than
    that. A row whose maximum is 448 * 2^k has scale exactly 2^k (the division
    is exact), so its codes are the E4M3 codes of the row divided by 2^k.
    A scale of amax / 447 or amax / 449 fails the first check."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((256, 128)) * np.exp2(rng.uniform(-20, 20, (256, 1)))).astype(np.float32)
    codes, scale = quant.quantize_rows(x)
    amax = np.max(np.abs(x.astype(np.float64)), axis=1)
    ratio = amax / scale.astype(np.float64)
    assert np.all(np.abs(ratio - 448.0) <= 448.0 * 2.0 ** -23)
    worst = np.max(np.abs(x.astype(np.float64)) / scale[:, None].astype(np.float64), axis=1)
    assert np.all(worst <= 448.0 * (1 + 2.0 ** -23))
    # rows whose maximum is 448 * 2^k: scale 2^k exactly, codes of x / 2^k
    k = rng.integers(-30, 30, size=64)
    y = np.clip(rng.standard_normal((64, 128)), -1, 1) * 448.0
    y[np.arange(64), rng.integers(0, 128, size=64)] = 448.0 * np.where(rng.random(64) < 0.5, 1.0, -1.0)
    y = np.trunc(y).astype(np.float32)                     # whole numbers below 448: exactly scalable
    xs = (y * np.exp2(k)[:, None]).astype(np.float32)
    c2, s2 = quant.quantize_rows(xs)
    assert np.array_equal(s2, np.exp2(k).astype(np.float32))
    assert np.array_equal(c2, quant.encode_e4m3(y))


def test_quantize_rows_scale_pin_catches_planted_divisors(monkeypatch):
    """The pin above fails for the plausible mistake in the scale: the
    divisor off by one either way."""
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((256, 128)) * np.exp2(rng.uniform(-20, 20, (256, 1)))).astype(np.float32)
    amax = np.max(np.abs(x.astype(np.float64)), axis=1)
    for wrong in (np.float32(447.0), np.float32(449.0)):
        monkeypatch.setattr(quant, "E4M3_MAX", float(wrong))
        _, scale = quant.quantize_rows(np.clip(x, -1e30, 1e30))
        assert not np.all(np.abs(amax / scale.astype(np.float64) - 448.0) <= 448.0 * 2.0 ** -23)


def test_planted_bias_mistake_fails_the_pin(monkeypatch):
    x = np.clip(_sweep(), -224, 224)
    monkeypatch.setattr(quant, "_BIAS", 8)
    assert not np.array_equal(quant.encode_e4m3(x), _torch_codes(x))


def test_ties_pin_discriminates_the_rounding_rule():
    """At every tie between neighbouring codes the encoder (and torch) pick
    the even mantissa; rounding ties up would give the upper neighbour, which
    differs at half of them."""
    pos = _representable()
    pos = pos[pos > 0]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    even = quant.encode_e4m3(mids)
    upper = quant.encode_e4m3(np.nextafter(mids, np.float32(1000)))
    assert np.array_equal(even, _torch_codes(mids))
    assert not np.array_equal(even, upper)
    assert np.all(even % 2 == 0)


def test_paged_fp8_replay_equals_quantised_logical_sdpa():
    """The oracle's FP8 paged decode (quantise at append, gather codes and
    scales through the block tables, dequantise) equals torch SDPA over the
    logical rows quantised directly - an independent route with no blocks."""
    import workloads
    from oracle.runner import OracleReplay
    from tests.logical import logical_decodes, sdpa_reference
    wl = workloads.custom_decode(seed=3, dtype="f16", ctx=[1, 17, 100, 300], num_q_heads=4, num_kv_heads=2,
                                 head_dim=64, block_size=16, n_steps=2, kv_cache_dtype="fp8")
    recs = [r for r in OracleReplay(wl).run() if r.kind == "decode"]
    for rec, (seqs, q, rows) in zip(recs, logical_decodes(wl)):
        for i, s in enumerate(seqs):
            K, V = rows[s]
            kc, ks = quant.quantize_rows(K.float().numpy())
            vc, vs = quant.quantize_rows(V.float().numpy())
            ref = sdpa_reference(q[i], torch.from_numpy(quant.dequantize(kc, ks)),
                                 torch.from_numpy(quant.dequantize(vc, vs)), wl.scale).numpy()
            assert np.max(np.abs(rec.out[i] - ref)) <= 1e-12


# ---------------------------------------------------------------------------
# INT8
# ---------------------------------------------------------------------------
def _torch_int8(x, scale):
    """torch's per-channel symmetric int8 quantisation of the rows of x."""
    xt = torch.from_numpy(np.asarray(x, np.float32))
    st = torch.from_numpy(np.where(scale > 0, scale, 1).astype(np.float64))
    q = torch.quantize_per_channel(xt, st, torch.zeros(len(st), dtype=torch.int64), 0, torch.qint8)
    return q.int_repr().numpy()


def test_int8_codes_match_torch():
    """A library routine: torch.quantize_per_channel (zero point 0) with the
    oracle's scales gives the oracle's codes on random rows of every
    magnitude, rows with a zero, and rows holding exact ties."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((512, 128)) * np.exp2(rng.uniform(-20, 20, (512, 1)))).astype(np.float32)
    codes, scale = quant.quantize_rows_int8(x)
    assert codes.dtype == np.int8 and scale.dtype == np.float32
    assert np.array_equal(codes, _torch_int8(x, scale))


def test_int8_closed_forms():
    """The row's largest magnitude gives code +-127 and amax / scale lands on
    127 within one rounding; a zero row gives scale 0 and zero codes; every
    code is in [-127, 127]; the round trip is within half a step (scale / 2,
    plus the division's one rounding); ties go to the even integer."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, 128)) * rng.uniform(1e-3, 50, (64, 1))).astype(np.float32)
    x[5] = 0.0
    codes, scale = quant.quantize_rows_int8(x)
    assert scale[5] == 0.0 and not codes[5].any()
    rows = [i for i in range(64) if i != 5]
    top = codes[rows, np.argmax(np.abs(x[rows]), axis=1)]
    assert np.all(np.abs(top.astype(int)) == 127)
    amax = np.max(np.abs(x[rows].astype(np.float64)), axis=1)
    assert np.all(np.abs(amax / scale[rows] - 127.0) <= 127.0 * 2.0 ** -23)
    assert codes.min() >= -127 and codes.max() <= 127
    back = quant.dequantize_int8(codes, scale)
    assert np.all(np.abs(back - x) <= scale[:, None].astype(np.float64) * (0.5 + 2.0 ** -20) + 1e-30)
    # exact ties: x / scale = k + 0.5 exactly (scale a power of two)
    t = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5]], dtype=np.float32)
    c, s = quant.quantize_rows_int8(t)
    assert s[0] == 1.0 and c[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 126]


def test_int8_pins_catch_planted_mistakes(monkeypatch):
    """Plausible mistakes fail the pins: a divisor of 128 breaks the
    row-maximum pin, truncation instead of rounding breaks the torch pin."""
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((256, 128)) * 3).astype(np.float32)
    monkeypatch.setattr(quant, "INT8_MAX", 128.0)
    codes, scale = quant.quantize_rows_int8(x)
    amax = np.max(np.abs(x.astype(np.float64)), axis=1)
    assert not np.all(np.abs(amax / scale - 127.0) <= 127.0 * 2.0 ** -23)
    monkeypatch.setattr(quant, "INT8_MAX", 127.0)
    monkeypatch.setattr(quant.np, "rint", np.trunc)
    codes, scale = quant.quantize_rows_int8(x)
    monkeypatch.undo()
    assert not np.array_equal(codes, _torch_int8(x, scale))


def test_paged_int8_replay_equals_quantised_logical_sdpa():
    """The oracle's INT8 paged decode (quantise at append, gather codes and
    scales through the block tables, dequantise) equals torch SDPA over the
    logical rows quantised directly - an independent route with no blocks."""
    import workloads
    from oracle.runner import OracleReplay
    from tests.logical import logical_decodes, sdpa_reference
    wl = workloads.custom_decode(seed=4, dtype="bf16", ctx=[1, 17, 100, 300], num_q_heads=8, num_kv_heads=2,
                                 head_dim=128, block_size=8, n_steps=2, kv_cache_dtype="int8")
    recs = [r for r in OracleReplay(wl).run() if r.kind == "decode"]
    for rec, (seqs, q, rows) in zip(recs, logical_decodes(wl)):
        for i, s in enumerate(seqs):
            K, V = rows[s]
            kc, ks = quant.quantize_rows_int8(K.float().numpy())
            vc, vs = quant.quantize_rows_int8(V.float().numpy())
            ref = sdpa_reference(q[i], torch.from_numpy(quant.dequantize_int8(kc, ks)),
                                 torch.from_numpy(quant.dequantize_int8(vc, vs)), wl.scale).numpy()
            assert np.max(np.abs(rec.out[i] - ref)) <= 1e-12
