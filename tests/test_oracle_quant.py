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
    np.testing.assert_array_equal(scale, (np.max(np.abs(x), axis=1) / np.float32(448)).astype(np.float32))
    back = quant.dequantize(codes, scale)
    y = np.abs(x.astype(np.float64)) / np.where(scale > 0, scale, 1)[:, None]
    bound = np.where(y >= 2.0 ** -6, y * 2.0 ** -4, 2.0 ** -10) * scale[:, None]
    assert np.all(np.abs(back - x) <= bound + 1e-30)


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
