"""Pins for the oracle's closed forms (against the figures the pages print)
and for its bitwise cache operations (against hand-built expectations)."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import cache_ops, sizes

FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_block_elements_printed():
    f = FIG["block_elements"]
    n = sizes.block_elements(f["block_size"], f["num_heads"], f["head_dim"])
    assert n == f["elements"]
    assert n * 2 == f["fp16_kilobytes"] * 1024


def test_kv_bytes_per_token_printed():
    f = FIG["kv_per_token"]
    b = sizes.kv_bytes_per_token(f["num_layers"], f["num_heads"], f["head_dim"], f["elem_bytes"])
    assert round(b / 2**20, f["printed_decimals"]) == f["approx_mib_per_token"]
    assert round(b * f["tokens"] / 2**30, f["gib_decimals"]) == pytest.approx(f["approx_gib_per_sequence"], abs=0.05)


def test_utilization_printed():
    f = FIG["contiguous_utilization"]
    assert 100 * sizes.contiguous_utilization(f["used"], f["reserved"]) == f["utilization_percent"]
    assert 100 * sizes.contiguous_waste(f["used"], f["reserved"]) == f["waste_percent"]
    g = FIG["contiguous_waste_50_of_2048"]
    w = 100 * sizes.contiguous_waste(g["used"], g["reserved"])
    assert g["printed_waste_percent"] <= w < g["printed_waste_percent"] + 0.1   # printed truncated


def test_paged_waste_bound():
    f = FIG["paged_internal_fragmentation"]
    B = f["block_size"]
    ws = [sizes.paged_waste_slots(n, B) for n in range(1, 200)]
    assert max(ws) == f["max_waste_slots"] and min(ws) == 0


def test_contiguous_bytes_formula():
    # 3 requests x 2 (K and V) x 4096 x 32 heads x 128 x 2 bytes
    assert sizes.contiguous_bytes(3, 4096, 32, 128, 2) == 3 * 2 * 4096 * 32 * 128 * 2


def test_kv_append_bitwise():
    N, H, B, d = 3, 2, 4, 5
    kc = np.zeros((N, H, B, d), np.uint16)
    vc = np.zeros((N, H, B, d), np.uint16)
    k = np.arange(3 * H * d, dtype=np.uint16).reshape(3, H, d) + 1
    v = k + 1000
    cache_ops.kv_append(kc, vc, k, v, [9, -1, 0])
    exp_k = np.zeros_like(kc)
    exp_k[2, :, 1, :] = k[0]            # slot 9 = block 2, offset 1
    exp_k[0, :, 0, :] = k[2]            # slot 0
    assert np.array_equal(kc, exp_k)
    exp_v = np.zeros_like(vc)
    exp_v[2, :, 1, :] = v[0]
    exp_v[0, :, 0, :] = v[2]
    assert np.array_equal(vc, exp_v)
    with pytest.raises(IndexError):
        cache_ops.kv_append(kc, vc, k, v, [12])


def test_copy_blocks_bitwise_and_nan_payload():
    x = torch.tensor([float("nan"), -0.0, 1.5, -2.0], dtype=torch.float16).reshape(1, 1, 2, 2)
    pool = torch.cat([x, torch.zeros_like(x)])
    kb = cache_ops.bits(pool).copy()
    vb = cache_ops.bits(pool * 2).copy()
    cache_ops.copy_blocks(kb, vb, [(0, 1)])
    assert np.array_equal(kb[1], kb[0]) and np.array_equal(vb[1], vb[0])
    assert kb[1].reshape(-1)[1] == 0x8000                  # -0.0 kept


def test_decode_bits():
    for dt, td in (("f32", torch.float32), ("f16", torch.float16), ("bf16", torch.bfloat16)):
        t = torch.tensor([1.0, -2.5, 3.140625, 65504.0 if dt != "bf16" else 1e30], dtype=td)
        assert np.array_equal(cache_ops.decode_bits(cache_ops.bits(t), dt), t.double().numpy())
