"""Oracle: bitwise K/V append and whole-block copy (TEST INFRASTRUCTURE).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.

* ``kv_append`` - [PA] §3.3 "按需分配策略", last step: write the new token's
  K and V vectors into the slot the block table gives it. A slot is the
  physical block id times the block size plus the offset inside the block
  ([PA] §3.2 "块表与地址转换": base + offset); a slot of -1 means "skip".
* ``copy_blocks`` - [VM] "写时复制与块共享机制" and [PA] §4.1: when a shared
  block must be modified, its content is first copied into a new physical
  block. The copy covers the whole block: every slot, every head, K and V.
* ``swap_blocks`` - the same whole-block copy between two pools (the GPU
  cache and the CPU swap space).

Both operate on the raw bits (integer views), so that the GPU result can be
compared bit for bit, NaN payloads and signed zeros included.
"""

from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np
import torch

_UINT = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def bits(x) -> np.ndarray:
    """Unsigned-integer view of a tensor/array with the same element width."""
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        width = x.element_size()
        return x.view({1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[width]).numpy().view(_UINT[width])
    x = np.ascontiguousarray(x)
    return x.view(_UINT[x.dtype.itemsize])


def decode_bits(b: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values of stored bits: IEEE binary32 (``f32``), IEEE binary16
    (``f16``) or bfloat16 (``bf16``, the upper 16 bits of a binary32)."""
    if dtype == "f32":
        return b.view(np.float32).astype(np.float64)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def kv_append(k_cache_bits: np.ndarray, v_cache_bits: np.ndarray, k_bits: np.ndarray,
              v_bits: np.ndarray, slot_mapping: Sequence[int]) -> None:
    """In place: for i in order, if slot_mapping[i] >= 0, row i of k/v
    (``[Hkv, d]``) goes to block slot // B, offset slot % B of every head.
    Caches are ``[N, Hkv, B, d]`` integer views."""
    N, H, B, d = k_cache_bits.shape
    for i, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        blk, off = divmod(slot, B)
        if blk >= N:
            raise IndexError(f"slot {slot} outside the pool")
        # every head's row at this (block, offset)
        k_cache_bits[blk, :, off, :] = k_bits[i]
        v_cache_bits[blk, :, off, :] = v_bits[i]


def copy_blocks(k_cache_bits: np.ndarray, v_cache_bits: np.ndarray,
                pairs: Sequence[Tuple[int, int]]) -> None:
    """In place: for each (src, dst) in order, K[dst] = K[src] and V[dst] = V[src],
    whole blocks."""
    for src, dst in pairs:
        k_cache_bits[int(dst)] = k_cache_bits[int(src)]
        v_cache_bits[int(dst)] = v_cache_bits[int(src)]


def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                pairs: Sequence[Tuple[int, int]]) -> None:
    """In place: for each (src, dst), dst_k[dst] = src_k[src] and dst_v[dst] =
    src_v[src], whole blocks, between two pools (the GPU cache and the swap
    space, [VM] "显存管理与调度策略设计": evicted KV moves to CPU memory and back)."""
    for src, dst in pairs:
        dst_k[int(dst)] = src_k[int(src)]
        dst_v[int(dst)] = src_v[int(src)]


def kv_append_fp8(k_codes, v_codes, k_scale, v_scale, k_rows, v_rows, slot_mapping, fmt: str = "fp8") -> None:
    """In place, quantised caches: for i in order, if slot_mapping[i] >= 0,
    every head's row of k[i] / v[i] is quantised (one float32 scale per row;
    ``fmt`` "fp8": E4M3 codes, ``quant.quantize_rows``; "int8": int8 codes,
    ``quant.quantize_rows_int8``) and its codes and scale go to block slot // B,
    offset slot % B. Codes are ``[N, Hkv, B, d]`` (uint8 / int8), scales
    ``[N, Hkv, B]`` float32; ``k_rows`` / ``v_rows`` are the source values
    ``[n, Hkv, d]`` as float32."""
    from . import quant
    N, H, B, d = k_codes.shape
    q = quant.quantize_rows if fmt == "fp8" else quant.quantize_rows_int8
    kc, ks = q(k_rows)
    vc, vs = q(v_rows)
    for i, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        blk, off = divmod(slot, B)
        if blk >= N:
            raise IndexError(f"slot {slot} outside the pool")
        k_codes[blk, :, off, :] = kc[i]
        v_codes[blk, :, off, :] = vc[i]
        k_scale[blk, :, off] = ks[i]
        v_scale[blk, :, off] = vs[i]
