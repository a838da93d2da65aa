"""Test helper: the logical (unpaged) view of a workload.

Tracks, for every sequence, the list of its K/V rows in position order by
following the workload's operations with plain list handling: a prompt sets
the list, a fork copies it, an append adds one row. No blocks, tables or
slots are involved, so this is an independent route to the contiguous K/V
that paged attention must reproduce.
"""

from __future__ import annotations

from typing import Dict, List, Tuple

import torch


def logical_decodes(wl) -> List[Tuple[Tuple[int, ...], torch.Tensor, Dict[int, Tuple[torch.Tensor, torch.Tensor]]]]:
    """For each decode op: (seq_ids, q, {seq: (K [ctx, Hkv, d], V [ctx, Hkv, d])})."""
    rows: Dict[int, Tuple[List[torch.Tensor], List[torch.Tensor]]] = {}
    out = []
    for op in wl.ops:
        if op.kind == "add_seq":
            s = op.seq_ids[0]
            rows[s] = (list(op.k.unbind(0)), list(op.v.unbind(0)))
        elif op.kind == "fork":
            p, c = op.seq_ids
            rows[c] = (list(rows[p][0]), list(rows[p][1]))
        elif op.kind == "append":
            for i, s in enumerate(op.seq_ids):
                rows[s][0].append(op.k[i])
                rows[s][1].append(op.v[i])
        elif op.kind == "decode":
            snap = {}
            for s in op.seq_ids:
                ks, vs = rows[s]
                shape = (0, wl.num_kv_heads, wl.head_dim)
                snap[s] = (torch.stack(ks) if ks else torch.zeros(shape, dtype=wl.torch_dtype),
                           torch.stack(vs) if vs else torch.zeros(shape, dtype=wl.torch_dtype))
            out.append((op.seq_ids, op.q, snap))
    return out


def sdpa_reference(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, scale: float) -> torch.Tensor:
    """torch scaled_dot_product_attention in float64 on the CPU for one sequence:
    q [Hq, d], K/V [ctx, Hkv, d] -> [Hq, d]; grouped-query heads via
    ``enable_gqa`` (query head h reads KV head h // (Hq / Hkv))."""
    Hq, d = q.shape
    if K.shape[0] == 0:
        return torch.zeros(Hq, d, dtype=torch.float64)
    qq = q.double().reshape(1, Hq, 1, d)
    kk = K.double().permute(1, 0, 2).unsqueeze(0).contiguous()
    vv = V.double().permute(1, 0, 2).unsqueeze(0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale,
                                                         enable_gqa=Hq != K.shape[1])
    return o.reshape(Hq, d)
