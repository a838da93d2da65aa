"""Paged KV-cache decode attention for AMD MI355X (gfx950).

Python binding of ``libpagedkv.so`` (C ABI declared in ``include/pagedkv.h``).
Argument marshalling only: every step of the decode path runs in the
library's HIP kernels or its C++ host allocator. torch tensors supply device
pointers and the current HIP stream; nothing here computes attention, slots
or copies. If the library has not been built, importing works but every call
raises ``LibraryNotBuilt`` - there is no fallback.

    python -m paged_kv_cache_411_amd.build      # builds libpagedkv.so in-tree

Calls (same names as the C ABI):
    pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, ...)
    kv_append(k, v, slot_mapping, k_cache, v_cache)
    copy_blocks(k_cache, v_cache, src_dst_pairs)
    stage_copy(dst, src)              # pa_stage_copy: pinned host -> device by a kernel
    BlockAllocator(num_blocks, block_size, free_order=None)  # pa_alloc_*
"""

from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "LIB_PATH", "LibraryNotBuilt", "PagedKVError", "NoFreeBlocks", "lib",
    "pa_decode", "pa_decode_noalloc", "pa_decode_noalloc_scratch_bytes", "pa_decode_workspace_bytes", "pa_decode_supported", "pa_decode_schedule", "pa_decode_share_width",
    "default_partition_size", "Schedule",
    "kv_append", "kv_append_staged", "kv_append_fp8", "copy_blocks", "copy_blocks_fp8", "stage_copy",
    "PA_FP8_E4M3", "PA_INT8", "is_fp8_cache",
    "BlockAllocator", "DTYPE_CODES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_NO_BLOCKS, PA_ERR_HIP = 0, -1, -2, -3, -4
DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
PA_FP8_E4M3 = 3
PA_INT8 = 4
FP8_CACHE_DTYPES = (torch.uint8, torch.float8_e4m3fn)   # tensors that hold E4M3 codes
QUANT_CACHE_DTYPES = FP8_CACHE_DTYPES + (torch.int8,)   # one-byte codes with a float32 scale per row


class LibraryNotBuilt(RuntimeError):
    pass


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class NoFreeBlocks(PagedKVError, MemoryError):
    pass


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("cache", CacheDesc), ("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
                ("partition_size", ctypes.c_int32), ("num_work", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("prof_events", ctypes.c_void_p * 2), ("work", ctypes.c_void_p), ("members", ctypes.c_void_p),
                ("num_members", ctypes.c_int32), ("num_slots", ctypes.c_void_p), ("max_slots", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("compact_tables", ctypes.c_int32), ("table_entries", ctypes.c_int32)]


class StepLayout(ctypes.Structure):
    _fields_ = [("slots", ctypes.c_size_t), ("pairs", ctypes.c_size_t), ("tables", ctypes.c_size_t),
                ("context_lens", ctypes.c_size_t), ("work", ctypes.c_size_t), ("members", ctypes.c_size_t),
                ("num_slots", ctypes.c_size_t), ("total", ctypes.c_size_t), ("num_seqs", ctypes.c_int32),
                ("width", ctypes.c_int32), ("work_capacity", ctypes.c_int32), ("partition_size", ctypes.c_int32)]


class StepPlan(ctypes.Structure):
    _fields_ = [("num_cow", ctypes.c_int32), ("num_work", ctypes.c_int32), ("num_members", ctypes.c_int32),
                ("max_slots", ctypes.c_int32), ("max_context", ctypes.c_int32), ("table_entries", ctypes.c_int32),
                ("tables_at", ctypes.c_size_t), ("upload_bytes", ctypes.c_size_t)]


class StepDesc(ctypes.Structure):
    _fields_ = [("cache", CacheDesc), ("num_q_heads", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("share_width", ctypes.c_int32), ("schedule", ctypes.c_int32), ("scale", ctypes.c_float),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("prof_events", ctypes.c_void_p * 2), ("layout", StepLayout),
                ("host_stage", ctypes.c_void_p), ("dev_stage", ctypes.c_void_p), ("done_flag", ctypes.c_void_p),
                ("done_value", ctypes.c_uint64)]


_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)
_VP = ctypes.c_void_p
_SIGS = {
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_decode": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, ctypes.POINTER(DecodeDesc), _VP]),
    "pa_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(DecodeDesc), ctypes.c_int32]),
    "pa_decode_noalloc": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, ctypes.POINTER(DecodeDesc),
                                         _VP]),
    "pa_decode_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "pa_decode_supported": (ctypes.c_int, [ctypes.c_int32] * 4),
    "pa_decode_supported_kv": (ctypes.c_int, [ctypes.c_int32] * 5),
    "kv_append_fp8": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, _VP, ctypes.c_int32, _VP, _VP, _VP, _VP,
                                     ctypes.POINTER(CacheDesc), _VP, _VP, ctypes.c_size_t, _VP]),
    "copy_blocks_fp8": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, ctypes.c_int32, ctypes.POINTER(CacheDesc), _VP]),
    "pa_decode_share_width": (ctypes.c_int32, []),
    "pa_decode_schedule": (ctypes.c_int32, [_VP, _VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_int32, _VP, ctypes.c_int32,
                                            _I32P, _VP, _I32P]),
    "kv_append": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int32, _VP, _VP, ctypes.POINTER(CacheDesc), _VP]),
    "copy_blocks": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int32, ctypes.POINTER(CacheDesc), _VP]),
    "pa_stage_copy": (ctypes.c_int, [_VP, _VP, ctypes.c_size_t, _VP]),
    "kv_append_staged": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int32, _VP, _VP, ctypes.POINTER(CacheDesc), _VP,
                                        _VP, ctypes.c_size_t, _VP]),
    "pa_alloc_create": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, _VP, ctypes.POINTER(_VP)]),
    "pa_alloc_destroy": (None, [_VP]),
    "pa_alloc_add_seq": (ctypes.c_int, [_VP, ctypes.c_int64, ctypes.c_int32]),
    "pa_alloc_fork": (ctypes.c_int, [_VP, ctypes.c_int64, ctypes.c_int64]),
    "pa_alloc_append_slots": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, _VP, _VP, ctypes.c_int32, _I32P]),
    "pa_alloc_table_width": (ctypes.c_int32, [_VP, _VP, ctypes.c_int32, ctypes.c_int32]),
    "pa_alloc_step": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _VP, _VP,
                                     ctypes.c_int32, _I32P, _VP, _VP, _I32P]),
    "pa_alloc_free_seq": (ctypes.c_int, [_VP, ctypes.c_int64]),
    "pa_alloc_seq_slots": (ctypes.c_int, [_VP, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _VP]),
    "pa_alloc_block_tables": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP]),
    "pa_alloc_num_free": (ctypes.c_int32, [_VP]),
    "pa_alloc_num_blocks": (ctypes.c_int32, [_VP]),
    "pa_alloc_ref_count": (ctypes.c_int32, [_VP, ctypes.c_int32]),
    "pa_alloc_context_len": (ctypes.c_int32, [_VP, ctypes.c_int64]),
    "pa_alloc_num_table_blocks": (ctypes.c_int32, [_VP, ctypes.c_int64]),
    "pa_alloc_free_list": (ctypes.c_int32, [_VP, _VP, ctypes.c_int32]),
    "swap_blocks": (ctypes.c_int, [_VP, _VP, _VP, _VP, ctypes.POINTER(CacheDesc), _VP, _VP, _VP, _VP,
                                   ctypes.c_int32, _VP, ctypes.c_int32, ctypes.c_int32, _VP]),
    "pa_alloc_set_swap_space": (ctypes.c_int, [_VP, ctypes.c_int32, _VP]),
    "pa_alloc_swap_out": (ctypes.c_int, [_VP, ctypes.c_int64, _VP, ctypes.c_int32, _I32P]),
    "pa_alloc_swap_in": (ctypes.c_int, [_VP, ctypes.c_int64, _VP, ctypes.c_int32, _I32P]),
    "pa_alloc_num_free_swap": (ctypes.c_int32, [_VP]),
    "pa_alloc_swap_free_list": (ctypes.c_int32, [_VP, _VP, ctypes.c_int32]),
    "pa_alloc_is_swapped": (ctypes.c_int32, [_VP, ctypes.c_int64]),
    "pa_alloc_seq_table": (ctypes.c_int32, [_VP, ctypes.c_int64, _VP, ctypes.c_int32]),
    "pa_alloc_enable_prefix_caching": (ctypes.c_int, [_VP]),
    "pa_alloc_add_seq_cached": (ctypes.c_int, [_VP, ctypes.c_int64, _VP, ctypes.c_int32, ctypes.c_int64, _I32P]),
    "pa_alloc_prefix_hits": (ctypes.c_int32, [_VP, _VP, ctypes.c_int32, ctypes.c_int64, _VP, ctypes.c_int32]),
    "pa_alloc_num_cached_blocks": (ctypes.c_int32, [_VP]),
    "pa_alloc_admit": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, _I32P]),
    "pa_alloc_block_is_cached": (ctypes.c_int32, [_VP, ctypes.c_int32]),
    "pa_alloc_set_watermark": (ctypes.c_int, [_VP, ctypes.c_double]),
    "pa_step_layout": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(StepLayout)]),
    "pa_decode_step": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, _VP,
                                      ctypes.POINTER(StepDesc), _VP, _I32P]),
    "pa_decode_step_plan": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(StepDesc),
                                           ctypes.POINTER(StepPlan)]),
    "pa_alloc_can_allocate": (ctypes.c_int, [_VP, ctypes.c_int32]),
}
EXPORTED = tuple(_SIGS)

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises LibraryNotBuilt if libpagedkv.so is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(f"{LIB_PATH} is missing: build it with "
                                  "`python -m paged_kv_cache_411_amd.build` (no fallback exists)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != PA_OK:
        msg = lib().pa_last_error().decode(errors="replace")
        cls = NoFreeBlocks if rc == PA_ERR_NO_BLOCKS else PagedKVError
        raise cls(rc, f"{what}: {msg}")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(t: torch.Tensor, stream) -> int:
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(t.device.index)   # torch's current stream on t's device, as a hipStream_t
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise PagedKVError(PA_ERR_INVALID, f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise PagedKVError(PA_ERR_INVALID, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PagedKVError(PA_ERR_INVALID, f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def is_fp8_cache(t: torch.Tensor) -> bool:
    """A cache of one-byte codes with a float32 scale per row: FP8 E4M3
    (uint8 / float8_e4m3fn tensors) or INT8 (int8 tensors)."""
    return t.dtype in QUANT_CACHE_DTYPES


def _quant_code(dtype: torch.dtype) -> int:
    return PA_INT8 if dtype == torch.int8 else PA_FP8_E4M3


def cache_desc(k_cache: torch.Tensor) -> CacheDesc:
    if k_cache.dim() != 4 or (k_cache.dtype not in DTYPE_CODES and not is_fp8_cache(k_cache)):
        raise PagedKVError(PA_ERR_INVALID, "cache must be [num_blocks, num_kv_heads, block_size, head_dim] "
                                           "f32/f16/bf16, uint8 / float8_e4m3fn E4M3 codes or int8 codes")
    N, H, B, d = k_cache.shape
    return CacheDesc(N, H, B, d, _quant_code(k_cache.dtype) if is_fp8_cache(k_cache) else DTYPE_CODES[k_cache.dtype])


def decode_desc(q, k_cache, block_tables, max_context_len=0, partition_size=0, max_blocks=None) -> DecodeDesc:
    c = cache_desc(k_cache)
    S, Hq, d = q.shape
    mb = block_tables.shape[1] if max_blocks is None else int(max_blocks)
    return DecodeDesc(c, S, Hq, mb, int(max_context_len), int(partition_size), 0, None, 0,
                      (_VP * 2)(None, None), None, None, 0, None, 0, DTYPE_CODES.get(q.dtype, 0), None, None)


def pa_decode_workspace_bytes(q, k_cache, block_tables, max_context_len=0, partition_size=0,
                              scheduled: bool = False) -> int:
    """Workspace bytes pa_decode needs (``scheduled``: for a launch with a schedule)."""
    desc = decode_desc(q, k_cache, block_tables, max_context_len, partition_size)
    n = lib().pa_decode_workspace_bytes(ctypes.byref(desc), int(bool(scheduled)))
    msg = lib().pa_last_error().decode()
    if n == 0 and msg:
        raise PagedKVError(PA_ERR_INVALID, f"pa_decode_workspace_bytes: {msg}")
    return int(n)


def default_partition_size(block_size: int) -> int:
    """The partition size pa_decode uses when given 0: min(1024, 64 * block_size)."""
    return min(1024, 64 * block_size)


_share_width: Optional[int] = None


def pa_decode_share_width() -> int:
    """Most sequences one shared schedule item serves (a constant of the library)."""
    global _share_width
    if _share_width is None:
        _share_width = int(lib().pa_decode_share_width())
    return _share_width


class Schedule(NamedTuple):
    """A pa_decode launch schedule (host arrays): ``work`` int32 ``[n, 8]``
    items, ``members`` int32, ``num_slots`` int32 ``[S]``, ``max_slots``."""
    work: np.ndarray
    members: np.ndarray
    num_slots: np.ndarray
    max_slots: int


def pa_decode_schedule(context_lens: np.ndarray, block_size: int, partition_size: int = 0,
                       max_context_len: int = 0, block_tables: Optional[np.ndarray] = None, share_width: int = 1,
                       out: Optional[np.ndarray] = None, out_members: Optional[np.ndarray] = None,
                       out_num_slots: Optional[np.ndarray] = None) -> Schedule:
    """Launch schedule (``pa_decode_schedule``). With ``share_width`` > 1 and
    the host ``block_tables`` (int32 ``[S, max_blocks]``), sequences whose
    tables start with the same physical blocks share the ranges of that run.
    ``out`` / ``out_members`` / ``out_num_slots`` receive the result in place
    when given."""
    ctx = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    S = ctx.shape[0]
    part = partition_size or default_partition_size(block_size)
    if out is None:
        cap = int(sum(max(1, -(-int(c) // part) + 1) for c in ctx))
        out = np.empty((max(cap, 1), 8), np.int32)
    if out_members is None:
        out_members = np.empty(max(S, 1), np.int32)
    if out_num_slots is None:
        out_num_slots = np.empty(max(S, 1), np.int32)
    for a_, cols in ((out, 8), (out_members, None), (out_num_slots, None)):
        if a_.dtype != np.int32 or not a_.flags.c_contiguous or (cols and (a_.ndim != 2 or a_.shape[1] != cols)):
            raise PagedKVError(PA_ERR_INVALID, "pa_decode_schedule: outputs must be contiguous int32 ([cap, 8] items)")
    if out_num_slots.shape[0] < S:
        raise PagedKVError(PA_ERR_INVALID, "pa_decode_schedule: out_num_slots too small")
    tab_ptr, mb = None, 0
    if block_tables is not None:
        if block_tables.dtype != np.int32 or not block_tables.flags.c_contiguous or block_tables.shape[0] < S:
            raise PagedKVError(PA_ERR_INVALID, "pa_decode_schedule: block_tables must be contiguous int32 [S, max_blocks]")
        tab_ptr, mb = block_tables.ctypes.data, block_tables.shape[1]
    nm = ctypes.c_int32(0)
    ms = ctypes.c_int32(0)
    n = lib().pa_decode_schedule(ctx.ctypes.data, tab_ptr, S, mb, block_size, partition_size, max_context_len,
                                 share_width, out.ctypes.data, out.shape[0], out_members.ctypes.data,
                                 out_members.shape[0], ctypes.byref(nm), out_num_slots.ctypes.data, ctypes.byref(ms))
    if n < 0:
        raise PagedKVError(PA_ERR_INVALID, "pa_decode_schedule: " + lib().pa_last_error().decode())
    return Schedule(out[:n], out_members[:nm.value], out_num_slots[:S], ms.value)


def pa_decode_supported(dtype: torch.dtype, head_dim: int, block_size: int, group: int,
                        cache_dtype: Optional[torch.dtype] = None) -> bool:
    """Whether pa_decode has a kernel for q/out of ``dtype`` over a cache of
    ``cache_dtype`` (default the same; uint8 / float8_e4m3fn for FP8 codes)."""
    kt = DTYPE_CODES[dtype] if cache_dtype is None else (
        _quant_code(cache_dtype) if cache_dtype in QUANT_CACHE_DTYPES else DTYPE_CODES[cache_dtype])
    return bool(lib().pa_decode_supported_kv(DTYPE_CODES[dtype], kt, head_dim, block_size, group))


def pa_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale: float, out, *,
                      max_context_len: int = 0, partition_size: int = 0,
                      prof_events: Optional[Tuple[torch.cuda.Event, torch.cuda.Event]] = None,
                      work: Optional[torch.Tensor] = None, members: Optional[torch.Tensor] = None,
                      num_slots: Optional[torch.Tensor] = None, max_slots: int = 0,
                      k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                      compact_width: Optional[int] = None, stream=None):
    """``pa_decode`` without a workspace and without allocating anything: the
    partial results go to the library's own scratch on the device (see
    ``pa_decode_noalloc`` in pagedkv.h). Same arguments as ``pa_decode``
    minus ``workspace``."""
    return _decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len, partition_size,
                   None, prof_events, work, members, num_slots, max_slots, k_scale, v_scale, compact_width,
                   stream, noalloc=True)


def pa_decode_noalloc_scratch_bytes() -> int:
    """Bytes of the scratch ``pa_decode_noalloc`` uses on each device."""
    return int(lib().pa_decode_noalloc_scratch_bytes())


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, out, *,
              max_context_len: int = 0, partition_size: int = 0, workspace: Optional[torch.Tensor] = None,
              prof_events: Optional[Tuple[torch.cuda.Event, torch.cuda.Event]] = None,
              work: Optional[torch.Tensor] = None, members: Optional[torch.Tensor] = None,
              num_slots: Optional[torch.Tensor] = None, max_slots: int = 0,
              k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
              compact_width: Optional[int] = None, stream=None):
    """Single-query paged attention into ``out`` (see ``pa_decode`` in pagedkv.h).

    q/out ``[S, Hq, d]``; caches ``[N, Hkv, B, d]``; block_tables int32 ``[S, max_blocks]``;
    context_lens int32 ``[S]``. ``workspace`` (uint8, at least
    ``pa_decode_workspace_bytes`` bytes) is allocated when not given.
    ``prof_events`` is an optional pair of timing events recorded around the
    partition kernel. ``work`` (int32 ``[n, 8]``), ``members`` (int32),
    ``num_slots`` (int32 ``[S]``) and ``max_slots`` are an optional device
    launch schedule as ``pa_decode_schedule`` makes it. With ``compact_width``
    (the longest row), ``block_tables`` is the compact int32 array (every
    sequence's ceil(ctx / B) entries back to back) and ``work`` must carry the
    rows (ints 6 and 7 of each item: the row's start and length). FP8 caches (uint8 or
    float8_e4m3fn codes) need ``k_scale`` / ``v_scale`` (float32
    ``[N, Hkv, B]``) and fp16 / bf16 q."""
    return _decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len, partition_size,
                   workspace, prof_events, work, members, num_slots, max_slots, k_scale, v_scale, compact_width,
                   stream, noalloc=False)


def _decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len, partition_size,
            workspace, prof_events, work, members, num_slots, max_slots, k_scale, v_scale, compact_width, stream,
            noalloc: bool):
    dt = q.dtype
    fp8 = is_fp8_cache(k_cache)
    if q.dim() != 3 or out.shape != q.shape or out.dtype != dt:
        raise PagedKVError(PA_ERR_INVALID, "q and out must both be [S, Hq, d] of one dtype")
    if k_cache.shape != v_cache.shape or v_cache.dtype != k_cache.dtype or (not fp8 and k_cache.dtype != dt):
        raise PagedKVError(PA_ERR_INVALID, "caches must match each other and q's dtype (or both hold FP8 codes)")
    if fp8 and (k_scale is None or v_scale is None or k_scale.shape != k_cache.shape[:3]
                or v_scale.shape != k_cache.shape[:3]):
        raise PagedKVError(PA_ERR_INVALID, "FP8 caches need k_scale / v_scale float32 [N, Hkv, B]")
    compact = compact_width is not None
    if compact:
        if block_tables.dim() != 1 or work is None or context_lens.shape != (q.shape[0],):
            raise PagedKVError(PA_ERR_INVALID, "compact block_tables: a 1-D int32 array, with a schedule")
    elif block_tables.dim() != 2 or block_tables.shape[0] != q.shape[0] or context_lens.shape != (q.shape[0],):
        raise PagedKVError(PA_ERR_INVALID, "block_tables [S, max_blocks] / context_lens [S] shape mismatch")
    if q.shape[2] != k_cache.shape[3]:
        raise PagedKVError(PA_ERR_INVALID, "head_dim mismatch between q and the caches")
    ptrs = [_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
            _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
            _dev(out, "out")]
    desc = decode_desc(q, k_cache, block_tables, max_context_len, partition_size,
                       max_blocks=compact_width if compact else None)
    if compact:
        desc.compact_tables = 1
        desc.table_entries = block_tables.numel()
    if not noalloc:
        need = lib().pa_decode_workspace_bytes(ctypes.byref(desc), int(work is not None))
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        desc.workspace = _dev(workspace, "workspace")
        desc.workspace_bytes = workspace.numel() * workspace.element_size()
    if prof_events is not None:
        desc.prof_events[0] = getattr(prof_events[0], "handle", None) or prof_events[0].cuda_event
        desc.prof_events[1] = getattr(prof_events[1], "handle", None) or prof_events[1].cuda_event
    if work is not None:
        if work.dim() != 2 or work.shape[1] != 8:
            raise PagedKVError(PA_ERR_INVALID, "work must be int32 [n, 8]")
        if num_slots is None or num_slots.shape != (q.shape[0],):
            raise PagedKVError(PA_ERR_INVALID, "a schedule needs num_slots int32 [S]")
        desc.work = _dev(work, "work", torch.int32)
        desc.num_work = work.shape[0]
        desc.num_slots = _dev(num_slots, "num_slots", torch.int32)
        desc.max_slots = int(max_slots)
        if members is not None and members.numel() > 0:
            desc.members = _dev(members, "members", torch.int32)
            desc.num_members = members.numel()
    if fp8:
        desc.k_scale = _dev(k_scale, "k_scale", torch.float32)
        desc.v_scale = _dev(v_scale, "v_scale", torch.float32)
    fn = lib().pa_decode_noalloc if noalloc else lib().pa_decode
    rc = fn(*ptrs[:5], ctypes.c_float(scale), ptrs[5], ctypes.byref(desc), _stream_ptr(q, stream))
    _check(rc, "pa_decode_noalloc" if noalloc else "pa_decode")
    return out


def kv_append(k, v, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """Write token rows k/v ``[N, Hkv, d]`` into the caches at ``slot_mapping``
    (int64 ``[N]``, -1 = skip)."""
    if k.shape != v.shape or k.dim() != 3 or k.shape[1:] != (k_cache.shape[1], k_cache.shape[3]):
        raise PagedKVError(PA_ERR_INVALID, "k/v must be [N, num_kv_heads, head_dim] matching the caches")
    if k.dtype != k_cache.dtype or v.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype \
            or v_cache.shape != k_cache.shape:
        raise PagedKVError(PA_ERR_INVALID, "k, v and both caches must share one dtype and shape")
    if slot_mapping.shape != (k.shape[0],):
        raise PagedKVError(PA_ERR_INVALID, "slot_mapping must be [N]")
    desc = cache_desc(k_cache)
    rc = lib().kv_append(_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping", torch.int64), k.shape[0],
                         _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), ctypes.byref(desc),
                         _stream_ptr(k, stream))
    _check(rc, "kv_append")


def _dev_or_pinned(t: torch.Tensor, name: str, dtype) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_contiguous() or t.dtype != dtype:
        raise PagedKVError(PA_ERR_INVALID, f"{name} must be a contiguous {dtype} tensor")
    if t.device.type != "cuda" and not t.is_pinned():
        raise PagedKVError(PA_ERR_INVALID, f"{name} must be on the device or in pinned host memory")
    return t.data_ptr()


def kv_append_staged(k, v, slot_mapping, k_cache, v_cache, stage_dst: torch.Tensor, stage_src: torch.Tensor,
                     stream=None) -> None:
    """``kv_append`` and ``stage_copy(stage_dst, stage_src)`` in one launch;
    ``slot_mapping`` (int64 ``[N]``) may live in pinned host memory."""
    if k.shape != v.shape or k.dim() != 3 or k.shape[1:] != (k_cache.shape[1], k_cache.shape[3]):
        raise PagedKVError(PA_ERR_INVALID, "k/v must be [N, num_kv_heads, head_dim] matching the caches")
    if k.dtype != k_cache.dtype or v.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype \
            or v_cache.shape != k_cache.shape:
        raise PagedKVError(PA_ERR_INVALID, "k, v and both caches must share one dtype and shape")
    if slot_mapping.shape != (k.shape[0],):
        raise PagedKVError(PA_ERR_INVALID, "slot_mapping must be [N]")
    if not stage_src.is_contiguous() or not stage_dst.is_contiguous() or stage_dst.device.type != "cuda":
        raise PagedKVError(PA_ERR_INVALID, "kv_append_staged: contiguous staging tensors, dst on the device")
    if stage_src.device.type != "cuda" and not stage_src.is_pinned():
        raise PagedKVError(PA_ERR_INVALID, "kv_append_staged: a host staging source must be pinned memory")
    nbytes = stage_src.numel() * stage_src.element_size()
    if stage_dst.numel() * stage_dst.element_size() < nbytes:
        raise PagedKVError(PA_ERR_INVALID, "kv_append_staged: staging destination too small")
    desc = cache_desc(k_cache)
    rc = lib().kv_append_staged(_dev(k, "k"), _dev(v, "v"), _dev_or_pinned(slot_mapping, "slot_mapping", torch.int64),
                                k.shape[0], _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), ctypes.byref(desc),
                                stage_dst.data_ptr(), stage_src.data_ptr(), nbytes, _stream_ptr(k_cache, stream))
    _check(rc, "kv_append_staged")


def kv_append_fp8(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, stage_dst: Optional[torch.Tensor] = None,
                  stage_src: Optional[torch.Tensor] = None, stream=None) -> None:
    """Quantise K/V rows ``[N, Hkv, d]`` (f32/f16/bf16) into FP8 caches (codes
    ``[N_blk, Hkv, B, d]`` uint8 / float8_e4m3fn, scales float32
    ``[N_blk, Hkv, B]``) at ``slot_mapping`` (int64 ``[N]``, device or pinned).
    ``stage_src`` -> ``stage_dst`` bytes are copied in the same launch when given."""
    if k.shape != v.shape or k.dim() != 3 or k.shape[1:] != (k_cache.shape[1], k_cache.shape[3]):
        raise PagedKVError(PA_ERR_INVALID, "k/v must be [N, num_kv_heads, head_dim] matching the caches")
    if not is_fp8_cache(k_cache) or v_cache.dtype != k_cache.dtype or v_cache.shape != k_cache.shape:
        raise PagedKVError(PA_ERR_INVALID, "kv_append_fp8 writes FP8 / INT8 caches (uint8 / float8_e4m3fn / int8)")
    if k.dtype not in DTYPE_CODES or v.dtype != k.dtype:
        raise PagedKVError(PA_ERR_INVALID, "k and v must share an f32/f16/bf16 dtype")
    if k_scale.shape != k_cache.shape[:3] or v_scale.shape != k_cache.shape[:3]:
        raise PagedKVError(PA_ERR_INVALID, "scales must be float32 [N, Hkv, B]")
    if slot_mapping.shape != (k.shape[0],):
        raise PagedKVError(PA_ERR_INVALID, "slot_mapping must be [N]")
    nbytes, dst_ptr, src_ptr = 0, None, None
    if stage_src is not None:
        if stage_dst is None or stage_dst.device.type != "cuda" or \
                (stage_src.device.type != "cuda" and not stage_src.is_pinned()):
            raise PagedKVError(PA_ERR_INVALID, "kv_append_fp8: staging needs a device dst and a pinned or device src")
        nbytes = stage_src.numel() * stage_src.element_size()
        if stage_dst.numel() * stage_dst.element_size() < nbytes:
            raise PagedKVError(PA_ERR_INVALID, "kv_append_fp8: staging destination too small")
        dst_ptr, src_ptr = stage_dst.data_ptr(), stage_src.data_ptr()
    desc = cache_desc(k_cache)
    rc = lib().kv_append_fp8(_dev(k, "k"), _dev(v, "v"), DTYPE_CODES[k.dtype],
                             _dev_or_pinned(slot_mapping, "slot_mapping", torch.int64), k.shape[0],
                             _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                             _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
                             ctypes.byref(desc), dst_ptr, src_ptr, nbytes, _stream_ptr(k_cache, stream))
    _check(rc, "kv_append_fp8")


def copy_blocks_fp8(k_cache, v_cache, k_scale, v_scale, src_dst_pairs, stream=None) -> None:
    """copy_blocks for FP8 caches: whole blocks of codes and of their scales."""
    if v_cache.shape != k_cache.shape or not is_fp8_cache(k_cache) or v_cache.dtype != k_cache.dtype:
        raise PagedKVError(PA_ERR_INVALID, "copy_blocks_fp8 takes matching FP8 caches")
    if src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise PagedKVError(PA_ERR_INVALID, "src_dst_pairs must be [M, 2]")
    desc = cache_desc(k_cache)
    rc = lib().copy_blocks_fp8(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                               _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
                               _dev_or_pinned(src_dst_pairs, "src_dst_pairs", torch.int64), src_dst_pairs.shape[0],
                               ctypes.byref(desc), _stream_ptr(k_cache, stream))
    _check(rc, "copy_blocks_fp8")


def copy_blocks(k_cache, v_cache, src_dst_pairs, stream=None) -> None:
    """Whole-block copies K[dst] = K[src], V[dst] = V[src] for int64 pairs ``[M, 2]``
    (device or pinned host memory)."""
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise PagedKVError(PA_ERR_INVALID, "caches must match")
    if src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise PagedKVError(PA_ERR_INVALID, "src_dst_pairs must be [M, 2]")
    desc = cache_desc(k_cache)
    rc = lib().copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev_or_pinned(src_dst_pairs, "src_dst_pairs", torch.int64), src_dst_pairs.shape[0],
                           ctypes.byref(desc), _stream_ptr(k_cache, stream))
    _check(rc, "copy_blocks")


PA_SWAP_OUT = 0
PA_SWAP_IN = 1


def _pool(t: Optional[torch.Tensor], name: str, dtype) -> int:
    """Pointer of a swap-space tensor: a contiguous device tensor or pinned host tensor."""
    if t is None:
        return None
    if not t.is_contiguous() or t.dtype != dtype:
        raise PagedKVError(PA_ERR_INVALID, f"{name} must be contiguous {dtype}")
    if t.device.type != "cuda" and not t.is_pinned():
        raise PagedKVError(PA_ERR_INVALID, f"{name}: host memory must be pinned")
    return t.data_ptr()


def swap_blocks(k_cache, v_cache, swap_k, swap_v, src_dst_pairs, direction: int, k_scale=None, v_scale=None,
                swap_k_scale=None, swap_v_scale=None, stream=None) -> None:
    """Whole-block moves between the device caches and a swap space
    ``[S, Hkv, B, d]`` (pinned host or device memory): ``direction`` PA_SWAP_OUT
    takes (device, swap) pairs, PA_SWAP_IN (swap, device) pairs, int64 ``[M, 2]``
    on the device or pinned. FP8 caches also move their scales."""
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise PagedKVError(PA_ERR_INVALID, "caches must match")
    if swap_k.shape[1:] != k_cache.shape[1:] or swap_v.shape != swap_k.shape:
        raise PagedKVError(PA_ERR_INVALID, "swap space must hold blocks shaped like the cache's")
    if src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise PagedKVError(PA_ERR_INVALID, "src_dst_pairs must be [M, 2]")
    fp8 = is_fp8_cache(k_cache)
    if fp8:
        for name, t, rows in (("k_scale", k_scale, k_cache.shape[0]), ("v_scale", v_scale, k_cache.shape[0]),
                              ("swap_k_scale", swap_k_scale, swap_k.shape[0]),
                              ("swap_v_scale", swap_v_scale, swap_k.shape[0])):
            if t is None or tuple(t.shape) != (rows, *k_cache.shape[1:3]):
                raise PagedKVError(PA_ERR_INVALID, f"{name} must be float32 [{rows}, Hkv, B]")
    desc = cache_desc(k_cache)
    rc = lib().swap_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev(k_scale, "k_scale", torch.float32) if fp8 else None,
                           _dev(v_scale, "v_scale", torch.float32) if fp8 else None, ctypes.byref(desc),
                           _pool(swap_k, "swap_k", k_cache.dtype), _pool(swap_v, "swap_v", k_cache.dtype),
                           _pool(swap_k_scale, "swap_k_scale", torch.float32) if fp8 else None,
                           _pool(swap_v_scale, "swap_v_scale", torch.float32) if fp8 else None,
                           swap_k.shape[0], _dev_or_pinned(src_dst_pairs, "src_dst_pairs", torch.int64),
                           src_dst_pairs.shape[0], int(direction), _stream_ptr(k_cache, stream))
    _check(rc, "swap_blocks")


def step_layout(num_seqs: int, width: int, block_size: int, partition_size: int = 0) -> StepLayout:
    """Byte layout of a decode step's staging buffer (``pa_step_layout``)."""
    out = StepLayout()
    _check(lib().pa_step_layout(num_seqs, width, block_size, partition_size, ctypes.byref(out)), "pa_step_layout")
    return out


def decode_step(alloc: "BlockAllocator", seq_ids: np.ndarray, append: bool, k_new, v_new, q, out, k_cache,
                v_cache, desc: StepDesc, stream=None) -> int:
    """``pa_decode_step``: one whole decode step (allocator step, schedule,
    copies, staged upload + append, attention). ``seq_ids`` int64 [n]; the
    tensors on the device; ``desc`` filled by the caller (see pagedkv.h).
    Returns the longest context."""
    mc = ctypes.c_int32(0)
    rc = lib().pa_decode_step(alloc._h, seq_ids.ctypes.data, seq_ids.shape[0], int(bool(append)),
                              k_new.data_ptr() if append else None, v_new.data_ptr() if append else None,
                              q.data_ptr(), out.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                              ctypes.byref(desc), _stream_ptr(q, stream), ctypes.byref(mc))
    _check(rc, "pa_decode_step")
    return mc.value


def stage_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    """Copy the bytes of ``src`` (pinned host or device tensor) into the device
    tensor ``dst`` with the library's copy kernel (``pa_stage_copy``)."""
    if not src.is_contiguous() or not dst.is_contiguous() or dst.device.type != "cuda":
        raise PagedKVError(PA_ERR_INVALID, "stage_copy: contiguous tensors, dst on the device")
    if src.device.type != "cuda" and not src.is_pinned():
        raise PagedKVError(PA_ERR_INVALID, "stage_copy: a host source must be pinned memory")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise PagedKVError(PA_ERR_INVALID, "stage_copy: destination too small")
    _check(lib().pa_stage_copy(dst.data_ptr(), src.data_ptr(), nbytes, _stream_ptr(dst, stream)), "pa_stage_copy")


def _np_ptr(a: np.ndarray, dtype) -> int:
    if a.dtype != dtype or not a.flags.c_contiguous:
        raise PagedKVError(PA_ERR_INVALID, f"host buffer must be contiguous {dtype}")
    return a.ctypes.data


class BlockAllocator:
    """Host block allocator (pa_alloc_* in pagedkv.h): FIFO free queue,
    reference counts, per-sequence block tables, fork, copy-on-write, free."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        self._l = lib()
        h = _VP()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if order.shape != (num_blocks,):
                raise PagedKVError(PA_ERR_INVALID, "free_order must hold num_blocks entries")
        _check(self._l.pa_alloc_create(num_blocks, block_size, None if order is None else order.ctypes.data,
                                       ctypes.byref(h)), "pa_alloc_create")
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._l.pa_alloc_destroy(h)
            self._h = None

    def add_seq(self, seq_id: int, num_tokens: int) -> None:
        _check(self._l.pa_alloc_add_seq(self._h, seq_id, num_tokens), "pa_alloc_add_seq")

    def fork(self, parent: int, child: int) -> None:
        _check(self._l.pa_alloc_fork(self._h, parent, child), "pa_alloc_fork")

    def append_slots(self, seq_ids, out_slots: Optional[np.ndarray] = None,
                     out_pairs: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        """One token for each listed sequence; returns (slots int64 [n],
        copy-on-write pairs int64 [M, 2]). Optional output buffers (for pinned
        staging) must be int64 [n] and int64 [>= n, 2]."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = ids.shape[0]
        slots = np.empty(n, np.int64) if out_slots is None else out_slots
        pairs = np.empty((max(n, 1), 2), np.int64) if out_pairs is None else out_pairs
        ncow = ctypes.c_int32(0)
        _check(self._l.pa_alloc_append_slots(self._h, ids.ctypes.data, n, _np_ptr(slots, np.int64),
                                             _np_ptr(pairs, np.int64), pairs.shape[0], ctypes.byref(ncow)),
               "pa_alloc_append_slots")
        return slots[:n], pairs[:ncow.value]

    def table_width(self, seq_ids, append: bool = False) -> int:
        """Longest table among ``seq_ids`` (after one more token each if ``append``)."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        w = self._l.pa_alloc_table_width(self._h, ids.ctypes.data, ids.shape[0], int(bool(append)))
        if w < 0:
            raise PagedKVError(PA_ERR_INVALID, "pa_alloc_table_width: " + self._l.pa_last_error().decode())
        return int(w)

    def step(self, seq_ids: np.ndarray, append: bool, max_blocks: int, slots: Optional[np.ndarray],
             pairs: Optional[np.ndarray], tables: np.ndarray, context_lens: np.ndarray) -> Tuple[int, int]:
        """pa_alloc_step into caller buffers (int64 ``seq_ids`` [n]; int64 ``slots`` [n];
        int64 ``pairs`` [cap, 2]; int32 ``tables`` [n, max_blocks]; int32
        ``context_lens`` [n]); returns (number of copy pairs, largest context)."""
        n = seq_ids.shape[0]
        if seq_ids.dtype != np.int64 or tables.dtype != np.int32 or context_lens.dtype != np.int32 \
                or tables.size < n * max_blocks or context_lens.shape[0] < n:
            raise PagedKVError(PA_ERR_INVALID, "step: buffer types or sizes")
        if append and (slots is None or pairs is None or slots.shape[0] < n or slots.dtype != np.int64
                       or pairs.dtype != np.int64):
            raise PagedKVError(PA_ERR_INVALID, "step: slot / pair buffers")
        ncow = ctypes.c_int32(0)
        mc = ctypes.c_int32(0)
        _check(self._l.pa_alloc_step(self._h, seq_ids.ctypes.data, n, int(bool(append)), max_blocks,
                                     None if slots is None else slots.ctypes.data,
                                     None if pairs is None else pairs.ctypes.data,
                                     0 if pairs is None else pairs.shape[0], ctypes.byref(ncow),
                                     tables.ctypes.data, context_lens.ctypes.data, ctypes.byref(mc)),
               "pa_alloc_step")
        return ncow.value, mc.value

    def free_seq(self, seq_id: int) -> None:
        _check(self._l.pa_alloc_free_seq(self._h, seq_id), "pa_alloc_free_seq")

    def seq_slots(self, seq_id: int, start: int, count: int) -> np.ndarray:
        out = np.empty(count, np.int64)
        _check(self._l.pa_alloc_seq_slots(self._h, seq_id, start, count, out.ctypes.data), "pa_alloc_seq_slots")
        return out

    def block_tables(self, seq_ids, max_blocks: int, out_tables: Optional[np.ndarray] = None,
                     out_context_lens: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = ids.shape[0]
        tables = np.empty((n, max_blocks), np.int32) if out_tables is None else out_tables
        ctx = np.empty(n, np.int32) if out_context_lens is None else out_context_lens
        if tables.shape != (n, max_blocks) or ctx.shape != (n,):
            raise PagedKVError(PA_ERR_INVALID, "block_tables output buffers have the wrong shape")
        _check(self._l.pa_alloc_block_tables(self._h, ids.ctypes.data, n, max_blocks, _np_ptr(tables, np.int32),
                                             _np_ptr(ctx, np.int32)), "pa_alloc_block_tables")
        return tables, ctx

    def num_free(self) -> int:
        return self._l.pa_alloc_num_free(self._h)

    def ref_count(self, block: int) -> int:
        return self._l.pa_alloc_ref_count(self._h, block)

    def ref_counts(self) -> list:
        return [self._l.pa_alloc_ref_count(self._h, b) for b in range(self.num_blocks)]

    def context_len(self, seq_id: int) -> int:
        return self._l.pa_alloc_context_len(self._h, seq_id)

    def num_table_blocks(self, seq_id: int) -> int:
        return self._l.pa_alloc_num_table_blocks(self._h, seq_id)

    def free_list(self) -> list:
        out = np.empty(max(self.num_blocks, 1), np.int32)
        n = self._l.pa_alloc_free_list(self._h, out.ctypes.data, out.shape[0])
        return out[:n].tolist()

    def set_swap_space(self, num_blocks: int, free_order: Optional[Sequence[int]] = None) -> None:
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if order.shape != (num_blocks,):
                raise PagedKVError(PA_ERR_INVALID, "free_order must hold num_blocks entries")
        _check(self._l.pa_alloc_set_swap_space(self._h, num_blocks, None if order is None else order.ctypes.data),
               "pa_alloc_set_swap_space")
        self.num_swap_blocks = num_blocks

    def _swap(self, fn, seq_id: int, what: str) -> np.ndarray:
        n = max(self.num_table_blocks(seq_id), 1)
        pairs = np.empty((n, 2), np.int64)
        got = ctypes.c_int32(0)
        _check(fn(self._h, seq_id, pairs.ctypes.data, n, ctypes.byref(got)), what)
        return pairs[:got.value]

    def swap_out(self, seq_id: int) -> np.ndarray:
        """Move a sequence's table to swap blocks; returns (device, swap) pairs int64 [M, 2]."""
        return self._swap(self._l.pa_alloc_swap_out, seq_id, "pa_alloc_swap_out")

    def swap_in(self, seq_id: int) -> np.ndarray:
        """Move a swapped-out sequence back to device blocks; returns (swap, device) pairs."""
        return self._swap(self._l.pa_alloc_swap_in, seq_id, "pa_alloc_swap_in")

    def num_free_swap(self) -> int:
        return self._l.pa_alloc_num_free_swap(self._h)

    def swap_free_list(self) -> list:
        cap = max(getattr(self, "num_swap_blocks", 0), 1)
        out = np.empty(cap, np.int32)
        n = self._l.pa_alloc_swap_free_list(self._h, out.ctypes.data, cap)
        return out[:min(n, cap)].tolist()

    def seq_table(self, seq_id: int) -> list:
        """The sequence's table as stored (swap block ids while it is swapped out)."""
        n = self._l.pa_alloc_seq_table(self._h, seq_id, None, 0)
        if n < 0:
            raise PagedKVError(PA_ERR_INVALID, f"unknown sequence {seq_id}")
        out = np.empty(max(n, 1), np.int32)
        self._l.pa_alloc_seq_table(self._h, seq_id, out.ctypes.data, n)
        return out[:n].tolist()

    def is_swapped(self, seq_id: int) -> bool:
        r = self._l.pa_alloc_is_swapped(self._h, seq_id)
        if r < 0:
            raise PagedKVError(PA_ERR_INVALID, f"unknown sequence {seq_id}")
        return bool(r)

    def enable_prefix_caching(self) -> None:
        _check(self._l.pa_alloc_enable_prefix_caching(self._h), "pa_alloc_enable_prefix_caching")

    def add_seq_cached(self, seq_id: int, tokens, extra_key: int = 0) -> int:
        """New sequence for a prompt of int32 token ids, reusing its indexed
        leading blocks; returns the number of leading tokens already cached."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        got = ctypes.c_int32(0)
        _check(self._l.pa_alloc_add_seq_cached(self._h, seq_id, t.ctypes.data if t.size else None, t.shape[0],
                                               int(extra_key), ctypes.byref(got)), "pa_alloc_add_seq_cached")
        return got.value

    def prefix_hits(self, tokens, extra_key: int = 0) -> list:
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        out = np.empty(max(1, t.shape[0] // self.block_size), np.int32)
        n = self._l.pa_alloc_prefix_hits(self._h, t.ctypes.data if t.size else None, t.shape[0], int(extra_key),
                                         out.ctypes.data, out.shape[0])
        if n < 0:
            raise PagedKVError(PA_ERR_INVALID, "pa_alloc_prefix_hits: " + self._l.pa_last_error().decode())
        return out[:n].tolist()

    def admit(self, seq_ids, lengths, tokens=None, extra_keys=None, out_slots: Optional[np.ndarray] = None):
        """pa_alloc_admit: returns (slots int64 [sum(lengths)] with -1 inside cached
        prefixes, cached-prefix length per prompt). ``tokens`` is one int32
        array of all prompts' ids back to back, or None for plain admission.
        If a prompt does not fit, the error is raised with ``admitted`` (the
        count that went in) and ``slots`` set on it."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
        n = ids.shape[0]
        total = int(lens.sum())
        slots = np.empty(max(total, 1), np.int64) if out_slots is None else out_slots
        cached = np.zeros(max(n, 1), np.int32)
        tok = None if tokens is None else np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        if tok is not None and tok.shape[0] != total:
            raise PagedKVError(PA_ERR_INVALID, "tokens must hold sum(lengths) ids")
        ext = None if extra_keys is None else np.ascontiguousarray(np.asarray(extra_keys, dtype=np.int64))
        got = ctypes.c_int32(0)
        rc = self._l.pa_alloc_admit(self._h, ids.ctypes.data, n, None if tok is None or not tok.size else tok.ctypes.data,
                                    lens.ctypes.data, None if ext is None else ext.ctypes.data,
                                    _np_ptr(slots, np.int64), cached.ctypes.data, ctypes.byref(got))
        if rc != PA_OK:
            try:
                _check(rc, "pa_alloc_admit")
            except PagedKVError as e:
                e.admitted, e.slots = got.value, slots[:total]
                raise
        return slots[:total], cached[:n].tolist()

    def num_cached_blocks(self) -> int:
        return self._l.pa_alloc_num_cached_blocks(self._h)

    def cached_blocks(self) -> list:
        return [b for b in range(self.num_blocks) if self._l.pa_alloc_block_is_cached(self._h, b) == 1]

    def set_watermark(self, fraction: float) -> None:
        _check(self._l.pa_alloc_set_watermark(self._h, fraction), "pa_alloc_set_watermark")

    def can_allocate(self, n: int) -> bool:
        return bool(self._l.pa_alloc_can_allocate(self._h, n))
