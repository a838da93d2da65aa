"""Oracle: FP8 (E4M3) and INT8 quantised K/V rows (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.

[PA] §7 "演进方向与优化空间" (compressed storage of historical blocks with
FP8/INT8) and [VM] "PagedAttention的工程实践与局限" (quantised KV values in the
blocks) name the method; the pages fix no format, so the readings here are:

* codes are OCP FP8 E4M3 ("fn": 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits, subnormals, largest finite value 448, no infinities, the
  all-ones pattern 0x7F / 0xFF is NaN);
* one float32 scale per (token, head) row: scale = max |x| / 448 (0 for an
  all-zero row); code = E4M3(clamp(x / scale, -448, 448)), rounded to nearest,
  ties to even; every code is 0 when the scale is 0;
* the arithmetic that decides the codes is float32, the precision of the
  values being stored, with the division x / scale correctly rounded (the
  plainest reading: one rounding per step); the dequantised value is
  code * scale. The scale is pinned by what it is for - the row's largest
  magnitude lands on 448 within one rounding - and the codes by the encoder's
  pins, not by restating the formula.

``encode_e4m3`` is written from the format's definition (value ranges,
exponent and mantissa fields), not from a library routine; the tests pin it to
torch's float8_e4m3fn conversion.

INT8 (the pages' other compressed format) takes the plainest symmetric
reading, with the same per-row scale so the two formats differ only in the
code: scale = max |x| / 127 (0 for an all-zero row), code = x / scale rounded
to the nearest integer, ties to even, held in [-127, 127] (two's complement
int8; -128 is never produced); the value is code * scale. float32 division,
correctly rounded, as for FP8. The tests pin the codes to torch's per-channel
int8 quantisation and the scale by what it is for.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_BIAS = 7


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e - _BIAS)
    sub = sign * (m / 8.0) * 2.0 ** (1 - _BIAS)
    v = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """E4M3 code of each float32 value with |x| <= 448, rounded to nearest,
    ties to even (the code with an even mantissa field)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))               # exact
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("encode_e4m3 takes finite values with |x| <= 448")
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    out = np.zeros(a.shape, dtype=np.int64)
    # binade of each value: 2^k <= a < 2^(k+1); below 2^-6 the spacing is the
    # subnormal step 2^-9
    with np.errstate(divide="ignore"):
        k = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    k = np.maximum(k, 1 - _BIAS)                   # subnormals share the 2^-6 binade's step
    step = np.exp2(k - 3)                          # 3 mantissa bits
    q = a / step                                   # exact (powers of two)
    lo = np.floor(q)
    frac = q - lo
    up = (frac > 0.5) | ((frac == 0.5) & (lo.astype(np.int64) % 2 == 1))
    n = (lo + up).astype(np.int64)                 # multiples of step; may reach 16 (next binade)
    val = n * step
    # re-express val as (exponent field, mantissa field)
    e_field = np.zeros_like(n)
    m_field = np.zeros_like(n)
    nz = val > 0
    kv = np.where(nz, np.floor(np.log2(np.where(nz, val, 1.0))), 0).astype(np.int64)
    is_sub = nz & (kv < 1 - _BIAS)
    is_norm = nz & ~is_sub
    e_field[is_norm] = kv[is_norm] + _BIAS
    m_field[is_norm] = np.rint(val[is_norm] / np.exp2(kv[is_norm]) * 8 - 8).astype(np.int64)
    m_field[is_sub] = np.rint(val[is_sub] / 2.0 ** (1 - _BIAS) * 8).astype(np.int64)
    out = sign | (e_field << 3) | m_field
    return out.astype(np.uint8)


def quantize_rows(x) -> "tuple[np.ndarray, np.ndarray]":
    """Quantise the last axis of ``x`` (float32 view of f32/f16/bf16 values):
    returns (uint8 codes, same shape; float32 scales, shape without the last
    axis). float32 arithmetic throughout."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = encode_e4m3(y)
    codes = np.where(scale[..., None] > 0, codes, np.uint8(0)).astype(np.uint8)
    return codes, scale


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values code * scale (scales broadcast over the last axis)."""
    return decode_e4m3(codes) * np.asarray(scales, dtype=np.float64)[..., None]


INT8_MAX = 127.0


def quantize_rows_int8(x) -> "tuple[np.ndarray, np.ndarray]":
    """INT8 codes of the last axis of ``x`` (float32 view of f32/f16/bf16
    values): returns (int8 codes, same shape; float32 scales, shape without
    the last axis). float32 arithmetic throughout."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(INT8_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)                 # one rounding
    codes = np.clip(np.rint(y), -INT8_MAX, INT8_MAX)             # nearest, ties to even (exact on float32)
    codes = np.where(scale[..., None] > 0, codes, 0).astype(np.int8)
    return codes, scale


def dequantize_int8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 values code * scale (scales broadcast over the last axis)."""
    return np.asarray(codes, dtype=np.int8).astype(np.float64) * np.asarray(scales, dtype=np.float64)[..., None]
