"""Oracle: a derived bound on how far a correct paged decode computed in
float32 may lie from the exact (float64) result (TEST INFRASTRUCTURE ONLY).

Only tests use this. It shares nothing with the kernels: it states what the
rounding of a correct float32 evaluation of [PA] §5.1's split softmax can
cost, so that a test can hold the GPU result to that, next to the fixed
tolerance the workloads state.

The computation whose error is bounded ([PA] §5.1 "分块Softmax算法", steps
1-5, applied per context range and then across ranges):

* every score s_t = scale * q . K_t is a float32 sum of head_dim products;
* inside a range p, m_p = max s_t, l_p = sum exp(s_t - m_p) and the partial
  output o_p = sum exp(s_t - m_p) V_t / l_p, all in float32;
* with more than one range, o_p is stored rounded to the output type (m_p and
  l_p stay float32), and the merge takes W_p = l_p exp(m_p - m),
  out = sum_p W_p o_p / sum_p W_p in float32;
* the result is rounded to the output type.

With y the exact output, omega_t the exact softmax weights, a = sum_t omega_t
|V_t| (a column of the weighted mean of |V|; |y| <= a), Omega_p the exact
share of range p and A = sum_p Omega_p |o_p| (0 for one range), the error of
one output element is at most

    E_fp32 = (2 eps_w / (1 - eps_w) + 2 gamma(k_v) + u32) * a
    E      = E_fp32 + [P > 1] (u_o A + eta_o)
    bound  = 1.01 * (E + u_o (|y| + E) + eta_o)

where (Higham's gamma(k) = k u32 / (1 - k u32), u32 = 2^-24):

* score error: a float32 sum of depth at most k_s (= 64) over products that
  are exact or rounded once, then the scale and base-2 conversion, gives
  |ds_t| <= (gamma(k_s) + 3 u32) C_t with C_t = scale * sum_i |q_i K_t,i|
  (which also bounds |s_t|);
* weight error: exp of (s_t - m) with the maximum m itself a computed score,
  the subtraction rounded once and exp accurate to 4 u32, plus the merge's
  factor exp(m_p - m) (same reasoning) and l_p: every weight carries a
  relative error of at most eps_w = (2 gamma(k_s) + 10 u32) C_max + 8 u32; a
  ratio sum w V / sum w whose weights carry relative errors <= eps_w moves
  by at most eps_w (a + |y|) / (1 - eps_w) <= 2 eps_w a / (1 - eps_w);
* accumulation: numerator and denominator are float32 sums of depth at most
  k_v (= 512: one lane's rows of a range, the rescales, the cross-lane and
  cross-wave combine, the merge across ranges) of non-negative weights, so
  each is off by gamma(k_v) times its sum of magnitudes: 2 gamma(k_v) a,
  and the division adds u32 |y|;
* partial outputs: rounding o_p to the output type (unit roundoff u_o,
  u_o = 2^-11 for float16, 2^-8 for bfloat16, 2^-24 for float32; eta_o is
  half the type's smallest subnormal spacing) moves the merged result by at
  most u_o A + eta_o, since the merge is a convex combination of the o_p;
* final rounding: u_o |computed| + eta_o <= u_o (|y| + E) + eta_o.

The factor 1.01 covers the products of the small terms above. The depths
k_s and k_v are the reading of how a kernel may order its float32 sums;
any order of at most that depth satisfies the bound.

Unlike a fixed tolerance, the bound shrinks with the output: on long
contexts, where outputs are small, leaving out or mis-weighting one range of
the merge moves the result by far more than it allows, while the fixed
tolerance of 2e-2 + 1e-2 |y| does not see it.
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence, Tuple

import numpy as np

U32 = 2.0 ** -24
UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
SUBNORMAL_HALF_STEP = {"f32": 2.0 ** -150, "f16": 2.0 ** -25, "bf16": 2.0 ** -134}
SCORE_DEPTH = 64
SUM_DEPTH = 512


def gamma(k: int, u: float = U32) -> float:
    return k * u / (1.0 - k * u)


def dense_partitions(ctx: int, size: int) -> list:
    """Ranges [t0, t0 + n) of ``size`` tokens tiling [0, ctx) from token 0."""
    return [(t0, min(size, ctx - t0)) for t0 in range(0, ctx, size)]


def split_partitions(ctx: int, size: int, first: int) -> list:
    """Ranges tiling [0, first) and then [first, ctx), each by ``size`` tokens
    (a context whose first ``first`` tokens are handled as a run of their own)."""
    lead = [(t0, min(size, first - t0)) for t0 in range(0, min(first, ctx), size)]
    return lead + [(t0, min(size, ctx - t0)) for t0 in range(first, ctx, size)]


def decode_error_bound_one(q_h: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                           ranges: Sequence[Tuple[int, int]], out_dtype: str) -> np.ndarray:
    """Bound [d] on |computed - exact| for one query head: ``q_h`` [d], ``K``
    and ``V`` [ctx, d] (float64 values), ``ranges`` the (t0, n) context
    ranges whose partial results are merged."""
    ctx, d = K.shape
    if ctx == 0:
        return np.full(d, SUBNORMAL_HALF_STEP[out_dtype])
    u_o = UNIT_ROUNDOFF[out_dtype]
    eta = SUBNORMAL_HALF_STEP[out_dtype]
    s = scale * (K @ q_h)
    C = scale * (np.abs(K) @ np.abs(q_h))
    w = np.exp(s - s.max())
    omega = w / w.sum()
    y = omega @ V
    a = omega @ np.abs(V)
    eps_w = (2 * gamma(SCORE_DEPTH) + 10 * U32) * float(C.max()) + 8 * U32
    e = (2 * eps_w / (1 - eps_w) + 2 * gamma(SUM_DEPTH) + U32) * a
    if len(ranges) > 1:
        A = np.zeros(d)
        for t0, n in ranges:
            wp = w[t0:t0 + n]
            A += np.abs(wp @ V[t0:t0 + n]) / w.sum()          # Omega_p |o_p| = |sum_p w V| / sum w
        e = e + u_o * A + eta
    return 1.01 * (e + u_o * (np.abs(y) + e) + eta)


def decode_error_bound(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                       candidate_ranges: Iterable[Sequence[Tuple[int, int]]], out_dtype: str) -> np.ndarray:
    """Bound [Hq, d] for one sequence (``q`` [Hq, d], ``K``/``V`` [ctx, Hkv, d],
    query head h on KV head h // (Hq // Hkv)). With several candidate range
    tilings (the launch may split the context one way or another), the
    elementwise largest bound."""
    Hq, d = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    cands = [list(r) for r in candidate_ranges]
    out = np.zeros((Hq, d))
    for h in range(Hq):
        kv = h // g
        for r in cands:
            out[h] = np.maximum(out[h], decode_error_bound_one(q[h], K[:, kv], V[:, kv], scale, r, out_dtype))
    return out
