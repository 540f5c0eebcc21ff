"""Scalar brute-force attention (test infrastructure only; tiny shapes).

The same definition as ``oracle.exact`` (standard attention of "LLM Lab Notes
07: Why FlashAttention Is Fast", §2, with the maximum subtracted before ``exp``),
written as plain Python loops over scalars with ``math.fsum`` for every sum, so a
mistake in the vectorised oracle's array handling (an axis swap, a broadcast, a
mask offset) shows up as a disagreement. Same readings: bottom-right causal
alignment, O = 0 and LSE = -inf for a row with no visible key, natural log.
"""
from __future__ import annotations

import math


def _get(x, *idx):
    for i in idx:
        x = x[i]
    return float(x)


def attention_brute(q, k, v, scale: float, causal: bool):
    """q (b,s_q,h,d), k and v (b,s_k,h_kv,d) as nested sequences or arrays; query
    head hi uses K/V head hi // (h // h_kv).

    Returns (O, LSE) as nested Python lists shaped (b,s_q,h,d) and (b,h,s_q).
    """
    b, s_q, h, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    s_k = len(k[0])
    group = h // len(k[0][0])
    O = [[[[0.0] * d for _ in range(h)] for _ in range(s_q)] for _ in range(b)]
    LSE = [[[0.0] * s_q for _ in range(h)] for _ in range(b)]
    for bi in range(b):
        for hi in range(h):
            for i in range(s_q):
                keys = [j for j in range(s_k) if (not causal) or j <= i + s_k - s_q]
                if not keys:
                    LSE[bi][hi][i] = -math.inf
                    continue
                scores = []
                for j in keys:
                    dot = math.fsum(_get(q, bi, i, hi, c) * _get(k, bi, j, hi // group, c)
                                    for c in range(d))
                    scores.append(scale * dot)
                m = max(scores)
                e = [math.exp(s - m) for s in scores]
                tot = math.fsum(e)
                for c in range(d):
                    O[bi][i][hi][c] = math.fsum(
                        e[t] * _get(v, bi, j, hi // group, c) for t, j in enumerate(keys)) / tot
                LSE[bi][hi][i] = m + math.log(tot)
    return O, LSE
