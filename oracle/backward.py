"""Float64 CPU oracle for the gradient of exact attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module. It shares no code with the GPU library and imports nothing from it.

The forward pass is the standard attention of "LLM Lab Notes 07: Why
FlashAttention Is Fast" (§2 "Code Walkthrough"): O = softmax(scale·Q·Kᵀ)·V per
batch entry and head, softmax over the visible keys.  flash-attention issue
#1335 ("2.6.3 is faster than 2.7.0 for flash-attn v2 CUDA fwd/bwd") times the
backward of that function without describing its algorithm, so the oracle is
the plain definition of the gradient: given an upstream gradient dO of O, the
vector-Jacobian product of the forward with respect to Q, K and V, written out
by the chain rule through the materialised matrices (no tiling, no recomputation
tricks):

    S    = scale · Q Kᵀ            (masked entries −inf)
    P    = softmax_rows(S)          (the forward's probabilities)
    O    = P V
    dV   = Pᵀ dO
    dP   = dO Vᵀ
    δ_i  = Σ_c dO_ic O_ic  ( = Σ_j P_ij dP_ij, the softmax Jacobian's row term)
    dS   = P ∘ (dP − δ 1ᵀ)
    dQ   = scale · dS K
    dK   = scale · dSᵀ Q

LSE is treated as an auxiliary output with no upstream gradient.  With shared
K/V heads (h_kv < h, query head hh reading K/V head hh // (h / h_kv)), a K/V
head's dK and dV are the sums over the query heads that read it.  A query row
that sees no key has P = 0, so it contributes nothing and gets dQ = 0 and δ = 0.
"""
from __future__ import annotations

import numpy as np

from . import exact as _fwd


def attention_bwd(q, k, v, dout, scale: float, causal: bool):
    """Gradient of exact attention.  q, dout (b,s_q,h,d); k, v (b,s_k,h_kv,d).

    Returns float64 (dq (b,s_q,h,d), dk (b,s_k,h_kv,d), dv (b,s_k,h_kv,d),
    delta (b,h,s_q)), delta being δ_i = Σ_c dO_ic O_ic.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    b, s_q, h, d = q.shape
    s_k, h_kv = k.shape[1], k.shape[2]
    kv = _fwd.kv_head_of(h, h_kv)
    mask = _fwd.visible_mask(s_q, s_k, causal)
    dq = np.zeros_like(q)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    delta = np.zeros((b, h, s_q))
    for bi in range(b):
        for hh in range(h):
            qh, kh, vh, doh = q[bi, :, hh], k[bi, :, kv[hh]], v[bi, :, kv[hh]], do[bi, :, hh]
            S = np.where(mask, scale * (qh @ kh.T), -np.inf)
            P, _, _ = _fwd.softmax_rows(S)
            O = P @ vh
            dP = doh @ vh.T
            dl = (doh * O).sum(-1)
            dS = P * (dP - dl[:, None])
            dq[bi, :, hh] = scale * (dS @ kh)
            dk[bi, :, kv[hh]] += scale * (dS.T @ qh)
            dv[bi, :, kv[hh]] += P.T @ doh
            delta[bi, hh] = dl
    return dq, dk, dv, delta


def attention_bwd_dq_rows(q, k, v, dout, scale: float, causal: bool, head: int, rows):
    """dQ and δ of the given query rows of one head (all batch entries), for
    shapes too long to materialise: each row needs only its own scores.

    Returns (dq (b, len(rows), d), delta (b, len(rows))), float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    s_q, h = q.shape[1], q.shape[2]
    s_k, h_kv = k.shape[1], k.shape[2]
    hk = int(_fwd.kv_head_of(h, h_kv)[head])
    mask = _fwd.visible_mask(s_q, s_k, causal, rows)
    b = q.shape[0]
    dq = np.zeros((b, rows.size, q.shape[3]))
    delta = np.zeros((b, rows.size))
    for bi in range(b):
        qh = np.asarray(q[bi, rows, head], dtype=np.float64)
        doh = np.asarray(dout[bi, rows, head], dtype=np.float64)
        kh = np.asarray(k[bi, :, hk], dtype=np.float64)
        vh = np.asarray(v[bi, :, hk], dtype=np.float64)
        S = np.where(mask, scale * (qh @ kh.T), -np.inf)
        P, _, _ = _fwd.softmax_rows(S)
        dP = doh @ vh.T
        dl = (doh * (P @ vh)).sum(-1)
        dq[bi] = scale * ((P * (dP - dl[:, None])) @ kh)
        delta[bi] = dl
    return dq, delta


def attention_bwd_dkdv_cols(q, k, v, dout, scale: float, causal: bool, kv_head: int, cols,
                            row_chunk: int = 1024):
    """dK and dV of the given keys of one K/V head (all batch entries).

    Every query row of every query head that reads ``kv_head`` contributes, so
    each row's softmax normaliser and δ are needed: rows are processed in chunks
    of ``row_chunk``, each chunk's full score rows materialised, and only the
    requested key columns kept.  Returns (dk (b, len(cols), d), dv (b, len(cols), d)).
    """
    cols = np.asarray(cols, dtype=np.int64)
    b, s_q, h, d = q.shape
    s_k, h_kv = k.shape[1], k.shape[2]
    heads = np.nonzero(_fwd.kv_head_of(h, h_kv) == kv_head)[0]
    dk = np.zeros((b, cols.size, d))
    dv = np.zeros((b, cols.size, d))
    for bi in range(b):
        kh = np.asarray(k[bi, :, kv_head], dtype=np.float64)
        vh = np.asarray(v[bi, :, kv_head], dtype=np.float64)
        for hh in heads:
            for r0 in range(0, s_q, row_chunk):
                rows = np.arange(r0, min(s_q, r0 + row_chunk))
                qh = np.asarray(q[bi, rows, hh], dtype=np.float64)
                doh = np.asarray(dout[bi, rows, hh], dtype=np.float64)
                mask = _fwd.visible_mask(s_q, s_k, causal, rows)
                S = np.where(mask, scale * (qh @ kh.T), -np.inf)
                P, _, _ = _fwd.softmax_rows(S)
                dl = (doh * (P @ vh)).sum(-1)
                Pc = P[:, cols]
                dSc = Pc * (doh @ vh[cols].T - dl[:, None])
                dk[bi] += scale * (dSc.T @ qh)
                dv[bi] += Pc.T @ doh
    return dk, dv
