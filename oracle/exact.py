"""Float64 CPU oracle for exact attention forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module. It shares no code with the GPU library and imports nothing from it.

What is computed (the standard attention of "LLM Lab Notes 07: Why FlashAttention
Is Fast", §2 "Code Walkthrough": the score matrix S = Q·Kᵀ/√d is formed in full,
softmax is taken along the key axis, and the result multiplies V; §3.3 "Online
Softmax" states that the fused kernel reaches this same result up to rounding):

    S_ij  = scale · Σ_c q_ic k_jc                 (per batch and head, all i, j)
    m_i   = max_j S_ij
    P_ij  = exp(S_ij − m_i) / Σ_j' exp(S_ij' − m_i)
    O_i   = Σ_j P_ij v_j
    LSE_i = m_i + ln Σ_j exp(S_ij − m_i)

The maximum is subtracted before exponentiating, as the log-sum-exp trick in the
split-reduction reply of flash-attention issue #1248 ("where is flash decoding
second stage (reduce) code?") prescribes.

Readings taken where the pages are silent:
  * causal masking is bottom-right aligned: query i sees key j iff
    j <= i + (s_k - s_q); with s_q == s_k this is the usual lower triangle;
  * a query row that sees no key has O = 0 and LSE = -inf;
  * LSE is a natural logarithm taken over the scaled scores;
  * all arithmetic is float64 on the exact fp16/bf16 input values;
  * the scale is an explicit argument (the pages use 1/sqrt(d)).

Layouts: q is (b, s_q, h, d); k and v are (b, s_k, h_kv, d) with h a multiple of
h_kv; O is (b, s_q, h, d); LSE is (b, h, s_q).  Query head hh attends with K/V
head hh // (h / h_kv): h_kv = h is plain multi-head attention, and a smaller
h_kv lets consecutive query heads share one K/V head (the several "q heads" over
one K tile asked about in issue #1248).

Paged K/V cache ("LLM Lab Notes 07", §5 "Engineering Takeaways", names the paged
KV cache as the standard companion of the fused kernel for long contexts and
gives no layout; the plainest reading is taken): the cache is an array of
fixed-size blocks, (num_blocks, block_size, h_kv, d); sequence bi has
seqlens_k[bi] keys, key j of it living in physical block block_table[bi, j //
block_size] at slot j % block_size.  Gathering a sequence's keys in order gives
the contiguous K of the definition above, and each sequence is attended over
its own key count (the causal rule uses that count as s_k).
"""
from __future__ import annotations

import numpy as np


def visible_mask(s_q: int, s_k: int, causal: bool, rows=None) -> np.ndarray:
    """Boolean (len(rows), s_k) matrix: True where query ``rows[r]`` may see key j.

    Causal rule (bottom-right aligned): j <= i + s_k - s_q.
    """
    rows = np.arange(s_q) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(s_k, dtype=np.int64)
    if not causal:
        return np.ones((rows.size, s_k), dtype=bool)
    return j[None, :] <= rows[:, None] + (s_k - s_q)


def softmax_rows(S: np.ndarray):
    """Row-wise softmax of a score array whose masked entries are -inf.

    The row maximum is subtracted before ``exp`` (log-sum-exp trick). Returns
    ``(P, m, lse)`` with ``lse = m + ln(sum exp(S - m))``. A row with no finite
    entry gives P = 0, m = -inf and lse = -inf.
    """
    if S.shape[-1] == 0:  # an empty key range
        m = np.full(S.shape[:-1], -np.inf)
        return np.zeros(S.shape), m, m.copy()
    m = S.max(axis=-1)
    finite = np.isfinite(m)
    m_shift = np.where(finite, m, 0.0)
    E = np.exp(S - m_shift[..., None])  # masked entries: exp(-inf) = 0
    l = E.sum(axis=-1)
    has = l > 0
    P = np.divide(E, l[..., None], out=np.zeros_like(E), where=has[..., None])
    lse = np.full(l.shape, -np.inf)
    np.add(m_shift, np.log(l, out=np.zeros_like(l), where=has), out=lse, where=has)
    return P, m, lse


def _attend(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float,
            mask: np.ndarray):
    """One materialised attention over leading batch axes.

    qh (..., n, d), kh and vh (..., s_k, d), mask broadcastable to (..., n, s_k).
    Returns O (..., n, d) and LSE (..., n).
    """
    S = scale * np.matmul(qh, np.swapaxes(kh, -1, -2))
    S = np.where(mask, S, -np.inf)
    P, _, lse = softmax_rows(S)
    return np.matmul(P, vh), lse


def _as_f64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def kv_head_of(h: int, h_kv: int) -> np.ndarray:
    """K/V head index of every query head: hh // (h / h_kv)."""
    if h_kv < 1 or h % h_kv:
        raise ValueError(f"h = {h} is not a multiple of h_kv = {h_kv}")
    return np.arange(h) // (h // h_kv)


def attention(q, k, v, scale: float, causal: bool):
    """Exact attention forward. Returns (O (b,s_q,h,d), LSE (b,h,s_q)), float64.

    The score matrix of one batch entry (all heads) is materialised at a time.
    """
    q, k, v = _as_f64(q, k, v)
    b, s_q, h, d = q.shape
    s_k = k.shape[1]
    kv = kv_head_of(h, k.shape[2])
    mask = visible_mask(s_q, s_k, causal)
    O = np.zeros((b, s_q, h, d))
    LSE = np.zeros((b, h, s_q))
    for bi in range(b):
        o, lse = _attend(q[bi].transpose(1, 0, 2), k[bi][:, kv].transpose(1, 0, 2),
                         v[bi][:, kv].transpose(1, 0, 2), scale, mask)
        O[bi] = o.transpose(1, 0, 2)
        LSE[bi] = lse
    return O, LSE


def attention_rows(q, k, v, scale: float, causal: bool, rows):
    """Exact attention for selected query rows only.

    ``rows`` is a list of ``h`` equally long index lists (one per head; the same
    rows are used for every batch entry). Returns O (b, h, n, d) and LSE (b, h, n),
    each row computed over its full visible key set.
    """
    q, k, v = _as_f64(q, k, v)
    b, s_q, h, d = q.shape
    s_k = k.shape[1]
    kv = kv_head_of(h, k.shape[2])
    n = len(rows[0])
    O = np.zeros((b, h, n, d))
    LSE = np.zeros((b, h, n))
    for hi in range(h):
        r = np.asarray(rows[hi], dtype=np.int64)
        mask = visible_mask(s_q, s_k, causal, r)
        for bi in range(b):
            o, lse = _attend(q[bi, r, hi, :], k[bi, :, kv[hi], :], v[bi, :, kv[hi], :], scale, mask)
            O[bi, hi] = o
            LSE[bi, hi] = lse
    return O, LSE


def split_bounds(s_k: int, n: int):
    """Balanced contiguous key ranges: split i covers [floor(i·s_k/n), floor((i+1)·s_k/n))."""
    return [((i * s_k) // n, ((i + 1) * s_k) // n) for i in range(n)]


def attention_split(q, k, v, scale: float, causal: bool, bounds):
    """Per-split attention for flash-decoding (issue #1248, the split/reduce thread).

    For each key range ``[lo, hi)`` in ``bounds`` the definition above is applied to
    those keys alone (the causal rule still uses absolute key indices). Each O_i is
    normalised within its own split. Returns O_parts (n, b, h, s_q, d) and
    LSE_parts (n, b, h, s_q); a row that sees no key of a split gets O_i = 0 and
    LSE_i = -inf.
    """
    q, k, v = _as_f64(q, k, v)
    b, s_q, h, d = q.shape
    s_k = k.shape[1]
    kv = kv_head_of(h, k.shape[2])
    full = visible_mask(s_q, s_k, causal)
    n = len(bounds)
    O = np.zeros((n, b, h, s_q, d))
    LSE = np.zeros((n, b, h, s_q))
    for si, (lo, hi) in enumerate(bounds):
        mask = full[:, lo:hi]
        for bi in range(b):
            o, lse = _attend(q[bi].transpose(1, 0, 2), k[bi, lo:hi][:, kv].transpose(1, 0, 2),
                             v[bi, lo:hi][:, kv].transpose(1, 0, 2), scale, mask)
            O[si, bi] = o
            LSE[si, bi] = lse
    return O, LSE


def combine(o_parts, lse_parts):
    """Split reduction of issue #1248: LSE = log Σ_i exp(LSE_i), O = Σ_i exp(LSE_i − LSE)·O_i.

    The maximum of the LSE_i is subtracted first (the reply notes the kernel repeats
    the log-sum-exp trick here). o_parts (n, ..., d), lse_parts (n, ...). If every
    LSE_i of a row is -inf the row gets O = 0 and LSE = -inf.
    """
    o_parts, lse_parts = _as_f64(o_parts, lse_parts)
    M = lse_parts.max(axis=0)
    finite = np.isfinite(M)
    M_shift = np.where(finite, M, 0.0)
    w = np.exp(lse_parts - M_shift[None])  # -inf splits weigh 0
    tot = w.sum(axis=0)
    lse = np.full(M.shape, -np.inf)
    np.add(M_shift, np.log(tot, out=np.zeros_like(tot), where=finite), out=lse, where=finite)
    scale = np.exp(lse_parts - np.where(finite, lse, 0.0)[None])
    scale = np.where(finite[None], scale, 0.0)
    O = (scale[..., None] * o_parts).sum(axis=0)
    return O, lse


def gather_paged(cache, table_row, length: int, block_size: int):
    """Keys 0..length-1 of one sequence from a paged cache, in order: key j is
    slot j % block_size of physical block table_row[j // block_size].
    cache (num_blocks, block_size, h_kv, d) -> (length, h_kv, d)."""
    j = np.arange(int(length))
    return np.asarray(cache)[np.asarray(table_row, dtype=np.int64)[j // block_size], j % block_size]


def attention_paged(q, k_cache, v_cache, block_table, seqlens_k, scale: float, causal: bool):
    """Exact attention over a paged K/V cache with a key count per sequence.

    Sequence bi attends over its seqlens_k[bi] keys gathered by ``gather_paged``,
    through ``attention`` (so the causal rule is j <= i + seqlens_k[bi] - s_q and a
    sequence with no visible key gets O = 0, LSE = -inf). Returns
    (O (b,s_q,h,d), LSE (b,h,s_q)), float64.
    """
    q = np.asarray(q, dtype=np.float64)
    b, s_q, h, d = q.shape
    bs = np.asarray(k_cache).shape[1]
    O = np.zeros((b, s_q, h, d))
    LSE = np.zeros((b, h, s_q))
    for bi in range(b):
        n = int(seqlens_k[bi])
        k = gather_paged(k_cache, block_table[bi], n, bs)[None]
        v = gather_paged(v_cache, block_table[bi], n, bs)[None]
        o, lse = attention(q[bi:bi + 1], k, v, scale, causal)
        O[bi] = o[0]
        LSE[bi] = lse[0]
    return O, LSE


def attention_split_paged(q, k_cache, v_cache, block_table, seqlens_k, scale: float,
                          causal: bool, n: int):
    """Per-split partials over a paged cache: split i of sequence bi covers that
    sequence's keys split_bounds(seqlens_k[bi], n)[i]. Returns O_parts
    (n, b, h, s_q, d) and LSE_parts (n, b, h, s_q), as ``attention_split``."""
    q = np.asarray(q, dtype=np.float64)
    b, s_q, h, d = q.shape
    bs = np.asarray(k_cache).shape[1]
    O = np.zeros((n, b, h, s_q, d))
    LSE = np.zeros((n, b, h, s_q))
    for bi in range(b):
        sk = int(seqlens_k[bi])
        k = gather_paged(k_cache, block_table[bi], sk, bs)[None]
        v = gather_paged(v_cache, block_table[bi], sk, bs)[None]
        o, lse = attention_split(q[bi:bi + 1], k, v, scale, causal, split_bounds(sk, n))
        O[:, bi] = o[:, 0]
        LSE[:, bi] = lse[:, 0]
    return O, LSE
