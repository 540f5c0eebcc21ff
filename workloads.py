"""Seeded synthetic inputs and the workload table for exact attention forward.

This module holds no attention arithmetic. It only draws Q, K, V and rounds them
to the storage dtype, so that the CPU oracle and the GPU library receive the very
same bits. Both sides import it; neither imports the other.

Recipe (the pages draw plain standard-normal tensors in (b, s, h, d) layout: the
timing script in flash-attention issue #1335 "2.6.3 is faster than 2.7.0 for
flash-attn v2 CUDA fwd/bwd" seeds torch with 42 and draws q, k, v with randn;
"LLM Lab Notes 07: Why FlashAttention Is Fast" §2 draws unseeded randn tensors
of shape (batch, seq, heads, dim)):

* a CPU ``torch.Generator`` seeded with ``seed`` (42 by default) draws q, then k,
  then v, each i.i.d. N(0, 1) in float32, in (b, s, h, d) order;
* each tensor is rounded to fp16 or bf16 with round-to-nearest-even;
* the rounded tensors are what both the oracle (after an exact upcast to
  float64) and the GPU path consume.

Device RNG streams differ between vendors, so drawing on the host is the only
way both sides see the same numbers.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One attention forward problem: shapes, dtype, scale and masking."""

    name: str
    dtype: str  # "fp16" or "bf16"
    b: int
    s_q: int
    s_k: int
    h: int
    d: int
    causal: bool
    kind: str = "prefill"  # "prefill" (attn_fwd) or "decode" (split-KV + combine)
    sample_rows: int = 0  # >0: the oracle checks this many seeded rows per head
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]


# The five synthetic workloads. The first two are the (batch, seq, heads, embed)
# shapes of the issue #1335 timing script with embed 256 split over 16 heads
# (head dim 16); the third is the tutorial shape of Lab Notes 07 §2; the fourth is
# the batch-1, one-query, 16-head decode of issue #1248 with head dim 128 and a
# 32768-long cache; the fifth is a long causal prefill.
WORKLOADS = {
    "C1": Workload("C1", "fp16", 2, 50, 50, 16, 16, False,
                   note="fp16 b=2 s=50 h=16 d=16, non-causal"),
    "C2": Workload("C2", "fp16", 512, 150, 150, 16, 16, False,
                   note="fp16 b=512 s=150 h=16 d=16, non-causal"),
    "C3": Workload("C3", "bf16", 4, 512, 512, 32, 128, False,
                   note="bf16 b=4 s=512 h=32 d=128, non-causal"),
    "C4": Workload("C4", "bf16", 1, 1, 32768, 16, 128, False, kind="decode",
                   note="bf16 decode b=1 s_q=1 s_k=32768 h=16 d=128, split-KV + combine"),
    "C5": Workload("C5", "bf16", 1, 16384, 16384, 32, 128, True, sample_rows=256,
                   note="bf16 causal b=1 s=16384 h=32 d=128"),
}


def make_qkv(b: int, s_q: int, s_k: int, h: int, d: int, dtype: str, seed: int = 42, h_kv: int = 0):
    """Draw q (b,s_q,h,d), k and v (b,s_k,h_kv,d) on the CPU, rounded to ``dtype``
    (h_kv = 0 means h_kv = h).

    Returns contiguous CPU tensors of the storage dtype.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    td = DTYPES[dtype]
    hk = h_kv or h
    q = torch.randn((b, s_q, h, d), generator=g, dtype=torch.float32).to(td)
    k = torch.randn((b, s_k, hk, d), generator=g, dtype=torch.float32).to(td)
    v = torch.randn((b, s_k, hk, d), generator=g, dtype=torch.float32).to(td)
    return q, k, v


def make_dout(b: int, s_q: int, h: int, d: int, dtype: str, seed: int = 43):
    """Draw an upstream gradient dO (b, s_q, h, d) for the backward pass: i.i.d.
    N(0, 1) from its own CPU generator (seed 43, so it is independent of the
    q, k, v drawn with seed 42), rounded to ``dtype``."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn((b, s_q, h, d), generator=g, dtype=torch.float32).to(DTYPES[dtype])


def make_paged(b: int, s_q: int, h: int, d: int, dtype: str, seqlens, block_size: int,
               h_kv: int = 0, seed: int = 42, spare_blocks: int = 3):
    """Draw a query and a paged K/V cache for per-sequence key counts ``seqlens``.

    * q (b, s_q, h, d), then k_cache and v_cache (num_blocks, block_size, h_kv, d),
      each i.i.d. N(0, 1) from one CPU generator seeded with ``seed``, rounded to
      ``dtype``;
    * block_table (b, max_blocks) int32: a seeded random permutation of the
      physical blocks, so each sequence owns distinct, scattered blocks; with
      max_blocks = ceil(max(seqlens) / block_size) (at least 1), num_blocks =
      b * max_blocks + spare_blocks, and the spare blocks belong to no sequence;
    * seqlens (b,) int32 as given.

    Returns CPU tensors (q, k_cache, v_cache, block_table, seqlens).
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    td = DTYPES[dtype]
    hk = h_kv or h
    max_blocks = max(1, -(-max(seqlens) // block_size))
    num_blocks = b * max_blocks + spare_blocks
    q = torch.randn((b, s_q, h, d), generator=g, dtype=torch.float32).to(td)
    k_cache = torch.randn((num_blocks, block_size, hk, d), generator=g, dtype=torch.float32).to(td)
    v_cache = torch.randn((num_blocks, block_size, hk, d), generator=g, dtype=torch.float32).to(td)
    perm = torch.randperm(num_blocks, generator=g)[: b * max_blocks]
    block_table = perm.reshape(b, max_blocks).to(torch.int32).contiguous()
    return q, k_cache, v_cache, block_table, torch.tensor(list(seqlens), dtype=torch.int32)


def make_workload(w: Workload, seed: int = 42):
    return make_qkv(w.b, w.s_q, w.s_k, w.h, w.d, w.dtype, seed)


# Rows that every sampled check includes: tile and diagonal edges for row blocks
# of 64, 128 and 256, and the last row.
EDGE_ROWS = (0, 1, 63, 64, 127, 128, 255, 256)


def sample_rows(s_q: int, n: int, h: int, seed: int = 42):
    """Seeded query-row sample, one independent draw (without replacement) per head.

    Always contains the edge rows above (those below ``s_q``) and ``s_q - 1``.
    Returns a list of ``h`` sorted int lists.
    """
    import numpy as np

    rng = np.random.default_rng(seed)
    must = sorted({r for r in EDGE_ROWS if r < s_q} | {s_q - 1})
    out = []
    for _ in range(h):
        k = max(0, min(n, s_q) - len(must))
        pool = np.setdiff1d(np.arange(s_q), np.array(must))
        extra = rng.choice(pool, size=min(k, pool.size), replace=False) if k else []
        out.append(sorted(set(must) | {int(x) for x in extra}))
    return out
