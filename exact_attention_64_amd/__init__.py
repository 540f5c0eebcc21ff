"""Exact attention forward for AMD MI355X (gfx950): fused prefill, flash-decoding
split-KV and LSE combine, over contiguous or paged K/V, as hand-written HIP kernels behind a C ABI
(include/attn.h).  This package is the thin Python binding over that ABI.

The HIP library is loaded on first use; functions raise if it is not built.
"""
from ._lib import (ATTN_BF16, ATTN_FP16, ATTN_MAX_SPLITS, EXPORTS, AttnArgs, AttnError,
                   AttnPagedArgs, AttnBwdArgs, BwdPlan, FwdPlan, attn_bwd, attn_bwd_noalloc, attn_combine, attn_decode, attn_decode_paged, attn_fwd,
                   attn_fwd_paged, attn_fwd_splitkv, attn_fwd_splitkv_paged, attn_num_splits,
                   attn_num_splits_for, attn_num_splits_paged, lib, make_args, make_paged_args, make_bwd_args,
                   status_str)

__all__ = ["ATTN_BF16", "ATTN_FP16", "ATTN_MAX_SPLITS", "EXPORTS", "AttnArgs", "AttnError",
           "AttnPagedArgs", "AttnBwdArgs", "BwdPlan", "FwdPlan", "attn_bwd", "attn_bwd_noalloc", "attn_combine", "attn_decode", "attn_decode_paged", "attn_fwd",
           "attn_fwd_paged", "attn_fwd_splitkv", "attn_fwd_splitkv_paged", "attn_num_splits",
           "attn_num_splits_for", "attn_num_splits_paged", "lib", "make_args", "make_paged_args", "make_bwd_args",
           "status_str"]
