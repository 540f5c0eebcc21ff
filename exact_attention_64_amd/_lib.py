"""ctypes binding of ``libattn.so`` (the gfx950 C ABI declared in include/attn.h).

Argument marshalling only: torch tensors are turned into device pointers,
element strides and the current HIP stream, outputs are allocated with torch
when the caller does not pass them, and every status code is turned into an
exception.  All attention arithmetic runs in the HIP kernels; if the library is
not built this module raises instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_FP16, ATTN_BF16 = 0, 1
ATTN_MAX_SPLITS = 256
_DTYPE_CODE = {torch.float16: ATTN_FP16, torch.bfloat16: ATTN_BF16}
_CODE_DTYPE = {v: k for k, v in _DTYPE_CODE.items()}

STATUS = {0: "ATTN_OK", -1: "ATTN_E_NULL", -2: "ATTN_E_DTYPE", -3: "ATTN_E_SHAPE",
          -4: "ATTN_E_HEADDIM", -5: "ATTN_E_LAYOUT", -6: "ATTN_E_SCALE", -7: "ATTN_E_SPLITS",
          -8: "ATTN_E_DEVICE", -9: "ATTN_E_LAUNCH", -10: "ATTN_E_SCRATCH"}

I64x3 = ctypes.c_int64 * 3

# Every symbol include/attn.h declares.
EXPORTS = ("attn_fwd", "attn_num_splits", "attn_num_splits_for", "attn_num_splits_kv",
           "attn_num_splits_kv_for", "attn_fwd_splitkv", "attn_combine", "attn_fwd_paged",
           "attn_fwd_splitkv_paged", "attn_num_splits_paged", "attn_bwd", "attn_bwd_noalloc", "attn_status_str")


class AttnArgs(ctypes.Structure):
    """Mirror of ``attn_args``."""

    _fields_ = [
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("b", ctypes.c_int64), ("s_q", ctypes.c_int64), ("s_k", ctypes.c_int64),
        ("h", ctypes.c_int64), ("d", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("q_stride", I64x3), ("k_stride", I64x3), ("v_stride", I64x3), ("o_stride", I64x3),
        ("softmax_scale", ctypes.c_float),
        ("h_kv", ctypes.c_int64),
    ]


class AttnPagedArgs(ctypes.Structure):
    """Mirror of ``attn_paged_args`` in include/attn.h."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("b", ctypes.c_int64), ("s_q", ctypes.c_int64), ("h", ctypes.c_int64),
        ("h_kv", ctypes.c_int64), ("d", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("q_stride", I64x3),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_stride", I64x3), ("v_stride", I64x3),
        ("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int64),
        ("max_blocks", ctypes.c_int64),
        ("seqlens_k", ctypes.c_void_p), ("max_seqlen_k", ctypes.c_int64),
        ("o", ctypes.c_void_p), ("o_stride", I64x3), ("lse", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
    ]


class AttnBwdArgs(ctypes.Structure):
    """Mirror of ``attn_bwd_args`` in include/attn.h."""
    _fields_ = [
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("b", ctypes.c_int64), ("s_q", ctypes.c_int64), ("s_k", ctypes.c_int64),
        ("h", ctypes.c_int64), ("h_kv", ctypes.c_int64), ("d", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p),
        ("q_stride", I64x3), ("k_stride", I64x3), ("v_stride", I64x3), ("o_stride", I64x3),
        ("dout_stride", I64x3),
        ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dq_stride", I64x3), ("dk_stride", I64x3), ("dv_stride", I64x3),
        ("delta", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
    ]


class AttnError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


_lib = None
_lock = threading.Lock()


def lib():
    """Load ``libattn.so`` once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build the HIP library first "
                    "(python -m exact_attention_64_amd.build)")
            L = ctypes.CDLL(LIB_PATH)
            P = ctypes.POINTER
            L.attn_fwd.argtypes = [P(AttnArgs), ctypes.c_void_p]
            L.attn_fwd.restype = ctypes.c_int32
            L.attn_num_splits.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int, P(ctypes.c_int32)]
            L.attn_num_splits.restype = ctypes.c_int32
            L.attn_num_splits_for.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int32, P(ctypes.c_int32)]
            L.attn_num_splits_for.restype = ctypes.c_int32
            L.attn_num_splits_kv.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int, P(ctypes.c_int32)]
            L.attn_num_splits_kv.restype = ctypes.c_int32
            L.attn_num_splits_kv_for.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int32, P(ctypes.c_int32)]
            L.attn_num_splits_kv_for.restype = ctypes.c_int32
            L.attn_fwd_splitkv.argtypes = [P(AttnArgs), ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
            L.attn_fwd_splitkv.restype = ctypes.c_int32
            L.attn_combine.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p, P(ctypes.c_int64), ctypes.c_void_p,
                                       ctypes.c_void_p]
            L.attn_combine.restype = ctypes.c_int32
            L.attn_fwd_paged.argtypes = [P(AttnPagedArgs), ctypes.c_void_p]
            L.attn_fwd_paged.restype = ctypes.c_int32
            L.attn_fwd_splitkv_paged.argtypes = [P(AttnPagedArgs), ctypes.c_int32, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p]
            L.attn_fwd_splitkv_paged.restype = ctypes.c_int32
            L.attn_num_splits_paged.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int, P(ctypes.c_int32)]
            L.attn_num_splits_paged.restype = ctypes.c_int32
            L.attn_bwd.argtypes = [P(AttnBwdArgs), ctypes.c_void_p]
            L.attn_bwd.restype = ctypes.c_int32
            L.attn_bwd_noalloc.argtypes = [P(AttnBwdArgs), ctypes.c_void_p]
            L.attn_bwd_noalloc.restype = ctypes.c_int32
            L.attn_status_str.argtypes = [ctypes.c_int32]
            L.attn_status_str.restype = ctypes.c_char_p
            _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise AttnError(status, lib().attn_status_str(status).decode())


def status_str(status: int) -> str:
    return lib().attn_status_str(status).decode()


def _stream_ptr(t: torch.Tensor, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _bshd(name, t: torch.Tensor):
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D (b, s, h, d), got shape {tuple(t.shape)}")
    if t.stride(3) != 1:
        raise ValueError(f"{name} must have a contiguous last (head-dim) dimension")
    return I64x3(t.stride(0), t.stride(1), t.stride(2))


def make_args(q, k, v, softmax_scale=None, causal=False, out=None, lse=None) -> AttnArgs:
    """Fill ``attn_args`` from (b, s, h, d) tensors (no copies)."""
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share dtype float16 or bfloat16")
    b, s_q, h, d = q.shape
    if k.dim() != 4:
        raise ValueError("k and v must be 4-D (b, s_k, h_kv, d)")
    s_k, h_kv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (b, s_k, h_kv, d) or tuple(v.shape) != (b, s_k, h_kv, d) or h_kv < 1 or h % h_kv != 0:
        raise ValueError(f"k and v must be (b, s_k, h_kv, d) = ({b}, s_k, h_kv, {d}) with h_kv dividing {h}")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    a = AttnArgs()
    a.dtype = _DTYPE_CODE[q.dtype]
    a.causal = 1 if causal else 0
    a.b, a.s_q, a.s_k, a.h, a.d = b, s_q, s_k, h, d
    a.q, a.k, a.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    a.q_stride, a.k_stride, a.v_stride = _bshd("q", q), _bshd("k", k), _bshd("v", v)
    if out is not None:
        if tuple(out.shape) != (b, s_q, h, d) or out.dtype != q.dtype:
            raise ValueError("out must match q's shape and dtype")
        a.o = out.data_ptr()
        a.o_stride = _bshd("out", out)
    if lse is not None:
        if tuple(lse.shape) != (b, h, s_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 (b, h, s_q) tensor")
        a.lse = lse.data_ptr()
    a.softmax_scale = float(softmax_scale)
    a.h_kv = h_kv
    return a


def attn_fwd(q, k, v, softmax_scale=None, causal=False, out=None, lse=None, stream=None,
             return_lse=True):
    """Fused exact attention forward. Returns (O, LSE) (LSE None if not requested)."""
    b, s_q, h, d = q.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None and return_lse:
        lse = torch.empty((b, h, s_q), dtype=torch.float32, device=q.device)
    a = make_args(q, k, v, softmax_scale, causal, out, lse)
    _check(lib().attn_fwd(ctypes.byref(a), _stream_ptr(q, stream)))
    return out, lse


class FwdPlan:
    """A fused-forward call with its arguments marshalled once: for callers that
    run the same shapes and buffers repeatedly (issue #1335's point: at small
    shapes host-side work per call is what costs time).  ``plan()`` only calls
    the C ABI with the stored ``attn_args`` on the stored stream; the tensors
    must stay alive and keep their storage (new values may be copied in)."""

    def __init__(self, q, k, v, softmax_scale=None, causal=False, out=None, lse=None, stream=None):
        b, s_q, h, d = q.shape
        self.out = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
        self.lse = torch.empty((b, h, s_q), dtype=torch.float32, device=q.device) if lse is None else lse
        self._keep = (q, k, v)
        self._args = make_args(q, k, v, softmax_scale, causal, self.out, self.lse)
        self._ref = ctypes.byref(self._args)
        self._stream = _stream_ptr(q, stream)
        self._fn = lib().attn_fwd

    def __call__(self):
        st = self._fn(self._ref, self._stream)
        if st != 0:
            _check(st)
        return self.out, self.lse


def attn_num_splits(b, h, s_q, s_k, d, device=None, h_kv=0) -> int:
    n = ctypes.c_int32(0)
    dev = torch.cuda.current_device() if device is None else int(device)
    _check(lib().attn_num_splits_kv(b, h, h_kv, s_q, s_k, d, dev, ctypes.byref(n)))
    return n.value


def attn_num_splits_for(b, h, s_q, s_k, d, num_cus, h_kv=0) -> int:
    n = ctypes.c_int32(0)
    _check(lib().attn_num_splits_kv_for(b, h, h_kv, s_q, s_k, d, num_cus, ctypes.byref(n)))
    return n.value


def attn_fwd_splitkv(q, k, v, num_splits=0, softmax_scale=None, causal=False, o_part=None,
                     lse_part=None, stream=None):
    """First flash-decoding stage. Returns fp32 (O_parts [n,b,h,s_q,d], LSE_parts [n,b,h,s_q])."""
    b, s_q, h, d = q.shape
    s_k = k.shape[1]
    if num_splits == 0:
        num_splits = attn_num_splits(b, h, s_q, s_k, d, q.device.index, h_kv=k.shape[2])
    if o_part is None:
        o_part = torch.empty((num_splits, b, h, s_q, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((num_splits, b, h, s_q), dtype=torch.float32, device=q.device)
    if (tuple(o_part.shape) != (num_splits, b, h, s_q, d) or not o_part.is_contiguous()
            or tuple(lse_part.shape) != (num_splits, b, h, s_q) or not lse_part.is_contiguous()
            or o_part.dtype != torch.float32 or lse_part.dtype != torch.float32):
        raise ValueError("o_part / lse_part must be dense fp32 [n,b,h,s_q,d] / [n,b,h,s_q]")
    a = make_args(q, k, v, softmax_scale, causal)
    _check(lib().attn_fwd_splitkv(ctypes.byref(a), num_splits, ctypes.c_void_p(o_part.data_ptr()),
                                  ctypes.c_void_p(lse_part.data_ptr()), _stream_ptr(q, stream)))
    return o_part, lse_part


def attn_combine(o_part, lse_part, dtype=torch.bfloat16, out=None, lse=None, stream=None,
                 return_lse=True):
    """Second flash-decoding stage. Returns (O (b,s_q,h,d) dtype, LSE (b,h,s_q) fp32)."""
    n, b, h, s_q, d = o_part.shape
    if tuple(lse_part.shape) != (n, b, h, s_q) or not (o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("o_part / lse_part must be dense [n,b,h,s_q,d] / [n,b,h,s_q]")
    if out is None:
        out = torch.empty((b, s_q, h, d), dtype=dtype, device=o_part.device)
    if lse is None and return_lse:
        lse = torch.empty((b, h, s_q), dtype=torch.float32, device=o_part.device)
    if out.dtype not in _DTYPE_CODE:
        raise TypeError("out must be float16 or bfloat16")
    ostr = _bshd("out", out)
    _check(lib().attn_combine(n, b, h, s_q, d, ctypes.c_void_p(o_part.data_ptr()),
                              ctypes.c_void_p(lse_part.data_ptr()), _DTYPE_CODE[out.dtype],
                              ctypes.c_void_p(out.data_ptr()), ostr,
                              ctypes.c_void_p(lse.data_ptr() if lse is not None else None),
                              _stream_ptr(o_part, stream)))
    return out, lse


def attn_decode(q, k, v, num_splits=0, softmax_scale=None, causal=False, stream=None):
    """Split-KV forward followed by the combine: flash-decoding end to end."""
    o_part, lse_part = attn_fwd_splitkv(q, k, v, num_splits, softmax_scale, causal, stream=stream)
    return attn_combine(o_part, lse_part, q.dtype, stream=stream)


# ------------------------------------------------------------ paged cache ----

def make_paged_args(q, k_cache, v_cache, block_table, seqlens_k, max_seqlen_k=None,
                    softmax_scale=None, causal=False, out=None, lse=None) -> AttnPagedArgs:
    """Fill ``attn_paged_args`` (no copies).

    q (b, s_q, h, d); k_cache, v_cache (num_blocks, block_size, h_kv, d) with a
    contiguous last dimension; block_table int32 (b, max_blocks) with unit column
    stride; seqlens_k int32 (b,) contiguous.  max_seqlen_k defaults to
    max_blocks * block_size (the host never reads the device-side counts).
    """
    if q.dtype not in _DTYPE_CODE or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache, v_cache must share dtype float16 or bfloat16")
    b, s_q, h, d = q.shape
    if k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[3] != d:
        raise ValueError("k_cache and v_cache must be (num_blocks, block_size, h_kv, d)")
    num_blocks, block_size, h_kv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if h_kv < 1 or h % h_kv != 0:
        raise ValueError(f"h_kv = {h_kv} must divide h = {h}")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != b \
            or block_table.stride(1) != 1:
        raise ValueError("block_table must be int32 (b, max_blocks) with unit column stride")
    if seqlens_k.dtype != torch.int32 or tuple(seqlens_k.shape) != (b,) or not seqlens_k.is_contiguous():
        raise ValueError("seqlens_k must be a contiguous int32 (b,) tensor")
    max_blocks = block_table.shape[1]
    if max_seqlen_k is None:
        max_seqlen_k = max_blocks * block_size
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    a = AttnPagedArgs()
    a.dtype = _DTYPE_CODE[q.dtype]
    a.causal = 1 if causal else 0
    a.b, a.s_q, a.h, a.h_kv, a.d = b, s_q, h, h_kv, d
    a.q, a.q_stride = q.data_ptr(), _bshd("q", q)
    a.k_cache, a.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
    a.k_stride, a.v_stride = _bshd("k_cache", k_cache), _bshd("v_cache", v_cache)
    a.num_blocks, a.block_size = num_blocks, block_size
    a.block_table, a.block_table_stride, a.max_blocks = block_table.data_ptr(), block_table.stride(0), max_blocks
    a.seqlens_k, a.max_seqlen_k = seqlens_k.data_ptr(), int(max_seqlen_k)
    if out is not None:
        if tuple(out.shape) != (b, s_q, h, d) or out.dtype != q.dtype:
            raise ValueError("out must match q's shape and dtype")
        a.o, a.o_stride = out.data_ptr(), _bshd("out", out)
    if lse is not None:
        if tuple(lse.shape) != (b, h, s_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 (b, h, s_q) tensor")
        a.lse = lse.data_ptr()
    a.softmax_scale = float(softmax_scale)
    return a


def attn_num_splits_paged(b, h, s_q, max_seqlen_k, d, device=None, h_kv=0) -> int:
    n = ctypes.c_int32(0)
    dev = torch.cuda.current_device() if device is None else int(device)
    _check(lib().attn_num_splits_paged(b, h, h_kv, s_q, max_seqlen_k, d, dev, ctypes.byref(n)))
    return n.value


def attn_fwd_paged(q, k_cache, v_cache, block_table, seqlens_k, max_seqlen_k=None, softmax_scale=None,
                   causal=False, out=None, lse=None, stream=None, return_lse=True):
    """Fused forward over a paged K/V cache. Returns (O, LSE)."""
    b, s_q, h, d = q.shape
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None and return_lse:
        lse = torch.empty((b, h, s_q), dtype=torch.float32, device=q.device)
    a = make_paged_args(q, k_cache, v_cache, block_table, seqlens_k, max_seqlen_k, softmax_scale,
                        causal, out, lse)
    _check(lib().attn_fwd_paged(ctypes.byref(a), _stream_ptr(q, stream)))
    return out, lse


def attn_fwd_splitkv_paged(q, k_cache, v_cache, block_table, seqlens_k, num_splits=0, max_seqlen_k=None,
                           softmax_scale=None, causal=False, o_part=None, lse_part=None, stream=None):
    """First flash-decoding stage over a paged cache. Returns fp32 (O_parts, LSE_parts)."""
    a = make_paged_args(q, k_cache, v_cache, block_table, seqlens_k, max_seqlen_k, softmax_scale, causal)
    b, s_q, h, d = q.shape
    if num_splits == 0:
        num_splits = attn_num_splits_paged(b, h, s_q, a.max_seqlen_k, d, q.device.index, h_kv=a.h_kv)
    if o_part is None:
        o_part = torch.empty((num_splits, b, h, s_q, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((num_splits, b, h, s_q), dtype=torch.float32, device=q.device)
    if (tuple(o_part.shape) != (num_splits, b, h, s_q, d) or not o_part.is_contiguous()
            or tuple(lse_part.shape) != (num_splits, b, h, s_q) or not lse_part.is_contiguous()
            or o_part.dtype != torch.float32 or lse_part.dtype != torch.float32):
        raise ValueError("o_part / lse_part must be dense fp32 [n,b,h,s_q,d] / [n,b,h,s_q]")
    _check(lib().attn_fwd_splitkv_paged(ctypes.byref(a), num_splits, ctypes.c_void_p(o_part.data_ptr()),
                                        ctypes.c_void_p(lse_part.data_ptr()), _stream_ptr(q, stream)))
    return o_part, lse_part


def attn_decode_paged(q, k_cache, v_cache, block_table, seqlens_k, num_splits=0, max_seqlen_k=None,
                      softmax_scale=None, causal=False, stream=None):
    """Flash-decoding over a paged cache: split-KV stage, then the combine."""
    o_part, lse_part = attn_fwd_splitkv_paged(q, k_cache, v_cache, block_table, seqlens_k, num_splits,
                                              max_seqlen_k, softmax_scale, causal, stream=stream)
    return attn_combine(o_part, lse_part, q.dtype, stream=stream)


# ---------------------------------------------------------------- backward ----

def make_bwd_args(q, k, v, out, dout, lse, dq, dk, dv, delta, softmax_scale=None,
                  causal=False) -> AttnBwdArgs:
    """Fill ``attn_bwd_args`` (no copies)."""
    if q.dtype not in _DTYPE_CODE or any(t.dtype != q.dtype for t in (k, v, out, dout, dq, dk, dv)):
        raise TypeError("q, k, v, out, dout, dq, dk, dv must share dtype float16 or bfloat16")
    b, s_q, h, d = q.shape
    if k.dim() != 4:
        raise ValueError("k and v must be 4-D (b, s_k, h_kv, d)")
    s_k, h_kv = k.shape[1], k.shape[2]
    kshape = (b, s_k, h_kv, d)
    if tuple(v.shape) != kshape or h_kv < 1 or h % h_kv != 0:
        raise ValueError(f"k and v must be (b, s_k, h_kv, d) = ({b}, s_k, h_kv, {d}) with h_kv dividing {h}")
    for name, t, shp in (("out", out, q.shape), ("dout", dout, q.shape), ("dq", dq, q.shape),
                         ("dk", dk, kshape), ("dv", dv, kshape)):
        if tuple(t.shape) != tuple(shp):
            raise ValueError(f"{name} must have shape {tuple(shp)}, got {tuple(t.shape)}")
    for name, t in (("lse", lse), ("delta", delta)):
        if t is None and name == "delta":
            continue
        if tuple(t.shape) != (b, h, s_q) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 (b, h, s_q) tensor")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    a = AttnBwdArgs()
    a.dtype = _DTYPE_CODE[q.dtype]
    a.causal = 1 if causal else 0
    a.b, a.s_q, a.s_k, a.h, a.h_kv, a.d = b, s_q, s_k, h, h_kv, d
    a.q, a.k, a.v, a.o, a.dout = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr()
    a.q_stride, a.k_stride, a.v_stride = _bshd("q", q), _bshd("k", k), _bshd("v", v)
    a.o_stride, a.dout_stride = _bshd("out", out), _bshd("dout", dout)
    a.lse = lse.data_ptr()
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.dq_stride, a.dk_stride, a.dv_stride = _bshd("dq", dq), _bshd("dk", dk), _bshd("dv", dv)
    a.delta = delta.data_ptr() if delta is not None else None
    a.softmax_scale = float(softmax_scale)
    return a


def attn_bwd(q, k, v, out, dout, lse, softmax_scale=None, causal=False, dq=None, dk=None, dv=None,
             delta=None, stream=None):
    """Gradient of exact attention: returns (dq, dk, dv) in q's dtype.

    ``out`` and ``lse`` are the forward's outputs for the same q, k, v, scale and
    causal flag; ``delta`` is the (b, h, s_q) fp32 workspace (allocated when None).
    """
    b, s_q, h, d = q.shape
    if dq is None:
        dq = torch.empty_like(q, memory_format=torch.contiguous_format)
    if dk is None:
        dk = torch.empty_like(k, memory_format=torch.contiguous_format)
    if dv is None:
        dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    if delta is None:
        delta = torch.empty((b, h, s_q), dtype=torch.float32, device=q.device)
    a = make_bwd_args(q, k, v, out, dout, lse, dq, dk, dv, delta, softmax_scale, causal)
    _check(lib().attn_bwd(ctypes.byref(a), _stream_ptr(q, stream)))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, out, dout, lse, dq, dk, dv, softmax_scale=None, causal=False, stream=None):
    """``attn_bwd`` with delta in the library's static device buffer: nothing is
    allocated, so dq, dk and dv must be given (written in place, returned)."""
    a = make_bwd_args(q, k, v, out, dout, lse, dq, dk, dv, None, softmax_scale, causal)
    _check(lib().attn_bwd_noalloc(ctypes.byref(a), _stream_ptr(q, stream)))
    return dq, dk, dv


class BwdPlan:
    """A backward call with its arguments marshalled once, like FwdPlan: ``plan()``
    only calls the C ABI with the stored ``attn_bwd_args`` on the stored stream;
    the tensors must stay alive and keep their storage (new values may be
    copied in).  Returns (dq, dk, dv)."""

    def __init__(self, q, k, v, out, dout, lse, softmax_scale=None, causal=False, dq=None, dk=None, dv=None,
                 delta=None, stream=None):
        b, s_q, h, d = q.shape
        self.dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
        self.dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
        self.dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
        self.delta = torch.empty((b, h, s_q), dtype=torch.float32, device=q.device) if delta is None else delta
        self._keep = (q, k, v, out, dout, lse)
        self._args = make_bwd_args(q, k, v, out, dout, lse, self.dq, self.dk, self.dv, self.delta,
                                   softmax_scale, causal)
        self._ref = ctypes.byref(self._args)
        self._stream = _stream_ptr(q, stream)
        self._fn = lib().attn_bwd

    def __call__(self):
        st = self._fn(self._ref, self._stream)
        if st != 0:
            _check(st)
        return self.dq, self.dk, self.dv
