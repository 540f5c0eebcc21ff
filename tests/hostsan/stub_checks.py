"""Checks that need the stub device layer (tests/hostsan/stub_device.cpp): with
every argument valid the C-ABI front end reaches its launchers, and the
parameters it hands them are the ones the arguments describe.  Run only against
the sanitizer build, by tests/test_host_sanitizer.py; never collected on its own."""
import ctypes
import math

import pytest

import exact_attention_64_amd as ea
from exact_attention_64_amd import _lib

FAKE = 0x10000
LOG2E = 1.0 / math.log(2.0)


def stub():
    L = ea.lib()
    L.stub_field.argtypes = [ctypes.c_char_p]
    L.stub_field.restype = ctypes.c_double
    L.stub_scratch.restype = ctypes.c_void_p
    return L


def field(name):
    return stub().stub_field(name.encode())


def fwd_args(**kw):
    a = _lib.AttnArgs()
    a.dtype, a.causal = ea.ATTN_BF16, 0
    a.b, a.s_q, a.s_k, a.h, a.d, a.h_kv = 2, 300, 333, 4, 128, 0
    a.q = a.k = a.v = a.o = a.lse = FAKE
    st = _lib.I64x3(300 * 4 * 128, 4 * 128, 128)
    a.q_stride = a.o_stride = st
    a.k_stride = a.v_stride = _lib.I64x3(333 * 4 * 128, 4 * 128, 128)
    a.softmax_scale = 0.125
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("scale", [0.125, -0.25, 0.0])
def test_fwd_reaches_prefill_launcher_with_scale_folded(scale):
    L = stub()
    n0 = L.stub_launches()
    assert L.attn_fwd(ctypes.byref(fwd_args(softmax_scale=scale, causal=1)), None) == 0
    assert L.stub_launches() == n0 + 1 and L.stub_last_kind() == 1
    assert field("causal") == 1 and field("split") == 0 and field("n_splits") == 1
    assert (field("b"), field("h"), field("s_q"), field("s_k"), field("d")) == (2, 4, 300, 333, 128)
    assert field("neg_q") == (scale < 0) and field("zero_q") == (scale == 0)
    want = 1.0 if scale == 0 else abs(scale) * LOG2E
    assert abs(field("scale_log2") - want) <= 1e-6 * want
    assert field("qs1") == 4 * 128


def test_decode_and_split_routing():
    L = stub()
    # one query row, no shared K/V heads: the decode kernel
    a = fwd_args(s_q=1, q_stride=_lib.I64x3(4 * 128, 4 * 128, 128), o_stride=_lib.I64x3(4 * 128, 4 * 128, 128))
    assert L.attn_fwd(ctypes.byref(a), None) == 0 and L.stub_last_kind() == 2
    assert L.attn_fwd_splitkv(ctypes.byref(a), 7, FAKE, FAKE, None) == 0
    assert L.stub_last_kind() == 2 and field("split") == 1 and field("n_splits") == 7
    assert field("o") == 0 and field("lse") == 0 and field("o_part") == FAKE
    # shared K/V heads (4 query heads per K/V head): the packed prefill kernel
    a.h_kv = 1
    assert L.attn_fwd_splitkv(ctypes.byref(a), 3, FAKE, FAKE, None) == 0
    assert L.stub_last_kind() == 1 and field("g") == 4 and field("n_splits") == 3


def test_small_head_routing():
    L = stub()
    # d <= 32 with both lengths <= 256: the persistent small-head kernel; longer
    # sequences, one query row or a split pass: the other kernels
    for d, s_q, s_k, kind in ((16, 150, 150, 5), (32, 256, 256, 5), (16, 257, 100, 1), (32, 100, 257, 1),
                              (64, 100, 100, 1), (16, 1, 100, 2)):
        a = fwd_args(s_q=s_q, s_k=s_k, d=d, q_stride=_lib.I64x3(s_q * 4 * d, 4 * d, d),
                     k_stride=_lib.I64x3(s_k * 4 * d, 4 * d, d), v_stride=_lib.I64x3(s_k * 4 * d, 4 * d, d),
                     o_stride=_lib.I64x3(s_q * 4 * d, 4 * d, d))
        assert L.attn_fwd(ctypes.byref(a), None) == 0 and L.stub_last_kind() == kind, (d, s_q, s_k)
        if kind == 5:
            assert field("s_q") == s_q and field("s_k") == s_k and field("split") == 0
    a = fwd_args(s_q=150, s_k=150, d=16, q_stride=_lib.I64x3(150 * 64, 64, 16), k_stride=_lib.I64x3(150 * 64, 64, 16),
                 v_stride=_lib.I64x3(150 * 64, 64, 16), o_stride=_lib.I64x3(150 * 64, 64, 16))
    assert L.attn_fwd_splitkv(ctypes.byref(a), 3, FAKE, FAKE, None) == 0 and L.stub_last_kind() == 1


def test_combine_params():
    L = stub()
    st = _lib.I64x3(5 * 16 * 64, 16 * 64, 64)
    assert L.attn_combine(9, 2, 16, 5, 64, FAKE, FAKE, ea.ATTN_FP16, FAKE, st, None, None) == 0
    assert L.stub_last_kind() == 3 and field("n_splits") == 9 and field("d") == 64 and field("os0") == 5 * 16 * 64


def test_paged_params():
    L = stub()
    a = _lib.AttnPagedArgs()
    a.dtype, a.causal = ea.ATTN_BF16, 1
    a.b, a.s_q, a.h, a.h_kv, a.d = 3, 2, 8, 2, 128
    a.q = a.k_cache = a.v_cache = a.o = FAKE
    a.block_table = a.seqlens_k = FAKE
    a.q_stride = a.o_stride = _lib.I64x3(2 * 8 * 128, 8 * 128, 128)
    a.k_stride = a.v_stride = _lib.I64x3(64 * 2 * 128, 2 * 128, 128)
    a.num_blocks, a.block_size = 40, 64
    a.block_table_stride, a.max_blocks, a.max_seqlen_k = 16, 13, 800
    a.softmax_scale = 0.1
    assert L.attn_fwd_paged(ctypes.byref(a), None) == 0
    assert L.stub_last_kind() == 1 and field("paged") == 1 and field("lbs") == 6
    assert field("num_blocks") == 40 and field("bt_stride") == 16 and field("s_k") == 800 and field("g") == 4


def test_bwd_delta_routing():
    L = stub()
    a = _lib.AttnBwdArgs()
    a.dtype, a.causal = ea.ATTN_FP16, 1
    a.b, a.s_q, a.s_k, a.h, a.h_kv, a.d = 2, 64, 80, 4, 2, 64
    for name in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "delta"):
        setattr(a, name, FAKE)
    for name in ("q_stride", "o_stride", "dout_stride", "dq_stride"):
        setattr(a, name, _lib.I64x3(64 * 4 * 64, 4 * 64, 64))
    for name in ("k_stride", "v_stride", "dk_stride", "dv_stride"):
        setattr(a, name, _lib.I64x3(80 * 2 * 64, 2 * 64, 64))
    a.softmax_scale = -0.3
    assert L.attn_bwd(ctypes.byref(a), None) == 0
    assert L.stub_last_kind() == 4 and field("delta") == FAKE and field("g") == 2 and field("causal") == 1
    assert abs(field("scale") + 0.3) < 1e-7 and abs(field("scale_log2") + 0.3 * LOG2E) < 1e-6
    a.delta = None
    assert L.attn_bwd(ctypes.byref(a), None) == -1
    assert L.attn_bwd_noalloc(ctypes.byref(a), None) == 0
    assert field("delta") == L.stub_scratch()
    big = a
    big.s_q = (1 << 22) // 8 + 1  # b*h*s_q just over the static buffer
    assert L.attn_bwd_noalloc(ctypes.byref(big), None) == -10


def test_sizes_at_the_limits_do_not_overflow():
    # the largest shapes the checks admit: every int64 product on the way to the
    # grid-size checks must stay defined (UBSan aborts on signed overflow)
    L = stub()
    for b, h, s in ((1, 1 << 24, 1 << 24), (1 << 24, 1, 1 << 24), (4096, 4096, 1 << 24)):
        a = fwd_args(b=b, h=h, s_q=s, s_k=s, d=128)
        L.attn_fwd(ctypes.byref(a), None)
        L.attn_fwd_splitkv(ctypes.byref(a), 256, FAKE, FAKE, None)
        n = ctypes.c_int32()
        L.attn_num_splits_for(b, h, s, s, 128, 256, ctypes.byref(n))
        st = _lib.I64x3(0, 0, 0)
        L.attn_combine(256, b, h, s, 128, FAKE, FAKE, ea.ATTN_BF16, FAKE, st, None, None)
