"""CPU checks of the C-ABI library: it loads, exports every symbol the header
declares, its struct mirror matches the C layout, argument validation returns the
documented status before anything is launched, and the split heuristic behaves.

None of these calls reaches a kernel launch: every argument set below fails a
host-side check first (fake pointers are never dereferenced).
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import exact_attention_64_amd as ea
from exact_attention_64_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:attn_status|const char \*)\s*(attn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == set(ea.EXPORTS), names
    L = ea.lib()
    for n in names:
        assert hasattr(L, n), n


def test_probe_library_exports_every_declared_symbol():
    from exact_attention_64_amd import _probe
    text = open(os.path.join(ROOT, "include", "attn_probe.h")).read()
    names = sorted(set(re.findall(r"^\s*int32_t\s+(attn_\w+)\s*\(", text, re.M)))
    assert set(names) == set(_probe.EXPORTS), names
    L = _probe.lib()
    for n in names:
        assert hasattr(L, n), n
    # host-side checks, nothing launched
    assert L.attn_probe_read(None, 1024, 1024, 1024, FAKE, 1, None) == -1
    assert L.attn_probe_read(FAKE, 1000, 1000, 1000, FAKE, 1, None) == -3   # not a multiple of 16
    assert L.attn_probe_read(FAKE, 1024, 512, 256, FAKE, 1, None) == -3     # chunk > stride
    assert L.attn_probe_read(FAKE, 1024, 48, 64, FAKE, 1, None) == -3       # bytes not whole chunks
    assert L.attn_probe_read(FAKE + 8, 1024, 1024, 1024, FAKE, 1, None) == -5
    assert L.attn_probe_read(FAKE, 1024, 1024, 1024, FAKE, -2, None) == -3
    assert L.attn_probe_grid(-1) == -3 and L.attn_probe_grid(37) == 37
    assert L.attn_probe_mfma(None, 10, 1, FAKE, None) == -1
    assert L.attn_probe_mfma(FAKE, 0, 1, FAKE, None) == -3
    assert L.attn_probe_clock(None, 100, None) == -1
    assert L.attn_probe_clock(FAKE, 0, None) == -3
    assert L.attn_probe_clock(FAKE, (1 << 31) + 1, None) == -3
    assert L.attn_probe_rates(None, None) == -1


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stddef.h>
#include <stdio.h>
#include "attn.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(attn_args), offsetof(attn_args, b),
         offsetof(attn_args, q), offsetof(attn_args, lse), offsetof(attn_args, q_stride),
         offsetof(attn_args, o_stride), offsetof(attn_args, softmax_scale),
         offsetof(attn_args, h_kv), sizeof(attn_status));
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    A = _lib.AttnArgs
    want = [ctypes.sizeof(A), A.b.offset, A.q.offset, A.lse.offset, A.q_stride.offset,
            A.o_stride.offset, A.softmax_scale.offset, A.h_kv.offset, 4]
    assert got == want


def test_paged_struct_layout_matches_c(tmp_path):
    src = tmp_path / "paged.c"
    fields = ["b", "h_kv", "q", "q_stride", "k_cache", "v_cache", "k_stride", "v_stride", "num_blocks",
              "block_size", "block_table", "block_table_stride", "max_blocks", "seqlens_k", "max_seqlen_k",
              "o", "o_stride", "lse", "softmax_scale"]
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"attn.h\"\nint main(void) {\n"
                   '  printf("%zu\\n", sizeof(attn_paged_args));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(attn_paged_args, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "paged"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    A = _lib.AttnPagedArgs
    assert got == [ctypes.sizeof(A)] + [getattr(A, f).offset for f in fields]


def _paged(**kw):
    a = _lib.AttnPagedArgs()
    a.dtype, a.causal = _lib.ATTN_BF16, 0
    a.b, a.s_q, a.h, a.h_kv, a.d = 2, 4, 8, 2, 128
    a.q = a.k_cache = a.v_cache = a.o = a.lse = FAKE
    a.block_table = a.seqlens_k = FAKE
    a.q_stride = _lib.I64x3(4 * 8 * 128, 8 * 128, 128)
    a.k_stride = a.v_stride = _lib.I64x3(64 * 2 * 128, 2 * 128, 128)
    a.num_blocks, a.block_size = 10, 64
    a.block_table_stride, a.max_blocks = 4, 4
    a.max_seqlen_k = 256
    a.o_stride = a.q_stride
    a.softmax_scale = 0.125
    for k, v in kw.items():
        setattr(a, k, v)
    return a


PAGED_BAD = [
    ("null_table", dict(block_table=None), -1),
    ("null_seqlens", dict(seqlens_k=None), -1),
    ("null_cache", dict(v_cache=None), -1),
    ("dtype", dict(dtype=3), -2),
    ("max_seqlen_0", dict(max_seqlen_k=0), -3),
    ("max_seqlen_beyond_table", dict(max_seqlen_k=257), -3),
    ("block_size_not_pow2", dict(block_size=48), -3),
    ("block_size_16", dict(block_size=16, max_seqlen_k=64), -3),
    ("table_stride_short", dict(block_table_stride=3), -3),
    ("no_blocks", dict(num_blocks=0), -3),
    ("h_kv_not_divisor", dict(h_kv=3), -3),
    ("headdim_32", dict(d=32), -4),
    ("misaligned_table", dict(block_table=FAKE + 2), -5),
    ("misaligned_cache", dict(k_cache=FAKE + 8), -5),
    ("cache_stride_not_mult8", dict(k_stride=_lib.I64x3(64 * 2 * 128, 2 * 128 + 4, 128)), -5),
    ("scale_nan", dict(softmax_scale=float("nan")), -6),
]


@pytest.mark.parametrize("name,kw,code", PAGED_BAD, ids=[b[0] for b in PAGED_BAD])
def test_paged_validation(name, kw, code):
    a = _paged(**kw)
    assert ea.lib().attn_fwd_paged(ctypes.byref(a), None) == code
    assert ea.lib().attn_fwd_splitkv_paged(ctypes.byref(a), 2, FAKE, FAKE, None) == code


def test_paged_split_count_and_partials_checked():
    L = ea.lib()
    a = _paged()
    assert L.attn_fwd_splitkv_paged(ctypes.byref(a), 0, FAKE, FAKE, None) == -7
    assert L.attn_fwd_splitkv_paged(ctypes.byref(a), 257, FAKE, FAKE, None) == -7
    assert L.attn_fwd_splitkv_paged(ctypes.byref(a), 2, None, FAKE, None) == -1
    assert L.attn_fwd_splitkv_paged(ctypes.byref(a), 2, FAKE + 4, FAKE, None) == -5
    a2 = _paged(max_seqlen_k=5)   # at most 5 splits
    assert L.attn_fwd_splitkv_paged(ctypes.byref(a2), 6, FAKE, FAKE, None) == -7
    assert L.attn_fwd_paged(None, None) == -1
    n = ctypes.c_int32()
    assert L.attn_num_splits_paged(1, 8, 2, 1, 100, 32, 0, ctypes.byref(n)) == -4
    assert L.attn_num_splits_paged(1, 8, 3, 1, 100, 128, 0, ctypes.byref(n)) == -3
    assert L.attn_num_splits_paged(1, 8, 2, 1, 100, 128, 0, None) == -1


def _args(**kw):
    a = _lib.AttnArgs()
    a.dtype, a.causal = _lib.ATTN_BF16, 0
    a.b, a.s_q, a.s_k, a.h, a.d = 2, 64, 64, 4, 128
    a.q = a.k = a.v = a.o = FAKE
    a.lse = FAKE
    s = _lib.I64x3(64 * 4 * 128, 4 * 128, 128)
    a.q_stride = a.k_stride = a.v_stride = a.o_stride = s
    a.softmax_scale = 0.125
    for k, v in kw.items():
        setattr(a, k, v)
    return a


BAD = [
    ("null_q", dict(q=None), -1),
    ("null_k", dict(k=None), -1),
    ("null_o", dict(o=None), -1),
    ("dtype", dict(dtype=7), -2),
    ("b0", dict(b=0), -3),
    ("s_k0", dict(s_k=0), -3),
    ("h_neg", dict(h=-1), -3),
    ("s_q_huge", dict(s_q=(1 << 24) + 1), -3),
    ("headdim_8", dict(d=8), -4),
    ("headdim_96", dict(d=96), -4),
    ("headdim_256", dict(d=256), -4),
    ("misaligned_q", dict(q=FAKE + 8), -5),
    ("misaligned_o", dict(o=FAKE + 2), -5),
    ("stride_not_mult8", dict(k_stride=_lib.I64x3(8 * 64 * 128, 4 * 128 + 4, 128)), -5),
    ("stride_negative", dict(v_stride=_lib.I64x3(-64 * 4 * 128, 4 * 128, 128)), -5),
    ("h_kv_negative", dict(h_kv=-1), -3),
    ("h_kv_above_h", dict(h_kv=8), -3),
    ("h_kv_not_divisor", dict(h_kv=3), -3),
    ("scale_nan", dict(softmax_scale=float("nan")), -6),
    ("scale_inf", dict(softmax_scale=float("inf")), -6),
]


@pytest.mark.parametrize("name,kw,code", BAD, ids=[b[0] for b in BAD])
def test_fwd_validation(name, kw, code):
    a = _args(**kw)
    assert ea.lib().attn_fwd(ctypes.byref(a), None) == code


def test_fwd_null_args():
    assert ea.lib().attn_fwd(None, None) == -1


@pytest.mark.parametrize("n,code", [(0, -7), (-3, -7), (257, -7), (65, -7)])
def test_splitkv_split_range(n, code):
    a = _args(s_k=64)
    assert ea.lib().attn_fwd_splitkv(ctypes.byref(a), n, ctypes.c_void_p(FAKE),
                                     ctypes.c_void_p(FAKE), None) == code


def test_splitkv_null_partials_and_alignment():
    a = _args()
    L = ea.lib()
    assert L.attn_fwd_splitkv(ctypes.byref(a), 2, None, ctypes.c_void_p(FAKE), None) == -1
    assert L.attn_fwd_splitkv(ctypes.byref(a), 2, ctypes.c_void_p(FAKE + 4),
                              ctypes.c_void_p(FAKE), None) == -5
    # o / o_stride are not used by the split kernel: a NULL o is accepted by validation
    # (the call then stops at an invalid dtype, still before any launch)
    b = _args(o=None, dtype=5)
    assert L.attn_fwd_splitkv(ctypes.byref(b), 2, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                              None) == -2


def test_combine_validation():
    L = ea.lib()
    s = (ctypes.c_int64 * 3)(16 * 128, 16 * 128, 128)
    F = ctypes.c_void_p(FAKE)
    assert L.attn_combine(4, 1, 16, 1, 128, None, F, 1, F, s, F, None) == -1
    assert L.attn_combine(4, 1, 16, 1, 128, F, F, 3, F, s, F, None) == -2
    assert L.attn_combine(4, 0, 16, 1, 128, F, F, 1, F, s, F, None) == -3
    assert L.attn_combine(4, 1, 16, 1, 48, F, F, 1, F, s, F, None) == -4
    assert L.attn_combine(4, 1, 16, 1, 128, ctypes.c_void_p(FAKE + 4), F, 1, F, s, F, None) == -5
    assert L.attn_combine(0, 1, 16, 1, 128, F, F, 1, F, s, F, None) == -7
    assert L.attn_combine(300, 1, 16, 1, 128, F, F, 1, F, s, F, None) == -7


def test_status_strings():
    for code in range(-10, 1):
        text = ea.status_str(code)
        assert text and text != "unknown status"
    assert ea.status_str(-42) == "unknown status"


def test_num_splits_device_error():
    n = ctypes.c_int32(0)
    assert ea.lib().attn_num_splits(1, 16, 1, 32768, 128, 999, ctypes.byref(n)) == -8


# --------------------------------------------------------- heuristic ----

def test_heuristic_no_split_with_enough_work():
    # issue #1248: when the work-groups of one split already cover the compute
    # units, the heuristic does not split.  8 batches x 48 heads with a few
    # query rows: 384 work-groups on 256 compute units.
    for s_q in (4, 10):
        assert ea.attn_num_splits_for(8, 48, s_q, 4096, 128, 256) == 1
    assert ea.attn_num_splits_for(4, 32, 512, 512, 128, 256) == 1
    # a single query row packs four heads per work-group: 8 x 128 heads give
    # 256 work-groups, 8 x 48 only 96, which the heuristic splits three ways
    assert ea.attn_num_splits_for(8, 128, 1, 4096, 128, 256) == 1
    assert ea.attn_num_splits_for(8, 48, 1, 4096, 128, 256) == 3


def test_heuristic_splits_small_decode():
    n = ea.attn_num_splits_for(1, 16, 1, 32768, 128, 256)
    assert 16 <= n <= 256
    # split count never exceeds what keeps >= 64 keys per split, nor the cap
    assert ea.attn_num_splits_for(1, 1, 1, 100, 128, 256) <= 2
    assert ea.attn_num_splits_for(1, 1, 1, 10 ** 6, 128, 1024) <= 256


def test_heuristic_monotone_in_work():
    prev = 10 ** 9
    for bh in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024):
        n = ea.attn_num_splits_for(1, bh, 1, 65536, 128, 256)
        assert n <= prev
        prev = n
    assert prev == 1


def test_heuristic_validation():
    n = ctypes.c_int32()
    L = ea.lib()
    assert L.attn_num_splits_for(1, 1, 1, 10, 128, 256, None) == -1
    assert L.attn_num_splits_for(0, 1, 1, 10, 128, 256, ctypes.byref(n)) == -3
    assert L.attn_num_splits_for(1, 1, 1, 10, 100, 256, ctypes.byref(n)) == -4
    assert L.attn_num_splits_for(1, 1, 1, 10, 128, 0, ctypes.byref(n)) == -8


# ---------------------------------------------------------------- backward ----

def test_bwd_struct_layout_matches_c(tmp_path):
    fields = ["b", "h_kv", "d", "q", "dout", "q_stride", "dout_stride", "lse", "dq", "dv",
              "dq_stride", "dv_stride", "delta", "softmax_scale"]
    src = tmp_path / "layout_bwd.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"attn.h\"\nint main(void) {\n"
                   "  printf(\"%zu\", sizeof(attn_bwd_args));\n"
                   + "".join(f"  printf(\" %zu\", offsetof(attn_bwd_args, {f}));\n" for f in fields)
                   + "  printf(\"\\n\");\n  return 0;\n}\n")
    exe = tmp_path / "layout_bwd"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    A = _lib.AttnBwdArgs
    assert got == [ctypes.sizeof(A)] + [getattr(A, f).offset for f in fields]


def _bwd(**kw):
    a = _lib.AttnBwdArgs()
    a.dtype, a.causal = ea.ATTN_BF16, 0
    a.b, a.s_q, a.s_k, a.h, a.h_kv, a.d = 2, 64, 64, 4, 0, 64
    for name in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "delta"):
        setattr(a, name, FAKE)
    st = _lib.I64x3(64 * 4 * 64, 4 * 64, 64)
    for name in ("q_stride", "k_stride", "v_stride", "o_stride", "dout_stride", "dq_stride",
                 "dk_stride", "dv_stride"):
        setattr(a, name, st)
    a.softmax_scale = 0.125
    for key, val in kw.items():
        if key.endswith("_stride"):
            val = _lib.I64x3(*val)
        setattr(a, key, val)
    return a


BWD_CASES = [
    ("null_q", dict(q=None), -1), ("null_dout", dict(dout=None), -1), ("null_lse", dict(lse=None), -1),
    ("null_delta", dict(delta=None), -1), ("null_dk", dict(dk=None), -1),
    ("bad_dtype", dict(dtype=7), -2), ("zero_b", dict(b=0), -3), ("zero_s_k", dict(s_k=0), -3),
    ("h_kv_not_divisor", dict(h_kv=3), -3), ("h_kv_above_h", dict(h_kv=8), -3),
    ("headdim_96", dict(d=96), -4), ("headdim_8", dict(d=8), -4),
    ("misaligned_dv", dict(dv=FAKE + 8), -5), ("misaligned_delta", dict(delta=FAKE + 2), -5),
    ("stride_not_8", dict(dout_stride=(64 * 4 * 64, 4 * 64, 60)), -5),
    ("negative_stride", dict(dq_stride=(-8, 256, 64)), -5),
    ("nan_scale", dict(softmax_scale=float("nan")), -6), ("inf_scale", dict(softmax_scale=float("inf")), -6),
]


@pytest.mark.parametrize("name,kw,code", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_validation(name, kw, code):
    a = _bwd(**kw)
    assert ea.lib().attn_bwd(ctypes.byref(a), None) == code


NOALLOC_CASES = [c for c in BWD_CASES if "delta" not in c[0]]


@pytest.mark.parametrize("name,kw,code", NOALLOC_CASES, ids=[c[0] for c in NOALLOC_CASES])
def test_bwd_noalloc_validation(name, kw, code):
    # the allocation-free backward runs the same checks (its delta is ignored)
    a = _bwd(**kw)
    assert ea.lib().attn_bwd_noalloc(ctypes.byref(a), None) == code


def test_bwd_noalloc_scratch_limit_and_ignored_delta():
    L = ea.lib()
    assert L.attn_bwd_noalloc(None, None) == -1
    # b*h*s_q above the static buffer (2^22 rows of delta): ATTN_E_SCRATCH before
    # any device work; at the limit the host goes on to the device check
    big = _bwd(b=2, h=4, s_q=(1 << 19) + 1, s_k=64)
    assert L.attn_bwd_noalloc(ctypes.byref(big), None) == -10
    import torch
    if not torch.cuda.is_available():
        at = _bwd(b=2, h=4, s_q=1 << 19, s_k=64, delta=None)
        assert L.attn_bwd_noalloc(ctypes.byref(at), None) == -8
        assert L.attn_bwd_noalloc(ctypes.byref(_bwd(delta=None)), None) == -8
        assert L.attn_bwd(ctypes.byref(_bwd(delta=None)), None) == -1


def test_bwd_null_args_and_no_device():
    assert ea.lib().attn_bwd(None, None) == -1
    # every argument valid: the host reaches the device check (no GPU here, or a
    # GPU that is not gfx950) only when no device is usable
    import torch
    if not torch.cuda.is_available():
        assert ea.lib().attn_bwd(ctypes.byref(_bwd()), None) == -8
