"""GPU parity: the HIP kernels (through the C ABI) against the float64 CPU oracle.

Both sides get the same seeded, dtype-rounded inputs (workloads.make_qkv).
Tolerances: max-abs 5e-3 (fp16) / 2e-2 (bf16) on O, 1e-3 on LSE.  Long causal
prefill is checked on a seeded sample of query rows per head.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_attention_64_amd as ea

pytestmark = pytest.mark.gpu

TOL_O = {"fp16": 5e-3, "bf16": 2e-2}
TOL_LSE = 1e-3
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def upload(*ts):
    return [t.to(DEV) for t in ts]


def host64(*ts):
    """Exact float64 copies of the dtype-rounded inputs, for the oracle."""
    return [t.to(torch.float64).numpy() for t in ts]


def check(O, L, O_ref, L_ref, dtype, what=""):
    O = f64(O)
    L = f64(L)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(L), fin), f"{what}: -inf rows differ"
    assert np.all(L[~fin] == -np.inf)
    eo = np.abs(O - O_ref).max() if O.size else 0.0
    el = np.abs(L[fin] - L_ref[fin]).max() if fin.any() else 0.0
    assert np.all(np.isfinite(O)), f"{what}: non-finite O"
    assert eo <= TOL_O[dtype], f"{what}: max |O - O_ref| = {eo:.3e}"
    assert el <= TOL_LSE, f"{what}: max |LSE - LSE_ref| = {el:.3e}"
    return eo, el


def run_fwd(q, k, v, scale, causal):
    qd, kd, vd = upload(q, k, v)
    O, L = ea.attn_fwd(qd, kd, vd, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    return O, L


SMALL = [
    # dtype, b, s_q, s_k, h, d  -- several tiles plus ragged tails
    ("bf16", 2, 300, 333, 3, 128),
    ("fp16", 2, 300, 333, 3, 128),
    ("bf16", 1, 517, 517, 2, 64),
    ("fp16", 3, 129, 257, 2, 64),
    ("bf16", 2, 200, 161, 3, 32),
    ("fp16", 2, 97, 130, 4, 32),
    ("bf16", 2, 150, 150, 5, 16),
    ("fp16", 1, 33, 65, 3, 16),
    ("bf16", 1, 1, 700, 4, 128),   # one query row (decode shape) through the fused kernel
    ("fp16", 1, 700, 5, 2, 128),   # fewer keys than rows: causal rows at the top see nothing
    ("bf16", 2, 128, 300, 3, 128), # at most 128 rows per head: the 4-wave launch
    ("fp16", 1, 100, 90, 2, 64),   # the same with rows that see no key
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-k{c[3]}-h{c[4]}-d{c[5]}" for c in SMALL])
def test_fwd_small(case, causal):
    dt, b, s_q, s_k, h, d = case
    say("attn_fwd", case, "causal", causal, "seed 42")
    q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, dt, seed=42)
    scale = 1 / math.sqrt(d)
    O, L = run_fwd(q, k, v, scale, causal)
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, causal)
    check(O, L, O_ref, L_ref, dt, str(case))


@pytest.mark.parametrize("name", ["C1", "C2", "C3"])
def test_fwd_workloads_full(name):
    w = workloads.WORKLOADS[name]
    say("attn_fwd", name, w.note)
    q, k, v = workloads.make_workload(w)
    O, L = run_fwd(q, k, v, w.scale, w.causal)
    O_ref, L_ref = oracle.attention(*host64(q, k, v), w.scale, w.causal)
    check(O, L, O_ref, L_ref, w.dtype, name)


def test_fwd_long_causal_sampled():
    w = workloads.WORKLOADS["C5"]
    say("attn_fwd", "C5", w.note, "sampled rows", w.sample_rows)
    q, k, v = workloads.make_workload(w)
    O, L = run_fwd(q, k, v, w.scale, w.causal)
    rows = workloads.sample_rows(w.s_q, w.sample_rows, w.h, seed=42)
    O_ref, L_ref = oracle.attention_rows(*host64(q, k, v), w.scale, w.causal, rows)
    Ocpu = O.cpu()
    Lcpu = L.cpu()
    r = torch.tensor(rows)  # (h, n)
    O_s = torch.stack([Ocpu[:, r[hi], hi, :] for hi in range(w.h)], dim=1)  # (b, h, n, d)
    L_s = torch.stack([Lcpu[:, hi, r[hi]] for hi in range(w.h)], dim=1)
    check(O_s, L_s, O_ref, L_ref, w.dtype, "C5 sampled")
    # rows past the sample still obey invariants: finite, |O| bounded by max |V|
    assert torch.isfinite(Ocpu.float()).all()
    assert (Ocpu.float().abs().amax() <= v.float().abs().amax() + 1e-2)


def test_decode_workload_split_and_combine():
    w = workloads.WORKLOADS["C4"]
    q, k, v = workloads.make_workload(w)
    qd, kd, vd = upload(q, k, v)
    n = ea.attn_num_splits(w.b, w.h, w.s_q, w.s_k, w.d)
    say("attn_fwd_splitkv + attn_combine", "C4", w.note, "splits", n)
    assert n > 1
    O, L = ea.attn_decode(qd, kd, vd, num_splits=n, softmax_scale=w.scale)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(*host64(q, k, v), w.scale, False)
    check(O, L, O_ref, L_ref, w.dtype, "C4 split")
    say("attn_fwd", "C4 unsplit")
    O1, L1 = ea.attn_fwd(qd, kd, vd, softmax_scale=w.scale)
    torch.cuda.synchronize()
    check(O1, L1, O_ref, L_ref, w.dtype, "C4 fused")


SPLIT_CASES = [
    ("bf16", 1, 1, 1000, 4, 128, 7),
    ("bf16", 2, 3, 257, 3, 64, 5),
    ("fp16", 1, 130, 300, 2, 128, 3),
    ("fp16", 2, 50, 50, 16, 16, 50),    # one key per split
    ("bf16", 1, 64, 64, 2, 32, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-k{c[3]}-n{c[6]}" for c in SPLIT_CASES])
def test_splitkv_partials_and_combine(case, causal):
    dt, b, s_q, s_k, h, d, n = case
    say("attn_fwd_splitkv", case, "causal", causal)
    q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, dt, seed=7)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = upload(q, k, v)
    Op, Lp = ea.attn_fwd_splitkv(qd, kd, vd, num_splits=n, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    Op_ref, Lp_ref = oracle.attention_split(*host64(q, k, v), scale, causal, oracle.split_bounds(s_k, n))
    # partials are fp32 but built from a P rounded to the input type: same tolerance
    Lp_h = f64(Lp)
    fin = np.isfinite(Lp_ref)
    assert np.array_equal(np.isfinite(Lp_h), fin)
    assert np.abs(Lp_h[fin] - Lp_ref[fin]).max() <= TOL_LSE
    assert np.abs(f64(Op) - Op_ref).max() <= TOL_O[dt]
    say("attn_combine", case)
    O, L = ea.attn_combine(Op, Lp, q.dtype)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, causal)
    check(O, L, O_ref, L_ref, dt, f"{case} combined")
    # split + combine agrees with the fused kernel
    O1, L1 = ea.attn_fwd(qd, kd, vd, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert (O1.float() - O.float()).abs().max().item() <= TOL_O[dt]


DECODE_CASES = [
    # dtype, b, h, s_k, d, splits: one query row through the decode kernel, which
    # packs four heads of the flattened b*h into one work-group
    ("bf16", 3, 5, 3000, 128, 37),   # 15 heads: the last work-group has 3 waves
    ("fp16", 2, 3, 1500, 64, 200),   # many splits: the combine loads them in chunks
    ("bf16", 1, 7, 999, 32, 5),
    ("fp16", 2, 2, 513, 16, 64),
    ("bf16", 5, 1, 4097, 128, 1),    # work-groups span batch entries
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"{c[0]}-b{c[1]}-h{c[2]}-k{c[3]}-d{c[4]}-n{c[5]}" for c in DECODE_CASES])
def test_decode_head_groups(case):
    dt, b, h, s_k, d, n = case
    say("attn_decode", case)
    q, k, v = workloads.make_qkv(b, 1, s_k, h, d, dt, seed=11)
    scale = 1 / math.sqrt(d)
    qd, kd, vd = upload(q, k, v)
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, False)
    O, L = ea.attn_decode(qd, kd, vd, num_splits=n, softmax_scale=scale)
    torch.cuda.synchronize()
    check(O, L, O_ref, L_ref, dt, f"{case} split")
    O1, L1 = ea.attn_fwd(qd, kd, vd, softmax_scale=scale)
    torch.cuda.synchronize()
    check(O1, L1, O_ref, L_ref, dt, f"{case} fused")


def test_decode_packed_kv_cache_views():
    # K and V as strided views into one packed (b, s, 2, h, d) cache
    say("attn_decode packed KV views")
    g = torch.Generator().manual_seed(13)
    b, s_k, h, d = 2, 2049, 6, 128
    kv = torch.randn((b, s_k, 2, h, d), generator=g).to(torch.bfloat16)
    q = torch.randn((b, 1, h, d), generator=g).to(torch.bfloat16)
    k, v = kv[:, :, 0], kv[:, :, 1]
    O_ref, L_ref = oracle.attention(*host64(q, k.contiguous(), v.contiguous()), 0.1, False)
    kvd = kv.to(DEV)
    O, L = ea.attn_decode(q.to(DEV), kvd[:, :, 0], kvd[:, :, 1], softmax_scale=0.1)
    torch.cuda.synchronize()
    check(O, L, O_ref, L_ref, "bf16", "packed KV")


GQA_CASES = [
    # dtype, b, s_q, s_k, h, h_kv, d, causal: groups of h / h_kv query heads share K/V
    ("bf16", 2, 300, 333, 6, 2, 128, True),
    ("fp16", 1, 517, 517, 8, 1, 64, False),    # one K/V head for all queries
    ("bf16", 2, 100, 130, 4, 2, 32, True),
    ("fp16", 3, 50, 70, 6, 3, 16, False),
]


@pytest.mark.parametrize("case", GQA_CASES, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-k{c[3]}-h{c[4]}-kv{c[5]}-d{c[6]}" for c in GQA_CASES])
def test_shared_kv_heads(case):
    dt, b, s_q, s_k, h, h_kv, d, causal = case
    say("attn_fwd shared K/V heads", case)
    q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, dt, seed=17, h_kv=h_kv)
    scale = 1 / math.sqrt(d)
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, causal)
    O, L = run_fwd(q, k, v, scale, causal)
    check(O, L, O_ref, L_ref, dt, f"{case} fused")
    qd, kd, vd = upload(q, k, v)
    O2, L2 = ea.attn_decode(qd, kd, vd, num_splits=3, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    check(O2, L2, O_ref, L_ref, dt, f"{case} split")


PACKED_CASES = [
    # dtype, b, s_q, s_k, h, h_kv, d, causal, splits: few query rows per head with
    # h / h_kv > 1 (d >= 64), so one work-group takes all query heads of a K/V
    # head; packed rows span work-groups and heads, with ragged ends
    ("bf16", 2, 64, 1000, 16, 2, 128, True, 5),    # 512 packed rows: 2 blocks per K/V head
    ("fp16", 1, 37, 700, 14, 2, 128, False, 3),    # 259 rows: a 3-row second block
    ("bf16", 3, 40, 30, 4, 1, 64, True, 2),        # s_q > s_k: causal rows that see no key
    ("fp16", 2, 1, 2049, 32, 4, 64, False, 7),     # one row per head, 8 heads per K/V head
    ("bf16", 1, 5, 333, 12, 3, 128, True, 1),
    ("fp16", 2, 9, 64, 6, 2, 128, True, 64),       # one key per split
    ("bf16", 2, 16, 900, 12, 2, 128, True, 3),     # 96 packed rows: the 8-wave launch
    ("fp16", 1, 9, 500, 16, 2, 64, False, 2),      # 72 packed rows at d = 64
    ("bf16", 2, 16, 400, 16, 4, 128, False, 2),    # 64 packed rows: four waves of 16 rows, all full
]


@pytest.mark.parametrize("case", PACKED_CASES, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-k{c[3]}-h{c[4]}-kv{c[5]}-d{c[6]}-n{c[8]}" for c in PACKED_CASES])
def test_packed_query_heads(case):
    dt, b, s_q, s_k, h, h_kv, d, causal, n = case
    say("attn_fwd packed query heads", case)
    q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, dt, seed=23, h_kv=h_kv)
    scale = 1 / math.sqrt(d)
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, causal)
    O, L = run_fwd(q, k, v, scale, causal)
    check(O, L, O_ref, L_ref, dt, f"{case} fused")
    qd, kd, vd = upload(q, k, v)
    Op, Lp = ea.attn_fwd_splitkv(qd, kd, vd, num_splits=n, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    Op_ref, Lp_ref = oracle.attention_split(*host64(q, k, v), scale, causal, oracle.split_bounds(s_k, n))
    Lp_h = f64(Lp)
    fin = np.isfinite(Lp_ref)
    assert np.array_equal(np.isfinite(Lp_h), fin)
    assert np.abs(Lp_h[fin] - Lp_ref[fin]).max() <= TOL_LSE
    assert np.abs(f64(Op) - Op_ref).max() <= TOL_O[dt]
    O2, L2 = ea.attn_combine(Op, Lp, q.dtype)
    torch.cuda.synchronize()
    check(O2, L2, O_ref, L_ref, dt, f"{case} split")


@pytest.mark.parametrize("s_q", [1, 4, 10])
def test_multi_token_decode_48_heads(s_q):
    # issue #1248's decode setting: batch 8, 48 query heads, 1-10 new tokens
    # (here over 8 K/V heads and a 4096-key cache, bf16, d = 128)
    say("multi-token decode b=8 h=48 h_kv=8 s_k=4096 s_q", s_q)
    q, k, v = workloads.make_qkv(8, s_q, 4096, 48, 128, "bf16", seed=19, h_kv=8)
    scale = 1 / math.sqrt(128)
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, True)
    O, L = run_fwd(q, k, v, scale, True)
    check(O, L, O_ref, L_ref, "bf16", f"s_q={s_q} fused")
    qd, kd, vd = upload(q, k, v)
    O2, L2 = ea.attn_decode(qd, kd, vd, softmax_scale=scale, causal=True)
    torch.cuda.synchronize()
    check(O2, L2, O_ref, L_ref, "bf16", f"s_q={s_q} split (heuristic)")


PAGED_CASES = [
    # dtype, b, s_q, h, h_kv, d, seqlens, block_size, causal, splits
    ("bf16", 3, 1, 16, 2, 128, [1000, 0, 77], 64, False, 4),     # packed decode, an empty sequence
    ("fp16", 2, 1, 4, 4, 128, [513, 2048], 32, False, 8),       # one row per head, block = tile
    ("bf16", 2, 7, 12, 3, 64, [300, 7], 128, True, 3),          # packed multi-token, s_k == s_q
    ("fp16", 2, 300, 4, 2, 128, [333, 290], 256, True, 1),      # chunked prefill; rows with no key
    ("bf16", 1, 3, 8, 1, 128, [4096], 1024, False, 5),
    ("fp16", 3, 2, 6, 6, 64, [95, 1, 64], 32, True, 2),
    ("bf16", 3, 1, 5, 5, 64, [1000, 0, 33], 32, True, 7),       # one-row decode kernel: 64-key batches
    ("bf16", 2, 1, 3, 3, 128, [4097, 31], 64, False, 3),        # over three 32-key blocks; mixed lengths
    ("bf16", 2, 12, 12, 2, 128, [700, 300], 64, True, 2),       # 72 packed rows per K/V head: 8 waves
]


def _paged_case(case):
    dt, b, s_q, h, h_kv, d, lens, bs, causal, n = case
    q, kc, vc, table, sl = workloads.make_paged(b, s_q, h, d, dt, lens, bs, h_kv=h_kv, seed=29)
    return q, kc, vc, table, sl


@pytest.mark.parametrize("case", PAGED_CASES, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-h{c[3]}-kv{c[4]}-d{c[5]}-bs{c[7]}-n{c[9]}" for c in PAGED_CASES])
def test_paged_kv_cache(case):
    dt, b, s_q, h, h_kv, d, lens, bs, causal, n = case
    say("paged K/V cache", case)
    q, kc, vc, table, sl = _paged_case(case)
    scale = 1 / math.sqrt(d)
    O_ref, L_ref = oracle.attention_paged(*host64(q, kc, vc), table.numpy(), sl.numpy(), scale, causal)
    qd, kcd, vcd, td, sld = upload(q, kc, vc, table, sl)
    O, L = ea.attn_fwd_paged(qd, kcd, vcd, td, sld, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    check(O, L, O_ref, L_ref, dt, f"{case} fused")
    Op, Lp = ea.attn_fwd_splitkv_paged(qd, kcd, vcd, td, sld, num_splits=n, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    Op_ref, Lp_ref = oracle.attention_split_paged(*host64(q, kc, vc), table.numpy(), sl.numpy(), scale,
                                                  causal, n)
    Lp_h = f64(Lp)
    fin = np.isfinite(Lp_ref)
    assert np.array_equal(np.isfinite(Lp_h), fin)
    if fin.any():
        assert np.abs(Lp_h[fin] - Lp_ref[fin]).max() <= TOL_LSE
    assert np.abs(f64(Op) - Op_ref).max() <= TOL_O[dt]
    O2, L2 = ea.attn_combine(Op, Lp, q.dtype)
    torch.cuda.synchronize()
    check(O2, L2, O_ref, L_ref, dt, f"{case} split")


@pytest.mark.parametrize("s_q,h_kv", [(4, 2), (1, 8)])
def test_paged_unused_table_entries_are_not_read(s_q, h_kv):
    # entries past each sequence's last block hold ids far outside the cache; the
    # kernels never read them (an exact bound, not the clamp, keeps them out)
    say("paged cache, junk table tail", s_q, h_kv)
    case = ("bf16", 3, s_q, 8, h_kv, 128, [100, 64, 1], 64, True, 3)
    q, kc, vc, table, sl = _paged_case(case)
    for bi, n in enumerate(case[6]):
        used = -(-n // 64)
        table[bi, used:] = torch.tensor([10 ** 9, -5, 7 * 10 ** 8])[: table.shape[1] - used]
    scale = 0.125
    ok = table.clone()
    ok[ok < 0] = 0
    ok[ok >= kc.shape[0]] = 0
    O_ref, L_ref = oracle.attention_paged(*host64(q, kc, vc), ok.numpy(), sl.numpy(), scale, True)
    qd, kcd, vcd, td, sld = upload(q, kc, vc, table, sl)
    for n in (1, 2, 3):
        O, L = ea.attn_decode_paged(qd, kcd, vcd, td, sld, num_splits=n, softmax_scale=scale, causal=True)
        torch.cuda.synchronize()
        check(O, L, O_ref, L_ref, "bf16", f"junk tail n={n}")


def test_paged_matches_contiguous_layout():
    # a cache whose blocks hold each sequence in order (identity table) against the
    # contiguous entry points on the same tensors, packed decode and prefill
    say("paged vs contiguous")
    for (b, s_q, s_k, h, h_kv) in ((2, 1, 2048, 16, 2), (1, 130, 512, 4, 4)):
        q, k, v = workloads.make_qkv(b, s_q, s_k, h, 128, "bf16", seed=31, h_kv=h_kv)
        bs = 64
        kc = k.reshape(b * s_k // bs, bs, h_kv, 128)
        vc = v.reshape(b * s_k // bs, bs, h_kv, 128)
        table = torch.arange(b * s_k // bs, dtype=torch.int32).reshape(b, s_k // bs)
        sl = torch.full((b,), s_k, dtype=torch.int32)
        qd, kd, vd, kcd, vcd, td, sld = upload(q, k, v, kc, vc, table, sl)
        O1, L1 = ea.attn_fwd(qd, kd, vd, causal=True)
        O2, L2 = ea.attn_fwd_paged(qd, kcd, vcd, td, sld, causal=True)
        torch.cuda.synchronize()
        assert (O1.float() - O2.float()).abs().max().item() <= TOL_O["bf16"]
        assert (L1 - L2).abs().max().item() <= TOL_LSE


def test_graph_capture_replay():
    # Every entry point enqueues kernels only (no allocation, copy, memset or
    # synchronisation), so a HIP graph can capture them; each replay must equal
    # an eager call on the same inputs, bit for bit, with eager work between replays.
    say("HIP graph capture: tiny attn_fwd + split-KV decode")
    qs, ks, vs = upload(*workloads.make_qkv(2, 50, 50, 16, 16, "fp16", seed=61))
    qd, kd, vd = upload(*workloads.make_qkv(1, 1, 2048, 4, 128, "bf16", seed=62))
    O = torch.empty_like(qs)
    L = torch.empty((2, 16, 50), device=DEV)
    op = torch.empty((8, 1, 4, 1, 128), device=DEV)
    lp = torch.empty((8, 1, 4, 1), device=DEV)
    Od = torch.empty_like(qd)
    Ld = torch.empty((1, 4, 1), device=DEV)

    def run(o, l, o_part, l_part, od, ld):
        ea.attn_fwd(qs, ks, vs, 0.25, False, out=o, lse=l)
        ea.attn_fwd_splitkv(qd, kd, vd, 8, None, False, o_part=o_part, lse_part=l_part)
        ea.attn_combine(o_part, l_part, qd.dtype, out=od, lse=ld)

    run(O, L, op, lp, Od, Ld)          # first use (library load, device query) outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(O, L, op, lp, Od, Ld)
    E = [torch.empty_like(t) for t in (O, L, op, lp, Od, Ld)]
    for rep in range(4):
        new = workloads.make_qkv(2, 50, 50, 16, 16, "fp16", seed=70 + rep)
        newd = workloads.make_qkv(1, 1, 2048, 4, 128, "bf16", seed=80 + rep)
        for dst, src in zip((qs, ks, vs, qd, kd, vd), (*new, *newd)):
            dst.copy_(src.to(DEV))
        g.replay()
        torch.cuda.synchronize()
        run(*E)
        torch.cuda.synchronize()
        for got, want in zip((O, L, Od, Ld), (E[0], E[1], E[4], E[5])):
            assert torch.equal(got, want), f"replay {rep} differs from the eager call"
        if rep in (0, 3):
            O_ref, L_ref = oracle.attention(*host64(*new), 0.25, False)
            check(O, L, O_ref, L_ref, "fp16", f"graph replay {rep}")
            Od_ref, Ld_ref = oracle.attention(*host64(*newd), 1 / math.sqrt(128), False)
            check(Od, Ld, Od_ref, Ld_ref, "bf16", f"graph replay {rep} decode")


def test_combine_identical_splits_adds_ln2():
    say("attn_combine identical splits")
    g = torch.Generator().manual_seed(3)
    o = torch.randn((1, 2, 3, 5, 64), generator=g)
    lse = torch.randn((1, 2, 3, 5), generator=g) * 30
    Op = torch.cat([o, o]).to(DEV)
    Lp = torch.cat([lse, lse]).to(DEV)
    O, L = ea.attn_combine(Op, Lp, torch.float16)
    torch.cuda.synchronize()
    assert (L.cpu() - (lse[0] + math.log(2))).abs().max() < 1e-4
    err = (O.cpu().float().permute(0, 2, 1, 3) - o[0]).abs()
    assert (err <= o[0].abs() * 2.0 ** -10 + 1e-6).all()
    # all splits empty: O = 0, LSE = -inf
    Lp2 = torch.full((3, 1, 2, 5), float("-inf"), device=DEV)
    Op2 = torch.zeros((3, 1, 2, 5, 16), device=DEV)
    O2, L2 = ea.attn_combine(Op2, Lp2, torch.bfloat16)
    torch.cuda.synchronize()
    assert (O2 == 0).all() and torch.isinf(L2).all() and (L2 < 0).all()


SMALL_HEAD_CASES = [
    # dtype, b, s_q, s_k, h, h_kv, d, scale: the persistent small-head kernel
    # (d <= 32, both lengths <= 256); thousands of (b, h) items, so that every
    # work-group loops over several of them through its two LDS buffers
    ("fp16", 96, 40, 70, 32, 32, 16, None),
    ("bf16", 64, 33, 64, 48, 16, 32, None),     # shared K/V heads, a ragged query block
    ("bf16", 4, 256, 256, 8, 8, 32, None),      # eight key tiles and eight waves
    ("fp16", 8, 100, 60, 16, 16, 16, None),     # s_q > s_k: causal rows that see no key
    ("fp16", 32, 50, 31, 8, 8, 16, 0.0),        # scale 0: uniform weights over visible keys
    ("bf16", 32, 77, 45, 8, 4, 32, -0.3),       # negative scale
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", SMALL_HEAD_CASES,
                         ids=[f"{c[0]}-b{c[1]}-q{c[2]}-k{c[3]}-h{c[4]}-kv{c[5]}-d{c[6]}-s{c[7]}" for c in SMALL_HEAD_CASES])
def test_small_heads_persistent(case, causal):
    dt, b, s_q, s_k, h, h_kv, d, scale = case
    say("attn_fwd small heads", case, "causal", causal)
    q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, dt, seed=23, h_kv=h_kv)
    scale = 1 / math.sqrt(d) if scale is None else scale
    O, L = run_fwd(q, k, v, scale, causal)
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, causal)
    check(O, L, O_ref, L_ref, dt, str(case))


@pytest.mark.parametrize("d", [16, 32])
def test_small_heads_q_zero_closed_form(d):
    # P = 1 on every visible key: LSE = ln(count) exactly and O = the mean of V
    say("attn_fwd small heads Q=0", d)
    _, k, v = workloads.make_qkv(40, 90, 150, 4, d, "fp16", seed=29)
    q = torch.zeros((40, 90, 4, d), dtype=torch.float16)
    for causal in (False, True):
        O, L = run_fwd(q, k, v, 0.25, causal)
        cnt = np.array([150 if not causal else i + 60 + 1 for i in range(90)], dtype=np.float64)
        np.testing.assert_allclose(f64(L), np.broadcast_to(np.log(cnt), (40, 4, 90)), atol=1e-5)
        vm = np.stack([f64(v)[:, :int(c)].mean(1) for c in cnt], 1)  # (b, s_q, h, d)
        assert np.abs(f64(O) - vm).max() < TOL_O["fp16"]


# ------------------------------------------------------------ edge cases ----

@pytest.mark.parametrize("d", [16, 128])
def test_single_key_returns_v(d):
    say("attn_fwd single key", d)
    q, k, v = workloads.make_qkv(2, 37, 1, 3, d, "bf16", seed=5)
    O, L = run_fwd(q, k, v, 0.3, False)
    assert torch.equal(O.cpu(), v.expand(2, 37, 3, d))  # weight exactly 1
    ref = 0.3 * torch.einsum("bshd,bhd->bhs", q.double(), k[:, 0].double())
    assert (L.cpu().double() - ref).abs().max() < TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_closed_form(causal):
    say("attn_fwd Q=0", causal)
    _, k, v = workloads.make_qkv(1, 80, 200, 2, 128, "bf16", seed=9)
    q = torch.zeros((1, 80, 2, 128), dtype=torch.bfloat16)
    O, L = run_fwd(q, k, v, 0.088, causal)
    off = 200 - 80
    cnt = np.array([200 if not causal else i + off + 1 for i in range(80)], dtype=np.float64)
    np.testing.assert_allclose(f64(L)[0, 0], np.log(cnt), atol=1e-5)
    vm = torch.stack([v[0, :int(c)].double().mean(0) for c in cnt])  # (80, h, d)
    assert (O[0].cpu().double() - vm).abs().max() < 2e-2


def test_scale_zero_and_negative():
    q, k, v = workloads.make_qkv(1, 70, 90, 2, 64, "fp16", seed=11)
    for scale in (0.0, -0.125):
        for causal in (False, True):
            say("attn_fwd scale", scale, "causal", causal)
            O, L = run_fwd(q, k, v, scale, causal)
            O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, causal)
            check(O, L, O_ref, L_ref, "fp16", f"scale {scale}")


def test_large_scores_stay_finite():
    # Scores far beyond exp's range: without the max subtraction this overflows.
    say("attn_fwd large scores")
    q, k, v = workloads.make_qkv(1, 64, 300, 2, 128, "bf16", seed=13)
    scale = 8.0
    O, L = run_fwd(q, k, v, scale, False)
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, False)
    assert np.abs(L_ref).max() > 150
    # |LSE| is large here, so compare it relative to its size
    assert torch.isfinite(O).all() and torch.isfinite(L).all()
    assert np.abs(f64(O) - O_ref).max() <= TOL_O["bf16"]
    assert np.abs(f64(L) - L_ref).max() <= 1e-5 * np.abs(L_ref).max() + TOL_LSE


def test_strided_views_and_no_lse():
    say("attn_fwd packed qkv views")
    g = torch.Generator().manual_seed(17)
    b, s, h, d = 2, 190, 4, 64
    qkv = torch.randn((b, s, 3, h, d), generator=g).to(torch.bfloat16)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    qkvd = qkv.to(DEV)
    qd, kd, vd = qkvd[:, :, 0], qkvd[:, :, 1], qkvd[:, :, 2]
    out_big = torch.zeros((b, s, h, 2 * d), dtype=torch.bfloat16, device=DEV)
    out = out_big[..., :d]
    O, L = ea.attn_fwd(qd, kd, vd, softmax_scale=0.125, causal=True, out=out, return_lse=False)
    torch.cuda.synchronize()
    assert L is None
    O_ref, _ = oracle.attention(*host64(q, k, v), 0.125, True)
    assert np.abs(f64(out) - O_ref).max() <= TOL_O["bf16"]
    assert (out_big[..., d:] == 0).all()  # the other half of each row is untouched


def test_outputs_leave_guard_bands_untouched():
    say("attn_fwd guard bands")
    q, k, v = workloads.make_qkv(1, 129, 77, 3, 32, "fp16", seed=19)
    qd, kd, vd = upload(q, k, v)
    n_o = q.numel()
    o_buf = torch.full((n_o + 4096,), 7.0, dtype=torch.float16, device=DEV)
    l_buf = torch.full((3 * 129 + 1024,), 7.0, dtype=torch.float32, device=DEV)
    O = o_buf[:n_o].view(q.shape)
    L = l_buf[:3 * 129].view(1, 3, 129)
    ea.attn_fwd(qd, kd, vd, causal=True, out=O, lse=L)
    torch.cuda.synchronize()
    assert (o_buf[n_o:] == 7.0).all() and (l_buf[3 * 129:] == 7.0).all()


def test_deterministic_bitwise():
    say("attn_fwd determinism")
    q, k, v = workloads.make_qkv(2, 333, 333, 4, 128, "bf16", seed=23)
    qd, kd, vd = upload(q, k, v)
    O1, L1 = ea.attn_fwd(qd, kd, vd, causal=True)
    O2, L2 = ea.attn_fwd(qd, kd, vd, causal=True)
    Op1, Lp1 = ea.attn_fwd_splitkv(qd, kd, vd, num_splits=5)
    Op2, Lp2 = ea.attn_fwd_splitkv(qd, kd, vd, num_splits=5)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    assert torch.equal(Op1, Op2) and torch.equal(Lp1, Lp2)


def test_deterministic_bitwise_many_blocks():
    # Many work-groups per compute unit and repeated launches: a missing barrier
    # between LDS reads and the loads that overwrite the buffer shows up as runs
    # that differ.
    say("attn_fwd determinism, causal b=1 s=8192 h=32 d=128 bf16, 6 runs")
    q, k, v = workloads.make_qkv(1, 8192, 8192, 32, 128, "bf16", seed=5)
    qd, kd, vd = upload(q, k, v)
    O1, L1 = ea.attn_fwd(qd, kd, vd, causal=True)
    for _ in range(5):
        O2, L2 = ea.attn_fwd(qd, kd, vd, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_bad_head_dim_rejected():
    say("attn_fwd bad head dim on device tensors")
    q = torch.zeros((1, 8, 2, 48), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ea.AttnError) as e:
        ea.attn_fwd(q, q, q)
    assert e.value.status == -4


def test_forward_plan_matches_call():
    """FwdPlan (arguments marshalled once) runs the same kernel: bit-identical to
    attn_fwd, also after new values are copied into the planned inputs."""
    say("FwdPlan vs attn_fwd")
    q, k, v = upload(*workloads.make_qkv(2, 50, 50, 16, 16, "fp16", seed=71))
    plan = ea.FwdPlan(q, k, v, 0.25, True)
    O1, L1 = plan()
    O2, L2 = ea.attn_fwd(q, k, v, 0.25, True)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    new = workloads.make_qkv(2, 50, 50, 16, 16, "fp16", seed=72)
    for dst, src in zip((q, k, v), new):
        dst.copy_(src.to(DEV))
    O1, L1 = plan()
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(*host64(*new), 0.25, True)
    check(O1, L1, O_ref, L_ref, "fp16", "plan after new inputs")


def test_read_probe_sums_what_it_reads():
    # The benchmark's HBM read probe (include/attn_probe.h): the per-work-group
    # wrapping sums of the 32-bit words it read add up to the host's sum of the
    # same words, contiguous and strided.
    from exact_attention_64_amd import _probe
    say("read probe checksum")
    g = torch.Generator().manual_seed(1)
    x = torch.randint(-2 ** 31, 2 ** 31 - 1, (3 * 1024 * 1024 + 4,), generator=g, dtype=torch.int32)
    u = x.to(torch.int64) & 0xFFFFFFFF
    xd = x.to(DEV)
    for nb, ch, st, gr in [(x.numel() * 4 - 16, 0, 0, 0), (1 << 20, 1024, 4096, 7), (4096 * 16, 64, 192, 300)]:
        sink = _probe.probe_read(xd, nb, ch, st, grid=gr)
        torch.cuda.synchronize()
        ch, st = ch or nb, st or ch or nb
        want = int(torch.cat([u[c * st // 4: c * st // 4 + ch // 4] for c in range(nb // ch)]).sum()) % 2 ** 32
        got = int((sink.cpu().to(torch.int64) & 0xFFFFFFFF).sum()) % 2 ** 32
        assert got == want, (nb, ch, st, gr)


def test_mfma_and_clock_probes_run():
    # The benchmark's MFMA-loop and clock probes: counters advance, the shader
    # clock they give lies between 100 MHz and the device's peak (plus 5%), and the
    # constant-operand loop's accumulators hold the exact count of products
    # (every operand is 1.0: each step adds 16 per element per MFMA chain).
    from exact_attention_64_amd import _probe
    say("mfma / clock probes")
    out, ticks, fl = _probe.probe_mfma(50, False)
    torch.cuda.synchronize()
    assert ticks[0].item() > 0 and ticks[1].item() > 0
    # four chains of 4 MFMAs per step, 16 products of 1.0 each per element: the
    # final sum over 4 chains x 16 elements is 50 * 4 * 16 * 16 * 4
    assert torch.all(out == 50 * 4 * 16 * 16 * 4)
    # 16 MFMAs of 32 cycles per loop iteration; wave 0 shares its SIMD with one
    # other wave, and runs 512 (served first) to 1024 cycles per iteration
    assert 500 < ticks[0].item() / 50 < 1100
    wall_attr_hz, peak_hz = _probe.rates()
    assert wall_attr_hz > 0 and peak_hz > 0
    # the steady counter's rate, from HIP events around a probe that runs ~20 ms;
    # the cycle counter counts shader cycles
    n = int(wall_attr_hz * 20e-3)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    c = _probe.probe_clock(n)
    b.record()
    torch.cuda.synchronize()
    c0, c1, w0, w1 = c.tolist()
    assert w1 - w0 >= n and c1 > c0
    secs = a.elapsed_time(b) * 1e-3
    wall_hz = (w1 - w0) / secs
    assert 0.75 * wall_attr_hz < wall_hz < 1.25 * wall_attr_hz, (wall_hz, wall_attr_hz)
    mhz = (c1 - c0) / ((w1 - w0) / wall_hz) / 1e6
    assert 100 < mhz < peak_hz / 1e6 * 1.05, mhz
