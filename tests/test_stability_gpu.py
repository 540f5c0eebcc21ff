"""GPU numerical-stability pins: the HIP kernels (through the C ABI) against the
float64 CPU oracle on inputs built to stress the online-softmax rescale.

"LLM Lab Notes 07: Why FlashAttention Is Fast", §3.3 Online Softmax: rescaling the
partial output by the running maximum keeps the tiled result exact; flash-attention
issue #1248 (the reduce reply) subtracts the maximum before exponentiating so that
nothing overflows.  The cases here make scores rise sharply after the first key
tile (so a stale reference would overflow fp16's P), climb steadily across the keys,
reach +-hundreds (scale 8, a large key shift), vanish (Q = 0: closed form), and
leave value columns constant (the output must reproduce them within one ulp).
Every path that runs the fused tile kernel is covered: attn_fwd at d = 16, 64 and
128, attn_fwd_splitkv with several query rows (one head per work-group and query
heads packed over a shared K/V head), the paged cache, and the one-row decode
kernel.  Tolerances: max-abs 5e-3 (fp16) / 2e-2 (bf16) on O, 1e-3 on LSE (relative
1e-5 on top where |LSE| is in the hundreds).
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
ULP = {"fp16": 2.0 ** -11, "bf16": 2.0 ** -8}  # spacing of the type in [0.5, 1)
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def host64(*ts):
    return [t.to(torch.float64).numpy() for t in ts]


def up(*ts):
    return [t.to(DEV) for t in ts]


def check(O, L, O_ref, L_ref, dtype, what, rel_lse=0.0):
    O, L = f64(O), f64(L)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(L), fin), f"{what}: -inf rows differ"
    assert np.all(np.isfinite(O)), f"{what}: non-finite O"
    eo = np.abs(O - O_ref).max()
    assert eo <= TOL_O[dtype], f"{what}: max |O - O_ref| = {eo:.3e}"
    if fin.any():
        el = np.abs(L[fin] - L_ref[fin])
        bound = TOL_LSE + rel_lse * np.abs(L_ref[fin])
        assert np.all(el <= bound), f"{what}: max |LSE - LSE_ref| = {el.max():.3e}"


# Keys planted at these positions score about this many natural units above an
# ordinary key for every query row: later keys climb past earlier references.
JUMPS = {77: 15.0, 277: 30.0, 530: 45.0}


def planted(b, s_q, s_k, h, d, dtype, seed, h_kv=0, jumps=JUMPS):
    """q with positive entries; k N(0,1) except the planted keys, which are the
    constant vector gamma (so q.k * scale ~ jump for every row); v N(0,1)."""
    q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, dtype, seed=seed, h_kv=h_kv)
    q = q.abs()
    scale = 1 / math.sqrt(d)
    mean_abs = math.sqrt(2 / math.pi)
    for j, nats in jumps.items():
        if j < s_k:
            k[:, j] = nats / (scale * mean_abs * d)
    return q, k, v, scale


def ramp(b, s_q, s_k, h, d, dtype, seed, h_kv=0, climb=30.0):
    """Scores that climb by about ``climb`` natural units from the first key to
    the last: k_j = N(0,1) + gamma * j / s_k with q positive."""
    q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, dtype, seed=seed, h_kv=h_kv)
    q = q.abs()
    scale = 1 / math.sqrt(d)
    g = climb / (scale * math.sqrt(2 / math.pi) * d)
    lin = torch.linspace(0.0, g, s_k).view(1, s_k, 1, 1)
    k = (k.float() + lin).to(k.dtype)
    return q, k, v, scale


FWD_CASES = [
    # dtype, b, s_q, s_k, h, h_kv, d  (attn_fwd: small-d kernel, d = 64, d = 128,
    # one-row decode kernel, packed query heads)
    ("fp16", 2, 150, 600, 3, 0, 16),
    ("fp16", 1, 200, 600, 2, 0, 32),
    ("fp16", 1, 300, 600, 2, 0, 64),
    ("fp16", 2, 260, 600, 2, 0, 128),
    ("fp16", 2, 1, 600, 5, 0, 128),     # one query row: decode kernel (fp32 P)
    ("fp16", 2, 5, 600, 8, 2, 128),     # packed: 4 query heads per K/V head
    ("bf16", 2, 260, 600, 2, 0, 128),
    ("bf16", 2, 150, 600, 3, 0, 16),
]


@pytest.mark.parametrize("pattern", ["planted", "ramp"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", FWD_CASES, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-k{c[3]}-h{c[4]}-kv{c[5]}-d{c[6]}" for c in FWD_CASES])
def test_rising_scores_fused(case, causal, pattern):
    dt, b, s_q, s_k, h, h_kv, d = case
    say("attn_fwd", pattern, case, "causal", causal)
    mk = planted if pattern == "planted" else ramp
    q, k, v, scale = mk(b, s_q, s_k, h, d, dt, seed=101, h_kv=h_kv)
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, causal)
    assert np.nanmax(L_ref) > 12.0  # the scores really do climb far above the first tile
    qd, kd, vd = up(q, k, v)
    O, L = ea.attn_fwd(qd, kd, vd, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    check(O, L, O_ref, L_ref, dt, f"{case} fused")


SPLIT_CASES = [
    # dtype, b, s_q, s_k, h, h_kv, d, splits: attn_fwd_splitkv with several query
    # rows (prefill kernel per split; packed when h_kv < h), then attn_combine
    ("fp16", 1, 100, 900, 2, 0, 128, 3),
    ("fp16", 2, 64, 900, 3, 0, 16, 2),
    ("fp16", 2, 4, 900, 12, 3, 128, 3),
    ("fp16", 1, 2, 900, 8, 1, 64, 2),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-k{c[3]}-h{c[4]}-kv{c[5]}-d{c[6]}-n{c[7]}" for c in SPLIT_CASES])
def test_rising_scores_split(case, causal):
    dt, b, s_q, s_k, h, h_kv, d, n = case
    say("attn_fwd_splitkv planted", case, "causal", causal)
    # a jump in the middle of every split, after that split's first tile
    jumps = {77: 15.0, 377: 30.0, 677: 45.0, 850: 20.0}
    q, k, v, scale = planted(b, s_q, s_k, h, d, dt, seed=103, h_kv=h_kv, jumps=jumps)
    qd, kd, vd = up(q, k, v)
    Op, Lp = ea.attn_fwd_splitkv(qd, kd, vd, num_splits=n, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    Op_ref, Lp_ref = oracle.attention_split(*host64(q, k, v), scale, causal, oracle.split_bounds(s_k, n))
    assert np.all(np.isfinite(f64(Op))), "non-finite partial O"
    assert np.abs(f64(Op) - Op_ref).max() <= TOL_O[dt]
    Lp_h = f64(Lp)
    fin = np.isfinite(Lp_ref)
    assert np.array_equal(np.isfinite(Lp_h), fin)
    assert np.abs(Lp_h[fin] - Lp_ref[fin]).max() <= TOL_LSE
    O, L = ea.attn_combine(Op, Lp, q.dtype)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, causal)
    check(O, L, O_ref, L_ref, dt, f"{case} combined")


PAGED_CASES = [
    # dtype, b, s_q, h, h_kv, d, seqlens, block_size, causal, splits
    ("fp16", 2, 200, 4, 4, 128, [700, 600], 64, True, 2),    # prefill kernel over blocks
    ("fp16", 2, 3, 8, 2, 128, [700, 650], 32, False, 3),     # packed multi-token decode
    ("fp16", 2, 1, 4, 4, 64, [700, 540], 64, False, 2),      # one-row decode kernel
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-h{c[3]}-kv{c[4]}-d{c[5]}-bs{c[7]}" for c in PAGED_CASES])
def test_rising_scores_paged(case):
    dt, b, s_q, h, h_kv, d, lens, bs, causal, n = case
    say("paged planted", case)
    q, kc, vc, table, sl = workloads.make_paged(b, s_q, h, d, dt, lens, bs, h_kv=h_kv, seed=107)
    q = q.abs()
    scale = 1 / math.sqrt(d)
    for bi, length in enumerate(lens):
        for j, nats in JUMPS.items():
            if j < length:
                kc[int(table[bi, j // bs]), j % bs] = nats / (scale * math.sqrt(2 / math.pi) * d)
    O_ref, L_ref = oracle.attention_paged(*host64(q, kc, vc), table.numpy(), sl.numpy(), scale, causal)
    assert np.nanmax(L_ref) > 12.0
    qd, kcd, vcd, td, sld = up(q, kc, vc, table, sl)
    O, L = ea.attn_fwd_paged(qd, kcd, vcd, td, sld, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    check(O, L, O_ref, L_ref, dt, f"{case} fused")
    O2, L2 = ea.attn_decode_paged(qd, kcd, vcd, td, sld, num_splits=n, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    check(O2, L2, O_ref, L_ref, dt, f"{case} split")


@pytest.mark.parametrize("d", [16, 128])
def test_fp16_scale8(d):
    # Scores of size ~ +-8 sqrt(d) both ways (the bf16 test's scale, in fp16).
    say("attn_fwd fp16 scale 8", d)
    q, k, v = workloads.make_qkv(1, 64, 300, 2, d, "fp16", seed=13)
    scale = 8.0
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, False)
    assert np.abs(L_ref).max() > 40
    for causal in (False, True):
        O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, causal)
        O, L = ea.attn_fwd(*up(q, k, v), softmax_scale=scale, causal=causal)
        torch.cuda.synchronize()
        check(O, L, O_ref, L_ref, "fp16", f"scale 8 d={d} causal={causal}", rel_lse=1e-5)


@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_large_key_shift(dt):
    # K + u for a constant u: every score of a row moves by scale * q.u (here by up
    # to a few hundred), which an unsubtracted exp would overflow; the result must
    # still match the definition on the shifted (rounded) inputs.
    say("attn_fwd large key shift", dt)
    q, k, v = workloads.make_qkv(2, 130, 400, 3, 128, dt, seed=37)
    ks = (k.float() + 100.0).to(k.dtype)
    scale = 1 / math.sqrt(128)
    for causal in (False, True):
        O_ref, L_ref = oracle.attention(*host64(q, ks, v), scale, causal)
        assert np.abs(L_ref).max() > 150
        qd, kd, vd = up(q, ks, v)
        O, L = ea.attn_fwd(qd, kd, vd, softmax_scale=scale, causal=causal)
        torch.cuda.synchronize()
        check(O, L, O_ref, L_ref, dt, f"shift causal={causal}", rel_lse=1e-5)
        O2, L2 = ea.attn_decode(qd, kd, vd, num_splits=3, softmax_scale=scale, causal=causal)
        torch.cuda.synchronize()
        check(O2, L2, O_ref, L_ref, dt, f"shift split causal={causal}", rel_lse=1e-5)


@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_closed_form_fp16(d, causal):
    # Q = 0: every visible score is 0, so O is the mean of the visible V rows and
    # LSE = ln |J(i)| (a closed form, independent of the oracle).
    say("attn_fwd fp16 Q=0", d, causal)
    _, k, v = workloads.make_qkv(1, 80, 200, 2, d, "fp16", seed=9)
    q = torch.zeros((1, 80, 2, d), dtype=torch.float16)
    qd, kd, vd = up(q, k, v)
    O, L = ea.attn_fwd(qd, kd, vd, softmax_scale=0.25, causal=causal)
    torch.cuda.synchronize()
    off = 200 - 80
    cnt = np.array([200 if not causal else i + off + 1 for i in range(80)], dtype=np.float64)
    np.testing.assert_allclose(f64(L)[0], np.broadcast_to(np.log(cnt), (2, 80)), atol=1e-5)
    vm = torch.stack([v[0, :int(c)].double().mean(0) for c in cnt])  # (80, h, d)
    assert (O[0].cpu().double() - vm).abs().max() < TOL_O["fp16"]
    if not causal:
        Od, Ld = ea.attn_decode(qd[:, :1].contiguous(), kd, vd, num_splits=4, softmax_scale=0.25)
        torch.cuda.synchronize()
        np.testing.assert_allclose(f64(Ld)[0, :, 0], np.log(200.0), atol=1e-5)
        assert (Od[0, 0].cpu().double() - v[0].double().mean(0)).abs().max() < TOL_O["fp16"]


CONST_CASES = [
    # dtype, b, s_q, s_k, h, d
    ("bf16", 2, 150, 333, 3, 128),
    ("fp16", 2, 150, 333, 3, 128),
    ("fp16", 2, 150, 150, 4, 16),
    ("bf16", 1, 1, 999, 4, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CONST_CASES, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-k{c[3]}-h{c[4]}-d{c[5]}" for c in CONST_CASES])
def test_constant_v_columns(case, causal):
    # V[:, :, :, c] == kappa for two columns: softmax weights sum to 1, so those
    # output columns equal kappa; the GPU rounds P to the input type before P.V
    # while l sums the unrounded P, so it holds within one output ulp.
    dt, b, s_q, s_k, h, d = case
    say("constant V columns", case, causal)
    q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, dt, seed=41)
    v[..., 3] = 0.75
    v[..., d - 1] = -0.625
    qd, kd, vd = up(q, k, v)
    O, L = ea.attn_fwd(qd, kd, vd, softmax_scale=1 / math.sqrt(d), causal=causal)
    Od, Ld = ea.attn_decode(qd, kd, vd, num_splits=3, softmax_scale=1 / math.sqrt(d), causal=causal)
    torch.cuda.synchronize()
    for out, what in ((O, "fused"), (Od, "split")):
        o = f64(out)
        seen = np.isfinite(f64(L)).transpose(0, 2, 1)  # (b, s_q, h): rows that see a key
        assert np.all(np.abs(o[..., 3][seen] - 0.75) <= ULP[dt]), what
        assert np.all(np.abs(o[..., d - 1][seen] + 0.625) <= ULP[dt]), what


SMALL_CASES = [
    # dtype, b, s_q, s_k, h, h_kv, d: the persistent small-head kernel (d <= 32,
    # both lengths <= 256).  Its single pass takes the reference from the first
    # key tile, so every pattern here makes later keys score far above it.
    ("fp16", 3, 150, 250, 4, 0, 16),
    ("bf16", 3, 150, 250, 4, 0, 16),
    ("fp16", 2, 100, 250, 4, 2, 32),
    ("bf16", 2, 100, 250, 4, 2, 32),
]
SMALL_JUMPS = {77: 15.0, 140: 30.0, 230: 45.0}
# a rise that keeps every P of the first pass finite and its row sums small
SMALL_MILD = {100: 5.0, 200: 8.0}


@pytest.mark.parametrize("pattern", ["planted", "ramp", "mild"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", SMALL_CASES, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-k{c[3]}-h{c[4]}-kv{c[5]}-d{c[6]}" for c in SMALL_CASES])
def test_rising_scores_small_heads(case, causal, pattern):
    dt, b, s_q, s_k, h, h_kv, d = case
    say("attn_fwd small heads", pattern, case, "causal", causal)
    if pattern == "ramp":
        q, k, v, scale = ramp(b, s_q, s_k, h, d, dt, seed=109, h_kv=h_kv)
    else:
        q, k, v, scale = planted(b, s_q, s_k, h, d, dt, seed=109, h_kv=h_kv,
                                 jumps=SMALL_JUMPS if pattern == "planted" else SMALL_MILD)
    O_ref, L_ref = oracle.attention(*host64(q, k, v), scale, causal)
    assert np.nanmax(L_ref) > (6.0 if pattern == "mild" else 12.0)
    O, L = ea.attn_fwd(*up(q, k, v), softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    check(O, L, O_ref, L_ref, dt, f"{case} {pattern}")


@pytest.mark.parametrize("d", [16, 32])
@pytest.mark.parametrize("dt", ["fp16", "bf16"])
def test_small_heads_scale8_and_key_shift(dt, d):
    # Scores of +-8 sqrt(d) both ways, and K + 100 (every score of a row moved by
    # scale * q.u), through the small-head kernel (s_k <= 256).
    say("attn_fwd small heads scale 8 / key shift", dt, d)
    q, k, v = workloads.make_qkv(2, 64, 200, 3, d, dt, seed=113)
    ks = (k.float() + 100.0).to(k.dtype)
    for kk, scale in ((k, 8.0), (ks, 1 / math.sqrt(d))):
        for causal in (False, True):
            O_ref, L_ref = oracle.attention(*host64(q, kk, v), scale, causal)
            assert np.abs(L_ref).max() > 40
            O, L = ea.attn_fwd(*up(q, kk, v), softmax_scale=scale, causal=causal)
            torch.cuda.synchronize()
            check(O, L, O_ref, L_ref, dt, f"scale {scale} causal={causal}", rel_lse=1e-5)
