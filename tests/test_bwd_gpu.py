"""GPU parity of the backward pass (attn_bwd through the C ABI) against the
float64 CPU gradient oracle (oracle/backward.py).

Both sides get the same seeded, dtype-rounded q, k, v and dO
(workloads.make_qkv, workloads.make_dout).  The GPU backward takes O and LSE from
the GPU forward, as a training step would; the oracle recomputes everything from
q, k, v and dO alone.

Tolerance (the pages give none for gradients): the forward's bounds, max-abs
5e-3 (fp16) / 2e-2 (bf16), applied relative to each gradient tensor's own scale,
max |dX - dX_ref| <= tol * max(1, max |dX_ref|).  The GPU rounds each output to
the input type (half an ulp is 2^-9 relative in bf16, 2^-12 in fp16) and rounds P
and dS to the input type before each product (fp32 accumulation), which the
oracle does not mimic; the bound leaves a margin of about ten over the output
rounding alone.  Rows that see no key must give exactly dQ = 0.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_attention_64_amd as ea

pytestmark = pytest.mark.gpu

TOL = {"fp16": 5e-3, "bf16": 2e-2}
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def host64(*ts):
    return [t.to(torch.float64).numpy() for t in ts]


def rel_err(x, ref):
    return float(np.abs(x - ref).max() / max(1.0, float(np.abs(ref).max()))) if ref.size else 0.0


def run_bwd(q, k, v, do, scale, causal):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    O, L = ea.attn_fwd(qd, kd, vd, softmax_scale=scale, causal=causal)
    dq, dk, dv = ea.attn_bwd(qd, kd, vd, O, dod, L, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_full(dq, dk, dv, ref, dtype, what):
    dq_r, dk_r, dv_r, _ = ref
    out = {}
    for name, x, r in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
        x = f64(x)
        assert np.all(np.isfinite(x)), f"{what}: non-finite {name}"
        e = rel_err(x, r)
        out[name] = e
        assert e <= TOL[dtype], f"{what}: {name} relative max error {e:.3e}"
    return out


SMALL = [
    # dtype, b, s_q, s_k, h, h_kv, d -- several tiles of 128 rows / keys plus ragged tails
    ("bf16", 2, 300, 333, 3, 3, 128),
    ("fp16", 2, 300, 333, 3, 3, 128),
    ("bf16", 1, 517, 517, 4, 2, 64),
    ("fp16", 3, 129, 257, 2, 2, 64),
    ("bf16", 2, 200, 161, 3, 3, 32),
    ("fp16", 2, 97, 130, 4, 1, 32),
    ("fp16", 2, 150, 150, 4, 4, 16),
    ("bf16", 1, 33, 65, 6, 2, 16),
    ("bf16", 1, 100, 90, 2, 2, 128),   # causal: the first rows see no key
    ("fp16", 1, 33, 300, 6, 2, 64),    # few rows, many keys, shared K/V heads
    ("bf16", 1, 1, 129, 2, 2, 128),    # one query row
    ("bf16", 2, 200, 300, 8, 2, 128),  # d = 128 with four query heads per K/V head
    ("fp16", 1, 257, 131, 6, 3, 128),  # the same in fp16, fewer keys than rows
    ("fp16", 2, 37, 1, 3, 3, 64),      # one key (causal: only the last row sees it)
    ("bf16", 1, 5, 3, 2, 1, 128),      # three keys, five rows, one K/V head
    ("bf16", 3, 70, 390, 5, 5, 32),    # 45 dK/dV and 15 dQ work-groups: uneven over the 8 XCDs
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-b{c[1]}-q{c[2]}-k{c[3]}-h{c[4]}-kv{c[5]}-d{c[6]}"
                                              for c in SMALL])
def test_bwd_small(case, causal):
    dtype, b, s_q, s_k, h, h_kv, d = case
    say("bwd", case, "causal", causal)
    q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, dtype, seed=42, h_kv=h_kv)
    do = workloads.make_dout(b, s_q, h, d, dtype)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = run_bwd(q, k, v, do, scale, causal)
    ref = oracle.attention_bwd(*host64(q, k, v, do), scale, causal)
    errs = check_full(dq, dk, dv, ref, dtype, f"{case} causal={causal}")
    say("rel errors", {kk: f"{e:.2e}" for kk, e in errs.items()})
    if causal and s_q > s_k:
        blind = np.arange(s_q) + (s_k - s_q) < 0
        assert np.all(f64(dq)[:, blind] == 0)


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.5])
def test_bwd_scales(scale):
    """Zero scale (uniform weights: dQ = dK = 0), a negative scale, a sharp one."""
    say("bwd scale", scale)
    q, k, v = workloads.make_qkv(2, 130, 140, 2, 64, "bf16", seed=5)
    do = workloads.make_dout(2, 130, 2, 64, "bf16", seed=6)
    dq, dk, dv = run_bwd(q, k, v, do, scale, True)
    ref = oracle.attention_bwd(*host64(q, k, v, do), scale, True)
    check_full(dq, dk, dv, ref, "bf16", f"scale={scale}")
    if scale == 0.0:
        assert np.all(f64(dq) == 0) and np.all(f64(dk) == 0)


def test_bwd_strided_views():
    """Packed QKV / gradient views with non-unit head and row strides."""
    say("bwd strided views")
    b, s, h, d = 2, 200, 3, 64
    q, k, v = workloads.make_qkv(b, s, s, h, d, "fp16", seed=9)
    do = workloads.make_dout(b, s, h, d, "fp16", seed=10)
    qkv = torch.stack([q, k, v], dim=3).to(DEV)          # (b, s, h, 3, d)
    qv, kv_, vv = qkv[:, :, :, 0], qkv[:, :, :, 1], qkv[:, :, :, 2]
    O, L = ea.attn_fwd(qv, kv_, vv, softmax_scale=0.125, causal=True)
    grads = torch.zeros((b, s, h, 3, d), dtype=torch.float16, device=DEV)
    ea.attn_bwd(qv, kv_, vv, O, do.to(DEV), L, softmax_scale=0.125, causal=True,
                dq=grads[:, :, :, 0], dk=grads[:, :, :, 1], dv=grads[:, :, :, 2])
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(*host64(q, k, v, do), 0.125, True)
    check_full(grads[:, :, :, 0], grads[:, :, :, 1], grads[:, :, :, 2], ref, "fp16", "strided")


@pytest.mark.parametrize("d", [32, 128])
def test_bwd_guard_bands_and_delta(d):
    """Every output is written only inside its view (sentinels after each), and the
    delta workspace holds rowsum(dO * O) of the O passed in."""
    say("bwd guard bands, d", d)
    b, s_q, s_k, h, h_kv = 1, 129, 77, 4, 2
    q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, "fp16", seed=21, h_kv=h_kv)
    do = workloads.make_dout(b, s_q, h, d, "fp16", seed=22)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    O, L = ea.attn_fwd(qd, kd, vd, softmax_scale=0.2, causal=True)

    def guarded(shape, dtype):
        n = int(np.prod(shape))
        full = torch.full((n + 4096,), 7.0, dtype=dtype, device=DEV)
        return full, full[:n].view(shape)

    bufs = [guarded(q.shape, torch.float16), guarded(k.shape, torch.float16),
            guarded(v.shape, torch.float16), guarded((b, h, s_q), torch.float32)]
    (_, dq), (_, dk), (_, dv), (_, delta) = bufs
    ea.attn_bwd(qd, kd, vd, O, dod, L, softmax_scale=0.2, causal=True, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    for full, view in bufs:
        assert (full[view.numel():] == 7.0).all()
    ref = oracle.attention_bwd(*host64(q, k, v, do), 0.2, True)
    check_full(dq, dk, dv, ref, "fp16", f"guard bands d={d}")
    delta_host = np.einsum("bshd,bshd->bhs", f64(do), f64(O))
    assert np.abs(f64(delta) - delta_host).max() <= 1e-4 * max(1.0, float(np.abs(delta_host).max()))


def test_backward_plan_matches_call():
    """BwdPlan (arguments marshalled once) runs the same kernels: bit-identical to
    attn_bwd, also after a new dO is copied into the planned input (then checked
    against the oracle)."""
    say("BwdPlan vs attn_bwd")
    q, k, v = workloads.make_qkv(2, 50, 50, 16, 16, "fp16", seed=71)
    do = workloads.make_dout(2, 50, 16, 16, "fp16", seed=72)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    O, L = ea.attn_fwd(qd, kd, vd, softmax_scale=0.25, causal=True)
    plan = ea.BwdPlan(qd, kd, vd, O, dod, L, 0.25, True)
    got = [t.clone() for t in plan()]
    ref = ea.attn_bwd(qd, kd, vd, O, dod, L, softmax_scale=0.25, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
    do2 = workloads.make_dout(2, 50, 16, 16, "fp16", seed=73)
    dod.copy_(do2.to(DEV))
    dq, dk, dv = plan()
    torch.cuda.synchronize()
    check_full(dq, dk, dv, oracle.attention_bwd(*host64(q, k, v, do2), 0.25, True), "fp16", "plan after new dO")


def test_bwd_deterministic():
    say("bwd determinism")
    q, k, v = workloads.make_qkv(1, 300, 300, 4, 128, "bf16", seed=12, h_kv=2)
    do = workloads.make_dout(1, 300, 4, 128, "bf16", seed=13)
    a = [t.clone() for t in run_bwd(q, k, v, do, 0.1, True)]
    b_ = run_bwd(q, k, v, do, 0.1, True)
    for x, y in zip(a, b_):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["C1", "C2"])
def test_bwd_issue_1335_workloads(name):
    """The fp16, head-dim-16 workloads whose backward issue #1335 times, in full."""
    w = workloads.WORKLOADS[name]
    say("bwd workload", name, w.note)
    q, k, v = workloads.make_workload(w)
    do = workloads.make_dout(w.b, w.s_q, w.h, w.d, w.dtype)
    dq, dk, dv = run_bwd(q, k, v, do, w.scale, w.causal)
    ref = oracle.attention_bwd(*host64(q, k, v, do), w.scale, w.causal)
    errs = check_full(dq, dk, dv, ref, w.dtype, name)
    say("rel errors", {kk: f"{e:.2e}" for kk, e in errs.items()})


def test_bwd_long_causal_sampled():
    """The 16k causal bf16 shape the benchmark times: sampled dQ rows of two
    heads, sampled dK/dV keys of one head (its every query row recomputed by the
    oracle in chunks), and two identities that hold at any size."""
    w = workloads.WORKLOADS["C5"]
    say("bwd long causal", w.note)
    q, k, v = workloads.make_workload(w)
    do = workloads.make_dout(w.b, w.s_q, w.h, w.d, w.dtype)
    dq, dk, dv = run_bwd(q, k, v, do, w.scale, True)
    q64, k64, v64, do64 = host64(q, k, v, do)
    for hh in (0, w.h - 1):
        rows = workloads.sample_rows(w.s_q, 64, 1, seed=42 + hh)[0]
        ref, _ = oracle.attention_bwd_dq_rows(q64, k64, v64, do64, w.scale, True, hh, rows)
        e = rel_err(f64(dq[:, rows, hh]), ref)
        say("dq head", hh, f"{e:.2e}")
        assert e <= TOL["bf16"]
    cols = np.array(sorted({0, 1, 31, 32, 127, 128, 4095, 8191, 12000, w.s_k - 2, w.s_k - 1}))
    dk_r, dv_r = oracle.attention_bwd_dkdv_cols(q64, k64, v64, do64, w.scale, True, 5, cols)
    ek, ev = rel_err(f64(dk[:, cols, 5]), dk_r), rel_err(f64(dv[:, cols, 5]), dv_r)
    say("dk/dv head 5", f"{ek:.2e} {ev:.2e}")
    assert ek <= TOL["bf16"] and ev <= TOL["bf16"]
    # sum_j dV_j = sum_i dO_i (every row sees a key) and sum_j dK_j = 0, per head
    sv = f64(dv).sum(axis=1)
    want = do64.sum(axis=1)
    assert np.abs(sv - want).max() <= 2e-2 * np.abs(want).max()
    sk = f64(dk).sum(axis=1)
    assert np.abs(sk).max() <= 2e-2 * np.abs(f64(dk)).sum(axis=1).max()


def test_bwd_graph_capture_replay():
    """attn_bwd enqueues kernels only, so a HIP graph can capture a forward +
    backward pair; each replay (new inputs copied in, eager work between
    replays) must equal an eager call bit for bit, and the first and last
    replays match the oracle."""
    say("HIP graph capture: attn_fwd + attn_bwd")
    shape = (2, 150, 150, 4, 64)
    b, s_q, s_k, h, d = shape
    q, k, v = (t.to(DEV) for t in workloads.make_qkv(b, s_q, s_k, h, d, "bf16", seed=90, h_kv=2))
    do = workloads.make_dout(b, s_q, h, d, "bf16", seed=91).to(DEV)
    O = torch.empty_like(q)
    L = torch.empty((b, h, s_q), device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((b, h, s_q), device=DEV)

    def run(o, l, gq, gk, gv, dl):
        ea.attn_fwd(q, k, v, 0.125, True, out=o, lse=l)
        ea.attn_bwd(q, k, v, o, do, l, 0.125, True, dq=gq, dk=gk, dv=gv, delta=dl)

    run(O, L, dq, dk, dv, delta)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(O, L, dq, dk, dv, delta)
    E = [torch.empty_like(t) for t in (O, L, dq, dk, dv, delta)]
    for rep in range(3):
        new = workloads.make_qkv(b, s_q, s_k, h, d, "bf16", seed=100 + rep, h_kv=2)
        new_do = workloads.make_dout(b, s_q, h, d, "bf16", seed=110 + rep)
        for dst, src in zip((q, k, v, do), (*new, new_do)):
            dst.copy_(src.to(DEV))
        g.replay()
        torch.cuda.synchronize()
        run(*E)
        torch.cuda.synchronize()
        for got, want in zip((O, L, dq, dk, dv), E[:5]):
            assert torch.equal(got, want), f"replay {rep} differs from the eager call"
        if rep in (0, 2):
            ref = oracle.attention_bwd(*host64(*new, new_do), 0.125, True)
            check_full(dq, dk, dv, ref, "bf16", f"graph replay {rep}")
