"""The allocation-free backward (attn_bwd_noalloc, for callers that cannot
allocate device memory) against the existing entry point attn_bwd, through the
C ABI: the same kernels with delta in the library's static buffer instead of a
caller workspace, so the results must be identical, on two calls in a row (the
second smaller, after the first has left its delta in the buffer), and within
the forward's tolerances of the float64 gradient oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import exact_attention_64_amd as ea

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"fp16": 5e-3, "bf16": 2e-2}


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_noalloc_matches_bwd(causal):
    cases = [("bf16", 2, 300, 333, 6, 2, 128), ("fp16", 1, 97, 130, 3, 3, 64)]  # second call smaller
    for dt, b, s_q, s_k, h, h_kv, d in cases:
        print("[case] attn_bwd_noalloc", dt, b, s_q, s_k, h, h_kv, d, "causal", causal, flush=True)
        q, k, v = workloads.make_qkv(b, s_q, s_k, h, d, dt, seed=51, h_kv=h_kv)
        do = workloads.make_dout(b, s_q, h, d, dt, seed=52)
        qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
        scale = 1 / math.sqrt(d)
        O, L = ea.attn_fwd(qd, kd, vd, softmax_scale=scale, causal=causal)
        ref = ea.attn_bwd(qd, kd, vd, O, dod, L, softmax_scale=scale, causal=causal)
        outs = [torch.full_like(t, float("nan")) for t in ref]
        got = ea.attn_bwd_noalloc(qd, kd, vd, O, dod, L, *outs, softmax_scale=scale, causal=causal)
        torch.cuda.synchronize()
        for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
            assert torch.equal(g, r), f"{name} differs from attn_bwd"
        h64 = [t.to(torch.float64).numpy() for t in (q, k, v, do)]
        grads = oracle.attention_bwd(*h64, scale, causal)[:3]
        for g, r in zip(got, grads):
            err = np.abs(g.double().cpu().numpy() - r).max() / max(1.0, np.abs(r).max())
            assert err <= TOL[dt], err
