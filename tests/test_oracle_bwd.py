"""Pins for the CPU oracle of the attention gradient (oracle/backward.py).

The gradient oracle is checked against things other than itself:
* central finite differences of the scalar brute-force forward (oracle.brute),
  element by element, on tiny shapes;
* directional finite differences of the (independently pinned) vectorised
  forward, on shapes with ragged causal masks and rows that see no key;
* a library special case: torch float64 autograd on the CPU through plain
  matmul / masked softmax;
* closed forms: a single key gives dQ = dK = 0 and dV = Σ dO; constant V
  columns give dQ = dK = 0; Q = 0 gives dV_j = Σ_i dO_i / |J(i)| over the rows
  that see key j;
* invariants: Σ_j dK_j = 0 (scores are invariant to a common key shift) and
  Σ_j dV_j = Σ_i dO_i over the rows that see any key (rows of P sum to 1);
* shared K/V heads = multi-head attention on repeated heads with dK, dV summed
  over each group;
* the per-row and per-key samplers used at long shapes agree with the full form.

A mutation test plants plausible mistakes in a copy of the gradient (on the
CPU) and checks that at least one pin catches each of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import backward as ob
from oracle import exact as oa
from oracle.brute import attention_brute


def _rand(b, s_q, s_k, h, h_kv, d, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((b, s_q, h, d)), r.standard_normal((b, s_k, h_kv, d)),
            r.standard_normal((b, s_k, h_kv, d)), r.standard_normal((b, s_q, h, d)))


def _loss_brute(q, k, v, do, scale, causal):
    O, _ = attention_brute(q, k, v, scale, causal)
    return math.fsum(float(a) * float(b) for a, b in zip(np.ravel(O), np.ravel(do)))


def _loss(q, k, v, do, scale, causal):
    O, _ = oa.attention(q, k, v, scale, causal)
    return float((O * do).sum())


def _visible_rows(s_q, s_k, causal):
    return oa.visible_mask(s_q, s_k, causal).any(axis=1)


# ---------------------------------------------------------------- pins ----

def pin_bwd_fd_brute():
    """Every gradient entry against a central difference of the scalar forward."""
    eps = 1e-6
    for causal, (s_q, s_k) in ((False, (3, 4)), (True, (3, 4)), (True, (4, 2))):
        q, k, v, do = _rand(1, s_q, s_k, 2, 1, 2, seed=7 + s_q + 10 * causal)
        scale = 0.8
        dq, dk, dv, _ = ob.attention_bwd(q, k, v, do, scale, causal)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + eps
                fp = _loss_brute(q, k, v, do, scale, causal)
                x[idx] = old - eps
                fm = _loss_brute(q, k, v, do, scale, causal)
                x[idx] = old
                fd = (fp - fm) / (2 * eps)
                assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(fd)), (causal, idx, fd, g[idx])


def pin_bwd_fd_directional():
    """⟨grad, u⟩ against a central difference of the vectorised forward along u."""
    eps = 1e-5
    cases = [(2, 9, 13, 4, 2, 8, False), (2, 9, 13, 4, 2, 8, True), (1, 11, 6, 2, 2, 4, True),
             (1, 17, 17, 3, 1, 16, True)]
    for n, (b, s_q, s_k, h, h_kv, d, causal) in enumerate(cases):
        q, k, v, do = _rand(b, s_q, s_k, h, h_kv, d, seed=100 + n)
        scale = 1 / math.sqrt(d)
        grads = ob.attention_bwd(q, k, v, do, scale, causal)[:3]
        r = np.random.default_rng(200 + n)
        for which in range(3):
            u = r.standard_normal((q, k, v)[which].shape)
            xs_p = [q, k, v]
            xs_m = [q, k, v]
            xs_p[which] = xs_p[which] + eps * u
            xs_m[which] = xs_m[which] - eps * u
            fd = (_loss(*xs_p, do, scale, causal) - _loss(*xs_m, do, scale, causal)) / (2 * eps)
            an = float((grads[which] * u).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (n, which, fd, an)


def pin_bwd_torch_autograd():
    """torch float64 autograd through plain matmul and a masked softmax."""
    for causal in (False, True):
        b, s_q, s_k, h, d = 2, 7, 10, 3, 5
        q, k, v, do = _rand(b, s_q, s_k, h, h, d, seed=31 + causal)
        scale = 0.37
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        S = scale * torch.einsum("bihc,bjhc->bhij", tq, tk)
        if causal:
            keep = torch.arange(s_k)[None, :] <= torch.arange(s_q)[:, None] + (s_k - s_q)
            S = S.masked_fill(~keep, float("-inf"))
        O = torch.einsum("bhij,bjhc->bihc", torch.softmax(S, dim=-1), tv)
        O.backward(torch.tensor(do))
        dq, dk, dv, _ = ob.attention_bwd(q, k, v, do, scale, causal)
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def pin_bwd_single_key():
    """One key: every visible weight is exactly 1, so dQ = dK = 0 and dV = Σ dO."""
    q, k, v, do = _rand(2, 5, 1, 4, 2, 8, seed=3)
    dq, dk, dv, _ = ob.attention_bwd(q, k, v, do, 0.5, False)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13
    want = do.reshape(2, 5, 2, 2, 8).sum(axis=(1, 3))  # rows and the two heads of a group
    np.testing.assert_allclose(dv[:, 0], want, rtol=0, atol=1e-13)
    # causal, one key: only the last row sees it
    dq, dk, dv, _ = ob.attention_bwd(q, k, v, do, 0.5, True)
    np.testing.assert_allclose(dv[:, 0], do[:, -1].reshape(2, 2, 2, 8).sum(axis=2), rtol=0, atol=1e-13)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dq[:, :-1]).max() == 0


def pin_bwd_constant_v():
    """V columns constant over keys: O does not depend on the scores."""
    q, k, v, do = _rand(2, 6, 9, 2, 2, 4, seed=5)
    v[:] = np.array([0.75, -1.5, 2.0, 0.0])
    for causal in (False, True):
        dq, dk, _, _ = ob.attention_bwd(q, k, v, do, 0.9, causal)
        assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12


def pin_bwd_q_zero():
    """Q = 0: uniform weights 1/|J(i)|, so dV_j = Σ over rows seeing j of dO_i/|J(i)|."""
    for causal, (s_q, s_k) in ((False, (5, 7)), (True, (7, 5)), (True, (6, 6))):
        q, k, v, do = _rand(1, s_q, s_k, 1, 1, 3, seed=11)
        q[:] = 0
        _, _, dv, _ = ob.attention_bwd(q, k, v, do, 1.3, causal)
        want = np.zeros((s_k, 3))
        for i in range(s_q):
            vis = [j for j in range(s_k) if not causal or j <= i + s_k - s_q]
            for j in vis:
                want[j] += do[0, i, 0] / len(vis)
        np.testing.assert_allclose(dv[0, :, 0], want, rtol=0, atol=1e-14)


def pin_bwd_key_sums():
    """Σ_j dK_j = 0 and Σ_j dV_j = Σ_i dO_i over rows that see a key."""
    for causal, (s_q, s_k) in ((False, (8, 12)), (True, (12, 8)), (True, (9, 9))):
        q, k, v, do = _rand(2, s_q, s_k, 4, 2, 6, seed=13)
        _, dk, dv, _ = ob.attention_bwd(q, k, v, do, 0.6, causal)
        assert np.abs(dk.sum(axis=1)).max() <= 1e-12
        vis = _visible_rows(s_q, s_k, causal)
        want = (do * vis[None, :, None, None]).sum(axis=1).reshape(2, 2, 2, 6).sum(axis=2)
        np.testing.assert_allclose(dv.sum(axis=1), want, rtol=0, atol=1e-12)


def pin_bwd_delta():
    """δ is the row dot of dO with the forward oracle's O (0 on rows with no key)."""
    q, k, v, do = _rand(2, 10, 6, 2, 1, 4, seed=17)
    for causal in (False, True):
        O, _ = oa.attention(q, k, v, 0.7, causal)
        _, _, _, delta = ob.attention_bwd(q, k, v, do, 0.7, causal)
        np.testing.assert_allclose(delta, (O * do).sum(-1).transpose(0, 2, 1), rtol=0, atol=1e-13)


def pin_bwd_gqa_is_mha_on_repeated_heads():
    q, k, v, do = _rand(2, 7, 9, 6, 2, 4, seed=19)
    g = 3
    for causal in (False, True):
        dq, dk, dv, _ = ob.attention_bwd(q, k, v, do, 0.5, causal)
        kr, vr = np.repeat(k, g, axis=2), np.repeat(v, g, axis=2)
        dq2, dk2, dv2, _ = ob.attention_bwd(q, kr, vr, do, 0.5, causal)
        np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dk, dk2.reshape(2, 9, 2, g, 4).sum(3), rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv, dv2.reshape(2, 9, 2, g, 4).sum(3), rtol=0, atol=1e-13)


def pin_bwd_samplers_agree():
    q, k, v, do = _rand(2, 37, 41, 4, 2, 8, seed=23)
    rows, cols = [0, 5, 36], [0, 17, 40]
    for causal in (False, True):
        dq, dk, dv, delta = ob.attention_bwd(q, k, v, do, 0.4, causal)
        dqr, dlr = ob.attention_bwd_dq_rows(q, k, v, do, 0.4, causal, head=3, rows=rows)
        np.testing.assert_allclose(dqr, dq[:, rows, 3], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dlr, delta[:, 3, rows], rtol=0, atol=1e-13)
        dkc, dvc = ob.attention_bwd_dkdv_cols(q, k, v, do, 0.4, causal, kv_head=1, cols=cols, row_chunk=16)
        np.testing.assert_allclose(dkc, dk[:, cols, 1], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dvc, dv[:, cols, 1], rtol=0, atol=1e-13)


PINS = [pin_bwd_fd_brute, pin_bwd_fd_directional, pin_bwd_torch_autograd, pin_bwd_single_key,
        pin_bwd_constant_v, pin_bwd_q_zero, pin_bwd_key_sums, pin_bwd_delta,
        pin_bwd_gqa_is_mha_on_repeated_heads, pin_bwd_samplers_agree]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ------------------------------------------------------------ mutants ----
# A copy of the gradient with one plausible mistake switched on at a time.

def _bwd_mutant(mut):
    def f(q, k, v, dout, scale, causal):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
        b, s_q, h, d = q.shape
        s_k, h_kv = k.shape[1], k.shape[2]
        kv = np.arange(h) // (h // h_kv)
        mask = oa.visible_mask(s_q, s_k, causal)
        dq, dk, dv = np.zeros_like(q), np.zeros(k.shape), np.zeros(v.shape)
        delta = np.zeros((b, h, s_q))
        for bi in range(b):
            for hh in range(h):
                qh, kh, vh, doh = q[bi, :, hh], k[bi, :, kv[hh]], v[bi, :, kv[hh]], do[bi, :, hh]
                S = np.where(mask, scale * (qh @ kh.T), -np.inf)
                P, _, _ = oa.softmax_rows(S)
                O = P @ vh
                dP = doh @ vh.T
                dl = (doh * O).sum(-1)
                if mut == "no_delta":
                    dl = np.zeros_like(dl)
                if mut == "delta_from_v":
                    dl = (doh * vh[: s_q] if s_q <= s_k else doh).sum(-1)
                dS = P * (dP - dl[:, None])
                if mut == "ds_without_p":
                    dS = np.where(mask, dP - dl[:, None], 0.0)
                sq = 1.0 if mut == "dq_no_scale" else scale
                sk = scale * scale if mut == "dk_double_scale" else scale
                dq[bi, :, hh] = sq * (dS @ kh)
                dk_h = sk * (dS.T @ qh)
                if mut == "dk_uses_dp":
                    dk_h = sk * ((P * dP).T @ qh)
                dv_h = P.T @ doh
                if mut == "dv_unmasked_softmax":
                    dv_h = oa.softmax_rows(scale * (qh @ kh.T))[0].T @ doh
                if mut == "dq_uses_v":
                    dq[bi, :, hh] = sq * (dS @ vh)
                if mut == "gqa_last_head_only":
                    dk[bi, :, kv[hh]] = dk_h
                    dv[bi, :, kv[hh]] = dv_h
                else:
                    dk[bi, :, kv[hh]] += dk_h
                    dv[bi, :, kv[hh]] += dv_h
                delta[bi, hh] = dl
        return dq, dk, dv, delta
    return f


MUTANTS = ["no_delta", "delta_from_v", "ds_without_p", "dq_no_scale", "dk_double_scale",
           "dk_uses_dp", "dv_unmasked_softmax", "dq_uses_v", "gqa_last_head_only"]


@pytest.mark.parametrize("name", MUTANTS)
def test_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(ob, "attention_bwd", _bwd_mutant(name))
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except Exception:
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_copy_passes_every_pin(monkeypatch):
    """The mutant harness itself: with no mutation the copy passes all pins."""
    monkeypatch.setattr(ob, "attention_bwd", _bwd_mutant(None))
    for pin in PINS:
        pin()
