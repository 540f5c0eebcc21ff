"""Host model of the fused forward kernel's lazy online-softmax rescale.

The prefill kernel (fwdp_kernel) keeps, per query row, a reference m (base-2
units), the sum l of exp2(s - m) in fp32 and O accumulated against the same m.
The common step exponentiates a 32-key tile against the current m without taking
a maximum; a rare step ("rebase") moves m up to the tile's row maximum and
rescales O and l, which is the exact online rescale of "LLM Lab Notes 07: Why
FlashAttention Is Fast", §3.3 Online Softmax.  The rebase fires when a row has no
reference yet or when a lane's partial sum of P exceeds a bound PMAX.  P is
rounded to the input type before the P·V product, so PMAX must keep every P
finite in that type: fp16's largest finite value is 65504.

This file models that step sequence in NumPy (lane split of a 32-key tile as the
kernel holds it: lane half 0 owns keys {0-3, 8-11, 16-19, 24-27}, half 1 the
other 16), shows that the bound 2^64 lets an fp16 P overflow to inf when a later
score exceeds the reference by more than 16 base-2 units, and that the kernel's
dtype-dependent bound (read from the kernel source) keeps O finite and equal to
the float64 oracle within the forward tolerance.  CPU only; it calls nothing on
the GPU and shares no code with the library.
"""
import math
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LN2 = math.log(2.0)
LOG2E = 1.0 / LN2


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 (nearest even) -> float32, NaN/inf preserved."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isfinite(x), out, x)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        with np.errstate(over="ignore"):
            return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)
    return round_bf16(x)


# Keys of one 32-key tile held by lane half 0 and half 1 (register r of the
# 32x32 MFMA result holds key (r // 4) * 8 + half * 4 + r % 4).
HALF_KEYS = [np.array([(r // 4) * 8 + hh * 4 + r % 4 for r in range(16)]) for hh in (0, 1)]


def kernel_model_row(s2: np.ndarray, v: np.ndarray, pmax: float, dtype: str):
    """One query row through the kernel's step sequence.

    s2: (s_k,) scores already scaled to base 2 (scale * log2 e * q.k), masked
        keys as -inf; v: (s_k, d) values (exact input-type values).
    Returns (O (d,), LSE natural log) as the kernel would produce them, with fp32
    arithmetic for P, l and O and P rounded to ``dtype`` before P·V.
    """
    s2 = np.asarray(s2, np.float32)
    n = s2.size
    d = v.shape[1]
    m = np.float32(-np.inf)
    l = np.float32(0.0)
    o = np.zeros(d, np.float32)
    for k0 in range(0, n, 32):
        tile = np.full(32, -np.inf, np.float32)
        tile[: min(32, n - k0)] = s2[k0:k0 + 32]
        vt = np.zeros((32, d), np.float32)
        vt[: min(32, n - k0)] = v[k0:k0 + 32]

        def expo(mref):
            m_use = np.float32(0.0) if mref == -np.inf else mref
            with np.errstate(over="ignore", invalid="ignore"):
                p = np.exp2(tile - m_use).astype(np.float32)
            ls = [np.float32(p[hk].sum(dtype=np.float32)) for hk in HALF_KEYS]
            return p, ls

        p, ls = expo(m)
        bad = m == -np.inf or any(not (x <= pmax) for x in ls)
        if bad:  # the rebase (wave-wide in the kernel; per row here)
            m_new = np.float32(max(m, tile.max()))
            alpha = np.float32(1.0) if m_new == -np.inf else np.float32(np.exp2(m - m_new))
            m = m_new
            l = np.float32(l * alpha)
            o = (o * alpha).astype(np.float32)
            p, ls = expo(m)
        l = np.float32(l + ls[0] + ls[1])
        pr = round_to(p, dtype)
        with np.errstate(over="ignore", invalid="ignore"):
            o = (o + pr @ vt).astype(np.float32)
    if l > 0:
        return o / l, float((m + np.log2(l)) * LN2)
    return np.zeros(d, np.float32), -math.inf


def kernel_pmax(dtype: str) -> float:
    """The bound the kernel source uses for ``dtype`` (parsed from attn_fwd.hip)."""
    src = open(os.path.join(ROOT, "exact_attention_64_amd", "csrc", "attn_fwd.hip")).read()
    mt = re.search(r"constexpr float PMAX\s*=\s*T_ == kFP16 \? (0x1p\d+f) : (0x1p\d+f);", src)
    assert mt, "PMAX must be chosen per input type in fwdp_kernel"
    lit = mt.group(1) if dtype == "fp16" else mt.group(2)
    return float.fromhex(lit[:-1])


def rising_row(rng, n: int, d: int, jump_nats: float, at: int, dtype: str):
    """Scores N(0,1) (natural units) plus one key at index ``at`` scoring
    ``jump_nats`` above the rest; v N(0,1) rounded to ``dtype``."""
    s = rng.standard_normal(n)
    s[at] = jump_nats
    v = round_to(rng.standard_normal((n, d)).astype(np.float32), dtype)
    return s, v


def oracle_row(s_nat: np.ndarray, v: np.ndarray):
    """The definition for one row through the float64 oracle: a query whose score
    with key j is s_nat[j] (q = e_0 * 1, k_j = e_0 * s_nat[j], scale 1)."""
    n, d = v.shape
    q = np.zeros((1, 1, 1, d), np.float64)
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, n, 1, d), np.float64)
    k[0, :, 0, 0] = s_nat
    O, L = oracle.attention(q, k, v.reshape(1, n, 1, d).astype(np.float64), 1.0, False)
    return O[0, 0, 0], float(L[0, 0, 0])


@pytest.mark.parametrize("jump", [12.0, 15.0, 20.0, 40.0])
def test_old_bound_overflows_fp16(jump):
    # A key scoring `jump` natural units above the first tile's maximum, in the
    # third tile: with PMAX = 2^64 no rebase fires, P = 2^(jump*log2 e) > 65504
    # rounds to fp16 inf and O becomes inf/NaN.
    rng = np.random.default_rng(1)
    s, v = rising_row(rng, 200, 16, jump, 77, "fp16")
    s2 = (s * LOG2E).astype(np.float32)
    O, _ = kernel_model_row(s2, v, 2.0 ** 64, "fp16")
    if (jump - s[:32].max()) * LOG2E > 16.0:
        assert not np.all(np.isfinite(O))
    O, L = kernel_model_row(s2, v, kernel_pmax("fp16"), "fp16")
    O_ref, L_ref = oracle_row(s.astype(np.float32).astype(np.float64), v)
    assert np.all(np.isfinite(O))
    assert np.abs(O - O_ref).max() <= 5e-3 and abs(L - L_ref) <= 1e-3


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("pattern", ["jump", "ramp", "late_jump", "normal", "scale8"])
def test_kernel_bound_matches_oracle(dtype, pattern):
    rng = np.random.default_rng(7)
    n, d = 333, 32
    if pattern == "jump":
        s, v = rising_row(rng, n, d, 20.0, 70, dtype)
    elif pattern == "late_jump":
        s, v = rising_row(rng, n, d, 45.0, 330, dtype)
    elif pattern == "ramp":  # scores climb by 30 natural units across the keys
        s = rng.standard_normal(n) + np.linspace(0.0, 30.0, n)
        v = round_to(rng.standard_normal((n, d)).astype(np.float32), dtype)
    elif pattern == "scale8":  # large scores both ways
        s = 8.0 * rng.standard_normal(n) * math.sqrt(d) / 4
        v = round_to(rng.standard_normal((n, d)).astype(np.float32), dtype)
    else:
        s = rng.standard_normal(n)
        v = round_to(rng.standard_normal((n, d)).astype(np.float32), dtype)
    s = s.astype(np.float32).astype(np.float64)  # what an fp32 score holds
    O_ref, L_ref = oracle_row(s, v)
    O, L = kernel_model_row((s * LOG2E).astype(np.float32), v, kernel_pmax(dtype), dtype)
    tol = {"fp16": 5e-3, "bf16": 2e-2}[dtype]
    assert np.all(np.isfinite(O))
    assert np.abs(O - O_ref).max() <= tol
    assert abs(L - L_ref) <= 1e-3 + 1e-6 * abs(L_ref)


def test_fp16_bound_keeps_every_p_finite():
    # Every P of a lane is at most that lane's partial sum, so a bound at or below
    # fp16's largest finite value keeps each rounded P finite; and a rebase
    # leaves every P <= 1.
    assert kernel_pmax("fp16") <= 65504.0
    assert kernel_pmax("bf16") <= float(np.finfo(np.float32).max)
