"""Pins of the oracle's log-linear (Fenwick-tree) readout and its adaptive
level weights ("Technical summary: adaptive memory decay for log-linear
attention", "Problem definition" and "Methodology").

The level recurrence in lam_oracle.c is pinned to things outside it:
  * a brute-force definition, O(T^2) with explicit transition matrices:
    y_t = sum_{s<=t} lambda_t^{l(t,s)} (beta_s z_s k_s^T A_{s+1} ... A_t) q_t,
    A_r = D_r (I - beta_r e_r k_r^T), l(t,s) = 0 if s = t else
    msb(t xor s) + 1 -- token contributions tracked one by one, no levels;
  * lambda = 1 on every level gives the plain delta-rule scan (the oracle's
    own, pinned separately), and the levels sum to its memory;
  * lambda one-hot on level 0 reads only the fresh write: y_t = beta_t
    (k_t . q_t) z_t;
  * one call over [0, T) equals two chained calls (level states passed, the
    second starting at absolute position T1).
The softplus MLP is pinned by the page's initialisation (W2 = 0, bias 0.54
gives softplus(0.54) = log(1 + e^0.54), about 1) and a brute-force loop.
"""
import math

import numpy as np
import pytest

import oracle

VARIANTS = ["deltanet", "gdn", "kda", "gdn2"]


def _inputs(seed, variant, B=1, T=11, H=2, dk=4, dv=3, nL=None, t0=0):
    r = np.random.default_rng(seed)
    nL = nL or oracle.loglinear_levels(t0 + T - 1)
    x = {"q": r.standard_normal((B, T, H, dk)), "k": r.standard_normal((B, T, H, dk)) * 0.6,
         "v": r.standard_normal((B, T, H, dv)), "beta": r.uniform(0.2, 0.9, (B, T, H)),
         "lam": r.uniform(0.2, 1.5, (B, T, H, nL))}
    if variant == "kda":
        x["alpha"] = r.uniform(0.5, 1.0, (B, T, H, dk))
    elif variant != "deltanet":
        x["alpha"] = r.uniform(0.5, 1.0, (B, T, H))
    if variant == "gdn2":
        x["erase_b"] = r.uniform(0.1, 1.0, (B, T, H, dk))
        x["write_w"] = r.uniform(0.1, 1.0, (B, T, H, dv))
    return x


def _ll(variant, x, **kw):
    return oracle.loglinear_forward(variant, x["q"], x["k"], x["v"], x["beta"], x["lam"], alpha=x.get("alpha"),
                                    erase_b=x.get("erase_b"), write_w=x.get("write_w"), **kw)


def _level(t, s):
    return 0 if s == t else (t ^ s).bit_length()


def _brute(variant, x, b, h, t0=0):
    """The definition, token contributions one by one (no level states)."""
    q, k, v = x["q"][b, :, h], x["k"][b, :, h], x["v"][b, :, h]
    beta, lam = x["beta"][b, :, h], x["lam"][b, :, h]
    T, dk = q.shape
    e = k * (x["erase_b"][b, :, h] if variant == "gdn2" else 1.0)
    z = v * (x["write_w"][b, :, h] if variant == "gdn2" else 1.0)

    def A(r):
        if variant in ("gdn", "gdn2"):
            D = x["alpha"][b, r, h] * np.eye(dk)
        elif variant == "kda":
            D = np.diag(x["alpha"][b, r, h])
        else:
            D = np.eye(dk)
        return D @ (np.eye(dk) - beta[r] * np.outer(e[r], k[r]))

    y = np.zeros((T, v.shape[1]))
    for t in range(T):
        for s in range(t + 1):
            C = beta[s] * np.outer(z[s], k[s])
            for r in range(s + 1, t + 1):
                C = C @ A(r)
            y[t] += lam[t, _level(t0 + t, t0 + s)] * (C @ q[t])
    return y


@pytest.mark.parametrize("t0", [0, 5, 8])
@pytest.mark.parametrize("variant", VARIANTS)
def test_matches_brute_force_definition(variant, t0):
    x = _inputs(51 + VARIANTS.index(variant) + t0, variant, t0=t0)
    out, _ = _ll(variant, x, t0=t0)
    for h in range(2):
        np.testing.assert_allclose(out[0, :, h], _brute(variant, x, 0, h, t0=t0), rtol=1e-10, atol=1e-12,
                                   err_msg=f"{variant} t0={t0} h={h}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_unit_weights_give_the_plain_scan(variant):
    x = _inputs(61, variant, B=2, T=40)
    x["lam"][:] = 1.0
    r = np.random.default_rng(62)
    s0 = r.standard_normal((2, 2, 3, 4)) * 0.4
    nL = x["lam"].shape[3]
    lv = np.zeros((2, 2, nL, 3, 4))
    lv[:, :, nL - 1] = s0  # any split of the initial memory over the levels
    out, levels = _ll(variant, x, state_in=lv)
    ref, st = oracle.delta_forward(variant, x["q"], x["k"], x["v"], x["beta"], alpha=x.get("alpha"),
                                   erase_b=x.get("erase_b"), write_w=x.get("write_w"), state_in=s0)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(levels.sum(axis=2), st, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("variant", VARIANTS)
def test_level_zero_reads_the_fresh_write(variant):
    x = _inputs(71, variant, T=20)
    x["lam"][:] = 0.0
    x["lam"][..., 0] = 1.0
    out, _ = _ll(variant, x)
    z = x["v"] * (x["write_w"] if variant == "gdn2" else 1.0)
    want = (x["beta"] * np.sum(x["k"] * x["q"], -1))[..., None] * z
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T1", [1, 7, 8, 13])
@pytest.mark.parametrize("variant", VARIANTS)
def test_chained_calls(variant, T1):
    x = _inputs(81, variant, B=2, T=29)
    out, lv = _ll(variant, x)
    a = {k_: v_[:, :T1] for k_, v_ in x.items()}
    b = {k_: v_[:, T1:] for k_, v_ in x.items()}
    o1, l1 = _ll(variant, a)
    o2, l2 = _ll(variant, b, state_in=l1, t0=T1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, lv, rtol=1e-12, atol=1e-13)


def test_fenwick_occupancy():
    """Every token's write sits at the level the Fenwick partition gives it:
    DeltaNet with one value slot per token and a tiny beta (so the writes
    barely erase one another) leaves, after the last token, value slot s
    held by level msb((T-1) xor s) + 1 alone (level 0 for s = T-1)."""
    T, nL = 13, oracle.loglinear_levels(12)
    k = np.zeros((1, T, 1, 4))
    k[..., 0] = 1.0
    # orthogonal writes cannot interfere: give each token its own value slot
    v = np.zeros((1, T, 1, T))
    for t in range(T):
        v[0, t, 0, t] = 1.0
    _, lv = oracle.loglinear_forward("deltanet", np.ones((1, T, 1, 4)), k, v, np.full((1, T, 1), 1e-9),
                                     np.ones((1, T, 1, nL)))
    # with tiny beta the writes barely erase each other: each value slot t is
    # held by exactly one level, the one Fenwick assigns token t for query T - 1
    for t in range(T):
        holder = np.flatnonzero(np.abs(lv[0, 0, :, t, 0]) > 1e-12)
        assert list(holder) == [_level(T - 1, t)], (t, holder)


def test_lambda_initialisation_is_near_identity():
    """W2 = 0 and bias 0.54: every weight is softplus(0.54) = 0.99916."""
    nL = 13
    lam = oracle.loglinear_lambda(np.random.default_rng(1).standard_normal((5, nL)),
                                  np.random.default_rng(2).standard_normal((nL, 2 * nL)),
                                  np.zeros((2 * nL, nL)), np.full(nL, 0.54))
    np.testing.assert_allclose(lam, math.log1p(math.exp(0.54)), rtol=1e-15)
    assert abs(lam[0, 0] - 0.99916) < 1e-5


def test_lambda_brute_force_and_tails():
    r = np.random.default_rng(3)
    nL, nh = 4, 8
    d, W1, W2, b = r.standard_normal((3, nL)), r.standard_normal((nL, nh)), r.standard_normal((nh, nL)), \
        r.standard_normal(nL)
    got = oracle.loglinear_lambda(d, W1, W2, b)
    for i in range(3):
        for l in range(nL):
            x = b[l] + sum(sum(d[i, a] * W1[a, j] for a in range(nL)) * W2[j, l] for j in range(nh))
            assert abs(got[i, l] - math.log(1.0 + math.exp(x))) <= 1e-13 * max(1.0, abs(x))
    # far tails: softplus(x) -> x and -> e^x without overflow
    big = oracle.loglinear_lambda(np.array([[1.0]]), np.array([[1.0]]), np.array([[1.0]]), np.array([59.0]))
    small = oracle.loglinear_lambda(np.array([[1.0]]), np.array([[1.0]]), np.array([[1.0]]), np.array([-61.0]))
    np.testing.assert_allclose(big, 60.0, rtol=1e-15)
    np.testing.assert_allclose(small, math.exp(-60.0), rtol=1e-12)
