"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, brute force on tiny inputs, a special case that reduces to another
variant or to a library routine (numpy.linalg.inv, torch's ELU), or an
invariant stated on the pages.  A plausible slip anywhere in the oracle (a
dropped term, a wrong sign or index, a transposed operand, reading before
instead of after the write) fails at least one of them.

Sources:
  linear-attention architectures page = "Mechanisms, trade-offs and
    cross-layer routing of linear-attention architectures" (aitrends.kr):
    "Understanding the core idea", "Methodology", "Technical details".
  VLA page = "Technical summary: Variational Linear Attention (VLA)"
    (gist.science): sections 2.1-2.3 and 3.1.
"""
import numpy as np
import pytest

import oracle
from tests import chunked_model

rng0 = np.random.default_rng


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_delta(seed, B=2, T=12, H=3, dk=8, dv=6, variant="gdn", weak=False):
    r = rng0(seed)
    q = _unit(r.standard_normal((B, T, H, dk)))
    k = _unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    mu = -3.0 if weak else 0.5
    if variant == "kda":
        alpha = 1 / (1 + np.exp(r.standard_normal((B, T, H, dk)) + mu))
    else:
        alpha = 1 / (1 + np.exp(r.standard_normal((B, T, H)) + mu))
    eb = 1 / (1 + np.exp(-r.standard_normal((B, T, H, dk))))
    ww = 1 / (1 + np.exp(-r.standard_normal((B, T, H, dv))))
    s0 = r.standard_normal((B, H, dv, dk)) * 0.3
    return dict(q=q, k=k, v=v, beta=beta, alpha=alpha, erase_b=eb, write_w=ww, state_in=s0)


def _run(variant, d, **over):
    a = dict(d)
    a.update(over)
    return oracle.delta_forward(variant, a["q"], a["k"], a["v"], a["beta"], alpha=a["alpha"],
                                erase_b=a["erase_b"], write_w=a["write_w"],
                                state_in=a["state_in"], drop_delta=a.get("drop_delta", False))


# ---------------------------------------------------------------- P-1 recall
def test_deltanet_orthonormal_recall():
    """DeltaNet with beta = 1 and orthonormal keys stores each pair exactly:
    W_T k_i = v_i and a query equal to key s reads v_s once s has been written,
    zero before (delta rule, 'Understanding the core idea')."""
    r = rng0(1)
    d, T, dv = 8, 8, 5
    Kb, _ = np.linalg.qr(r.standard_normal((d, d)))
    keys = Kb.T[:T]                                   # orthonormal rows
    v = r.standard_normal((T, dv))
    s_idx = r.integers(0, T, size=T)
    q = keys[s_idx]
    out, st = oracle.delta_forward("deltanet", q[None, :, None], keys[None, :, None],
                                   v[None, :, None], np.ones((1, T, 1)))
    W = st[0, 0]
    np.testing.assert_allclose(W @ keys.T, v.T, atol=1e-12)
    np.testing.assert_allclose(W, v.T @ keys, atol=1e-12)
    for t in range(T):
        want = v[s_idx[t]] if s_idx[t] <= t else np.zeros(dv)
        np.testing.assert_allclose(out[0, t, 0], want, atol=1e-12)


def test_deltanet_rewrite_replaces_value():
    """Writing the same unit key twice with beta = 1 replaces the stored value
    (the residual r = v - W k removes the old association); plain additive
    accumulation would return the sum."""
    r = rng0(2)
    k = _unit(r.standard_normal(6))
    v1, v2 = r.standard_normal(4), r.standard_normal(4)
    K = np.stack([k, k])[None, :, None]
    V = np.stack([v1, v2])[None, :, None]
    out, st = oracle.delta_forward("deltanet", K, K, V, np.ones((1, 2, 1)))
    np.testing.assert_allclose(out[0, 1, 0], v2, atol=1e-12)
    np.testing.assert_allclose(st[0, 0], np.outer(v2, k), atol=1e-12)
    out_la, _ = oracle.delta_forward("deltanet", K, K, V, np.ones((1, 2, 1)), drop_delta=True)
    np.testing.assert_allclose(out_la[0, 1, 0], v1 + v2, atol=1e-12)


def test_gdn_orthonormal_recall_decays():
    """Gated DeltaNet, beta = 1, orthonormal keys: the pair written at s is
    read at t >= s scaled by prod_{j=s+1..t} alpha_j (scalar decay,
    'Technical details')."""
    r = rng0(3)
    d, T = 6, 6
    Kb, _ = np.linalg.qr(r.standard_normal((d, d)))
    keys = Kb.T
    v = r.standard_normal((T, 3))
    alpha = r.uniform(0.3, 1.0, T)
    s_idx = r.integers(0, T, size=T)
    out, st = oracle.delta_forward("gdn", keys[s_idx][None, :, None], keys[None, :, None],
                                   v[None, :, None], np.ones((1, T, 1)),
                                   alpha=alpha[None, :, None])
    for t in range(T):
        s = s_idx[t]
        want = v[s] * np.prod(alpha[s + 1:t + 1]) if s <= t else np.zeros(3)
        np.testing.assert_allclose(out[0, t, 0], want, atol=1e-12)
    W = sum(np.prod(alpha[s + 1:]) * np.outer(v[s], keys[s]) for s in range(T))
    np.testing.assert_allclose(st[0, 0], W, atol=1e-12)


def test_kda_basis_keys_channel_decay():
    """Kimi Delta with basis keys e_c (distinct channels), beta = 1: the pair
    written at s on channel c is read at t scaled by prod_{j=s+1..t}
    alpha_j[c] -- each key channel forgets at its own rate."""
    r = rng0(4)
    d, T = 5, 5
    perm = r.permutation(d)[:T]
    keys = np.eye(d)[perm]
    v = r.standard_normal((T, 2))
    alpha = r.uniform(0.2, 1.0, (T, d))
    out, st = oracle.delta_forward("kda", keys[None, :, None], keys[None, :, None],
                                   v[None, :, None], np.ones((1, T, 1)),
                                   alpha=alpha[None, :, None])
    for t in range(T):
        c = perm[t]
        np.testing.assert_allclose(out[0, t, 0], v[t], atol=1e-12)   # q_t = k_t
    for s in range(T):
        c = perm[s]
        np.testing.assert_allclose(st[0, 0][:, c], v[s] * np.prod(alpha[s + 1:, c]), atol=1e-12)


# ------------------------------------------------------- P-2 brute force
def _brute_gated(q, k, v, beta, alpha_scalar=None, alpha_chan=None, W0=None, target=None):
    """O(T^2) sum of per-pair contributions with the delta term dropped."""
    T, dk = k.shape
    dv = v.shape[1]
    tgt = v if target is None else target
    Y = np.zeros((T, dv))
    for t in range(T):
        for s in range(t + 1):
            if alpha_chan is not None:
                g = np.prod(alpha_chan[s + 1:t + 1], axis=0) if t > s else np.ones(dk)
                Y[t] += beta[s] * tgt[s] * np.dot(q[t], k[s] * g)
            else:
                g = np.prod(alpha_scalar[s + 1:t + 1]) if alpha_scalar is not None else 1.0
                Y[t] += beta[s] * g * np.dot(q[t], k[s]) * tgt[s]
        if W0 is not None:
            if alpha_chan is not None:
                Y[t] += W0 @ (np.prod(alpha_chan[:t + 1], axis=0) * q[t])
            elif alpha_scalar is not None:
                Y[t] += np.prod(alpha_scalar[:t + 1]) * (W0 @ q[t])
            else:
                Y[t] += W0 @ q[t]
    return Y


@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda", "gdn2"])
def test_drop_delta_matches_brute_force(variant):
    """With the delta term dropped the scan is plain (gated) linear attention,
    S_t = S_{t-1} + v_t k_t^T (VLA page, section 2.1), so y_t is the causal sum
    over s <= t of beta_s (decay from s+1 to t) (q_t . k_s) target_s, plus the
    decayed initial memory read -- checked by O(T^2) brute force."""
    d = _rand_delta({"deltanet": 10, "gdn": 11, "kda": 12, "gdn2": 13}[variant], B=1, T=9, H=1,
                    variant=variant)
    out, _ = _run(variant, d, drop_delta=True)
    q, k, v = d["q"][0, :, 0], d["k"][0, :, 0], d["v"][0, :, 0]
    be = d["beta"][0, :, 0]
    W0 = d["state_in"][0, 0]
    if variant == "deltanet":
        Y = _brute_gated(q, k, v, be, W0=W0)
    elif variant == "gdn":
        Y = _brute_gated(q, k, v, be, alpha_scalar=d["alpha"][0, :, 0], W0=W0)
    elif variant == "kda":
        Y = _brute_gated(q, k, v, be, alpha_chan=d["alpha"][0, :, 0], W0=W0)
    else:
        Y = _brute_gated(q, k, v, be, alpha_scalar=d["alpha"][0, :, 0], W0=W0,
                         target=d["write_w"][0, :, 0] * v)
    np.testing.assert_allclose(out[0, :, 0], Y, atol=1e-12, rtol=1e-12)


def test_plain_linear_attention_unit_gates():
    """alpha = 1, beta = 1, delta dropped: y_t = sum_{s<=t} (q_t . k_s) v_s
    exactly, the additive accumulation of standard linear attention."""
    r = rng0(11)
    T, dk, dv = 10, 4, 3
    q, k, v = r.standard_normal((T, dk)), r.standard_normal((T, dk)), r.standard_normal((T, dv))
    out, st = oracle.delta_forward("deltanet", q[None, :, None], k[None, :, None], v[None, :, None],
                                   np.ones((1, T, 1)), drop_delta=True)
    Y = np.tril(q @ k.T) @ v
    np.testing.assert_allclose(out[0, :, 0], Y, atol=1e-12)
    np.testing.assert_allclose(st[0, 0], v.T @ k, atol=1e-12)


# ---------------------------------------------------- P-3 reductions
def test_gdn2_unit_gates_is_gdn():
    d = _rand_delta(20, variant="gdn2")
    ones_b = np.ones_like(d["erase_b"])
    ones_w = np.ones_like(d["write_w"])
    a = _run("gdn2", d, erase_b=ones_b, write_w=ones_w)
    b = _run("gdn", d)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)


def test_kda_equal_channels_is_gdn():
    d = _rand_delta(21, variant="gdn")
    ach = np.repeat(d["alpha"][..., None], d["q"].shape[3], axis=3)
    a = _run("kda", d, alpha=ach)
    b = _run("gdn", d)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)


def test_gdn_unit_decay_is_deltanet():
    d = _rand_delta(22, variant="gdn")
    a = _run("gdn", d, alpha=np.ones_like(d["alpha"]))
    b = _run("deltanet", d)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)


def _elu1(x):
    import torch

    return (torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0) + 1.0).numpy()


def test_vla_zero_penalty_is_deltanet_on_features():
    """With p = 0 the penalty never grows, A stays I, alpha-hat = k-hat, and
    VLA's rule 3 is DeltaNet with beta = 1 on the unit ELU+1 features (VLA page
    section 2.3).  The features come from torch's ELU, a library routine."""
    r = rng0(23)
    B, T, H, d = 1, 14, 2, 6
    q, k, v = (r.standard_normal((B, T, H, d)) for _ in range(3))
    out, A, S = oracle.vla_forward(q, k, v, np.zeros((B, T, H, d)))
    kh, qh = _unit(_elu1(k)), _unit(_elu1(q))
    o2, s2 = oracle.delta_forward("deltanet", qh, kh, v, np.ones((B, T, H)))
    np.testing.assert_allclose(out, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, s2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(A, np.broadcast_to(np.eye(d), A.shape), atol=0)


# ------------------------------------------------------ P-4 edge cases
@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda", "gdn2"])
def test_zero_beta_only_decays(variant):
    """beta = 0 writes nothing: W_t is the initial memory under the decays
    accumulated so far, and y_t reads it."""
    d = _rand_delta(30, B=1, T=7, H=1, variant=variant)
    out, st = _run(variant, d, beta=np.zeros_like(d["beta"]))
    W0 = d["state_in"][0, 0]
    for t in range(7):
        if variant == "kda":
            Wt = W0 * np.prod(d["alpha"][0, :t + 1, 0], axis=0)[None, :]
        elif variant == "deltanet":
            Wt = W0
        else:
            Wt = W0 * np.prod(d["alpha"][0, :t + 1, 0])
        np.testing.assert_allclose(out[0, t, 0], Wt @ d["q"][0, t, 0], atol=1e-13)
    np.testing.assert_allclose(st[0, 0], Wt, atol=1e-13)


def test_gdn_zero_decay_forgets_everything():
    """alpha = 0 clears the memory before each write: y_t = beta_t (k_t . q_t) v_t."""
    d = _rand_delta(31, B=1, T=6, H=1, variant="gdn")
    out, _ = _run("gdn", d, alpha=np.zeros_like(d["alpha"]))
    q, k, v, be = d["q"][0, :, 0], d["k"][0, :, 0], d["v"][0, :, 0], d["beta"][0, :, 0]
    want = (be * np.sum(k * q, axis=1))[:, None] * v
    np.testing.assert_allclose(out[0, :, 0], want, atol=1e-13)


def test_empty_sequence_passes_state_through():
    d = _rand_delta(32, B=2, T=0, H=2, variant="gdn")
    out, st = _run("gdn", d)
    assert out.shape == (2, 0, 2, 6)
    np.testing.assert_array_equal(st, d["state_in"])


# ------------------------------------------ P-5 per-step residual identities
@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda", "gdn2"])
def test_per_step_residual_identity(variant):
    """After one write, the memory's new prediction error along the read key
    shrinks by the factor (1 - beta k.kk): W_t kk_t - target_t =
    (1 - beta_t k_t.kk_t)(W~_{t-1} kk_t - target_t), with kk = k (kk = b*k,
    target = w*v for Gated DeltaNet-2) and W~ the decayed memory.  Any sign,
    beta or key slip in the write breaks it."""
    d = _rand_delta(40 + len(variant), B=1, T=8, H=1, variant=variant)
    W = d["state_in"].copy()
    for t in range(8):
        sl = lambda x: None if x is None else x[:, t:t + 1]
        _, Wn = oracle.delta_forward(variant, sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["beta"]),
                                     alpha=sl(d["alpha"]), erase_b=sl(d["erase_b"]),
                                     write_w=sl(d["write_w"]), state_in=W)
        k = d["k"][0, t, 0]
        be = d["beta"][0, t, 0]
        kk, tgt = k, d["v"][0, t, 0]
        Wp = W[0, 0]
        if variant == "gdn" or variant == "gdn2":
            Wp = d["alpha"][0, t, 0] * Wp
        elif variant == "kda":
            Wp = Wp * d["alpha"][0, t, 0][None, :]
        if variant == "gdn2":
            kk = d["erase_b"][0, t, 0] * k
            tgt = d["write_w"][0, t, 0] * tgt
        lhs = Wn[0, 0] @ kk - tgt
        rhs = (1 - be * np.dot(k, kk)) * (Wp @ kk - tgt)
        np.testing.assert_allclose(lhs, rhs, atol=1e-12)
        # and nothing changes orthogonally to the write key
        perp = rng0(t).standard_normal(k.shape[0])
        perp = perp - np.dot(perp, k) / np.dot(k, k) * k
        np.testing.assert_allclose(Wn[0, 0] @ perp, Wp @ perp, atol=1e-12)
        W = Wn


def test_vla_per_step_residual_identity():
    """VLA rule 3: S_t khat_t - v_t = (1 - alpha-hat . khat)(S_{t-1} khat_t - v_t)."""
    r = rng0(45)
    T, d = 10, 5
    q, k, v = (r.standard_normal((1, T, 1, d)) for _ in range(3))
    p = r.standard_normal((1, T, 1, d)) / np.sqrt(d)
    S = np.zeros((1, 1, d, d))
    A = np.broadcast_to(np.eye(d), (1, 1, d, d)).copy()
    for t in range(T):
        sl = lambda x: x[:, t:t + 1]
        _, An, Sn, dg = oracle.vla_forward(sl(q), sl(k), sl(v), sl(p), A_in=A, S_in=S, diagnostics=True)
        kh, ah = dg["khat"][0, 0, 0], dg["ahat"][0, 0, 0]
        lhs = Sn[0, 0] @ kh - v[0, t, 0]
        rhs = (1 - ah @ kh) * (S[0, 0] @ kh - v[0, t, 0])
        np.testing.assert_allclose(lhs, rhs, atol=1e-12)
        A, S = An, Sn


# ---------------------------------------------------- P-6 Sherman-Morrison
@pytest.mark.parametrize("d,T", [(4, 8), (32, 64)])
def test_sherman_morrison_equals_explicit_inverse(d, T):
    """A_t, kept by rank-1 Sherman-Morrison downdates, equals the explicit
    inverse of M_t = I + sum_{s<=t} p_s p_s^T (VLA page, section 2.2), and the
    denominator of step t is 1 + p_t^T M_{t-1}^{-1} p_t."""
    r = rng0(50 + d)
    p = r.standard_normal((1, T, 1, d)) / np.sqrt(d)
    q, k, v = (r.standard_normal((1, T, 1, d)) for _ in range(3))
    for t_end in (1, T // 2, T):
        sl = lambda x: x[:, :t_end]
        _, A, _, dg = oracle.vla_forward(sl(q), sl(k), sl(v), sl(p), diagnostics=True)
        P = p[0, :t_end, 0]
        M = np.eye(d) + P.T @ P
        np.testing.assert_allclose(A[0, 0], np.linalg.inv(M), rtol=1e-12, atol=1e-12)
        Mp = np.eye(d) + P[:-1].T @ P[:-1]
        np.testing.assert_allclose(dg["den"][0, -1, 0], 1 + P[-1] @ np.linalg.inv(Mp) @ P[-1],
                                   rtol=1e-12)


def test_vla_gate_is_normalised_inverse_penalty_times_key():
    """Rule 2: alpha-hat_t = M_t^{-1} khat_t / |M_t^{-1} khat_t| with M_t built
    explicitly (not by the downdate), and khat = unit ELU+1 feature of k
    (torch's ELU)."""
    r = rng0(55)
    T, d = 12, 7
    q, k, v = (r.standard_normal((1, T, 1, d)) for _ in range(3))
    p = r.standard_normal((1, T, 1, d)) / np.sqrt(d)
    _, _, _, dg = oracle.vla_forward(q, k, v, p, diagnostics=True)
    kh = _unit(_elu1(k))
    qh = _unit(_elu1(q))
    np.testing.assert_allclose(dg["khat"], kh, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dg["qhat"], qh, rtol=1e-13, atol=1e-15)
    for t in range(T):
        P = p[0, :t + 1, 0]
        a = np.linalg.inv(np.eye(d) + P.T @ P) @ kh[0, t, 0]
        np.testing.assert_allclose(dg["ahat"][0, t, 0], a / np.linalg.norm(a), rtol=1e-11, atol=1e-12)


# ----------------------------------------------- P-7 / P-8 invariants
def test_vla_normalisation_invariants_and_jacobian_spectrum():
    """Unit k-hat, q-hat, alpha-hat (VLA page, section 2.3); 0 < alpha-hat .
    khat <= 1 since A is SPD; 1 + p^T z >= 1; eig(A) in (0, 1]; and the step
    Jacobian I - alpha-hat khat^T (section 3.1, proposition 2) has spectral
    radius 1: eigenvalues 1 (d-1 times) and 1 - alpha-hat . khat."""
    r = rng0(60)
    B, T, H, d = 2, 40, 2, 8
    q, k, v = (r.standard_normal((B, T, H, d)) for _ in range(3))
    p = r.standard_normal((B, T, H, d)) / np.sqrt(d)
    _, A, _, dg = oracle.vla_forward(q, k, v, p, diagnostics=True)
    for n in ("khat", "qhat", "ahat"):
        np.testing.assert_allclose(np.linalg.norm(dg[n], axis=-1), 1.0, rtol=1e-13)
    c = np.sum(dg["ahat"] * dg["khat"], axis=-1)
    assert np.all(c > 0) and np.all(c <= 1 + 1e-13)
    assert np.all(dg["den"] >= 1.0)
    ev = np.linalg.eigvalsh(A.reshape(-1, d, d))
    assert np.all(ev > 0) and np.all(ev <= 1 + 1e-12)
    for b, t, h in [(0, 0, 0), (1, 17, 1), (0, 39, 1)]:
        J = np.eye(d) - np.outer(dg["ahat"][b, t, h], dg["khat"][b, t, h])
        e = np.sort(np.linalg.eigvals(J).real)
        want = np.sort(np.r_[np.ones(d - 1), 1 - c[b, t, h]])
        np.testing.assert_allclose(e, want, atol=1e-12)
        assert abs(max(abs(np.linalg.eigvals(J))) - 1) < 1e-12


# ------------------------------------------------------------ P-9 resume
@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda", "gdn2"])
def test_chained_calls_equal_one_call(variant):
    """Streaming: [0, T) in one call equals [0, T1) then [T1, T) chained
    through the state (fixed-size memory, no KV cache)."""
    d = _rand_delta(70, B=2, T=11, H=2, variant=variant)
    out, st = _run(variant, d)
    sl = lambda x, a, b: x[:, a:b]
    keys = ("q", "k", "v", "beta", "alpha", "erase_b", "write_w")
    d1 = dict(d, **{n: sl(d[n], 0, 4) for n in keys})
    o1, s1 = _run(variant, d1)
    d2 = dict(d, **{n: sl(d[n], 4, 11) for n in keys}, state_in=s1)
    o2, s2 = _run(variant, d2)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), out, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s2, st, rtol=1e-13, atol=1e-13)


def test_vla_chained_calls_equal_one_call():
    r = rng0(71)
    B, T, H, d = 1, 15, 2, 5
    q, k, v = (r.standard_normal((B, T, H, d)) for _ in range(3))
    p = r.standard_normal((B, T, H, d)) / np.sqrt(d)
    out, A, S = oracle.vla_forward(q, k, v, p)
    o1, A1, S1 = oracle.vla_forward(q[:, :6], k[:, :6], v[:, :6], p[:, :6])
    o2, A2, S2 = oracle.vla_forward(q[:, 6:], k[:, 6:], v[:, 6:], p[:, 6:], A_in=A1, S_in=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), out, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(A2, A, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S2, S, rtol=1e-13, atol=1e-13)


# ------------------------------------ decode: one token at a time (P-9)
@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda", "gdn2"])
def test_token_by_token_equals_one_call(variant):
    """A decode step is the scan over one token with the state carried in and
    out: T one-token calls chained through the state give the T-token scan."""
    d = _rand_delta(72, B=2, T=9, H=2, variant=variant)
    out, st = _run(variant, d)
    keys = ("q", "k", "v", "beta", "alpha", "erase_b", "write_w")
    state, outs = d.get("state_in"), []
    for t in range(9):
        dt = dict(d, **{n: d[n][:, t:t + 1] for n in keys if d.get(n) is not None}, state_in=state)
        o, state = _run(variant, dt)
        outs.append(o)
    np.testing.assert_allclose(np.concatenate(outs, axis=1), out, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(state, st, rtol=1e-13, atol=1e-13)


def test_vla_token_by_token_equals_one_call():
    r = rng0(73)
    B, T, H, d = 1, 8, 2, 5
    q, k, v = (r.standard_normal((B, T, H, d)) for _ in range(3))
    p = r.standard_normal((B, T, H, d)) / np.sqrt(d)
    out, A, S = oracle.vla_forward(q, k, v, p)
    A_t = S_t = None
    outs = []
    for t in range(T):
        o, A_t, S_t = oracle.vla_forward(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], p[:, t:t + 1],
                                         A_in=A_t, S_in=S_t)
        outs.append(o)
    np.testing.assert_allclose(np.concatenate(outs, 1), out, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(A_t, A, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S_t, S, rtol=1e-13, atol=1e-13)


# ---------------------------------------- layout, causality, independence
@pytest.mark.parametrize("variant", ["gdn", "kda", "gdn2"])
def test_chains_are_independent_and_layout_is_row_major(variant):
    """Each (b, h) chain computed alone equals its slice of the batched call
    (catches stride/index slips in the [B,T,H,d] and [B,H,dv,dk] layouts)."""
    d = _rand_delta(80, B=2, T=5, H=3, variant=variant)
    out, st = _run(variant, d)
    for b in range(2):
        for h in range(3):
            one = {n: (x[b:b + 1, :, h:h + 1] if n != "state_in" else x[b:b + 1, h:h + 1])
                   for n, x in d.items()}
            o, s = _run(variant, one)
            np.testing.assert_array_equal(o[0, :, 0], out[b, :, h])
            np.testing.assert_array_equal(s[0, 0], st[b, h])


def test_causality():
    d = _rand_delta(81, B=1, T=10, H=1, variant="gdn2")
    out, _ = _run("gdn2", d)
    d2 = {n: x.copy() for n, x in d.items()}
    for n in ("q", "k", "v", "beta", "alpha", "erase_b", "write_w"):
        d2[n][:, 6:] = d2[n][:, 6:] * 0.5 + 0.1
    out2, _ = _run("gdn2", d2)
    np.testing.assert_array_equal(out[:, :6], out2[:, :6])
    assert not np.allclose(out[:, 6:], out2[:, 6:])


# ----------------------------------------------- P-10 chunk algebra
@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda", "gdn2"])
@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunked_form_equals_recurrence(variant, C):
    """The chunkwise-parallel rewrite the HIP kernels evaluate (test-only
    numpy model) equals the token-by-token oracle to ~1e-12 relative, at a
    ragged length spanning several chunks."""
    d = _rand_delta(90, B=1, T=83, H=2, dk=16, dv=12, variant=variant, weak=True)
    out, st = _run(variant, d)
    o2, s2 = chunked_model.delta_chunked(variant, d["q"], d["k"], d["v"], d["beta"], alpha=d["alpha"],
                                         erase_b=d["erase_b"], write_w=d["write_w"],
                                         state_in=d["state_in"], C=C)
    scale = np.max(np.abs(out))
    assert np.max(np.abs(o2 - out)) <= 1e-12 * scale
    assert np.max(np.abs(s2 - st)) <= 1e-12 * np.max(np.abs(st))


@pytest.mark.parametrize("T", [5, 16, 32, 47, 83])
def test_kda_paired_form_equals_recurrence(T):
    """Kimi Delta stepped over pairs of 16-token sub-chunks (the chunked
    kernel's form: pair-relative tiles, cross blocks split at the sub-chunk
    boundary, U1 coupled to U0 through -T11 G10) equals the token-by-token
    oracle to ~1e-12 relative, for lengths that end inside the even or the
    odd sub-chunk of the last pair, with a carried-in state."""
    d = _rand_delta(93, B=1, T=T, H=2, dk=16, dv=12, variant="kda", weak=False)
    out, st = _run("kda", d)
    o2, s2 = chunked_model.kda_paired(d["q"], d["k"], d["v"], d["beta"], d["alpha"], state_in=d["state_in"])
    assert np.max(np.abs(o2 - out)) <= 1e-12 * np.max(np.abs(out))
    assert np.max(np.abs(s2 - st)) <= 1e-12 * np.max(np.abs(st))


@pytest.mark.parametrize("scale", [0.3, 3.0, 30.0])
def test_kda_level_blocks_equal_direct(scale):
    """The reference-token levels that form Kimi Delta's decayed Gram blocks
    without overflow cover every (t, s) with s <= t exactly once and equal
    the direct per-channel sum, also for decays far below 2^-100 per chunk."""
    r = rng0(92)
    n, dk = 16, 24
    K, Q = r.standard_normal((n, dk)), r.standard_normal((n, dk))
    lg = np.cumsum(-scale * r.exponential(size=(n, dk)), axis=0)
    Akk, Aqk = chunked_model.kda_blocks_by_levels(K, Q, lg)
    t, s = np.tril_indices(n)
    direct_k = np.zeros((n, n))
    direct_q = np.zeros((n, n))
    for i, j in zip(t, s):
        w = np.exp(lg[i] - lg[j])
        direct_q[i, j] = np.sum(Q[i] * K[j] * w)
        if i > j:
            direct_k[i, j] = np.sum(K[i] * K[j] * w)
    np.testing.assert_allclose(Akk, direct_k, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Aqk, direct_q, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_vla_chunked_form_equals_recurrence(C):
    r = rng0(91)
    B, T, H, d = 1, 77, 2, 8
    q, k, v = (r.standard_normal((B, T, H, d)) for _ in range(3))
    p = r.standard_normal((B, T, H, d)) / np.sqrt(d)
    out, A, S = oracle.vla_forward(q, k, v, p)
    o2, A2, S2 = chunked_model.vla_chunked(q, k, v, p, C=C)
    assert np.max(np.abs(o2 - out)) <= 1e-11 * np.max(np.abs(out))
    assert np.max(np.abs(A2 - A)) <= 1e-11
    assert np.max(np.abs(S2 - S)) <= 1e-11 * np.max(np.abs(S))


# ------------------------------------------- P-11 bounded state (soft)
def test_vla_state_stays_bounded_where_linear_attention_grows():
    """Proposition 1 (VLA page, section 3.1): VLA's |S_t|_F is self-limiting
    under bounded inputs, while plain linear attention keeps growing (O(T) in
    the worst case; like sqrt(T) here, since the values have zero mean).
    Soft check on a 32-dim head from 256 to 2048 tokens."""
    r = rng0(100)
    T, d = 2048, 32
    q, k, v = (r.standard_normal((1, T, 1, d)) for _ in range(3))
    p = r.standard_normal((1, T, 1, d)) / np.sqrt(d)
    kh = _unit(_elu1(k))
    vla, la = [], []
    for t_end in (256, 2048):
        _, _, S = oracle.vla_forward(q[:, :t_end], k[:, :t_end], v[:, :t_end], p[:, :t_end])
        vla.append(np.linalg.norm(S))
        _, Sla = oracle.delta_forward("deltanet", kh[:, :t_end], kh[:, :t_end], v[:, :t_end],
                                      np.ones((1, t_end, 1)), drop_delta=True)
        la.append(np.linalg.norm(Sla))
    assert vla[1] < 1.25 * vla[0]
    assert la[1] > 2.0 * la[0]
    assert la[1] > 5.0 * vla[1]


# ------------------------------------------- P-12 single-precision spread
@pytest.mark.parametrize("name", ["deltanet_f32_B1_T256_H2_d32", "vla_f32_B4_T4096_H8_d32",
                                  "vla_f32_B4_T4096_H8_d96"])
def test_single_precision_spread_is_below_the_gate(name):
    """The same scan evaluated in float32 stays within 1e-5 (max-normalised) of
    float64 on the fp32 workloads (two chains of the VLA ones), so the 1e-4
    fp32 parity gate is reachable with fp32 arithmetic."""
    from gated_linear_attention_chunked_amd import inputs as I

    w = I.WORKLOADS[name]
    if w.variant == "vla":
        w = w.replace(B=1, H=2)
    x = I.make_inputs(w)
    if w.variant == "vla":
        r64 = oracle.vla_forward(x["q"], x["k"], x["v"], x["p"])
        r32 = oracle.vla_forward(x["q"], x["k"], x["v"], x["p"], precision="f32")
    else:
        r64 = oracle.delta_forward(w.variant, x["q"], x["k"], x["v"], x["beta"])
        r32 = oracle.delta_forward(w.variant, x["q"], x["k"], x["v"], x["beta"], precision="f32")
    assert oracle.real_bytes("f32") == 4 and oracle.real_bytes("f64") == 8
    for a, b in zip(r64, r32):
        assert np.max(np.abs(a - b)) <= 1e-5 * np.max(np.abs(a))
