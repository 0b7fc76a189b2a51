"""Pins of the oracle's VLA ratio read ("Technical summary: Variational
Linear Attention (VLA)", section 2.3: the output is a ratio of recurrences as
in standard linear attention).

The denominator n follows the write rule with the value 1, so the pins tie
it to the plain VLA oracle (pinned separately) rather than to itself:
  * with every value channel set to 1 the plain scan's state rows all equal
    n, and its output equals n . q-hat in every channel, so
    y_ratio = y_plain(v) / y_plain(ones) elementwise, with the same A and S;
  * orthonormal feature keys with p = 0 (A stays I, alpha-hat = k-hat) and
    q = k recall exactly: S k-hat_t = v_t and n . k-hat_t = 1, so the ratio
    output is v_t;
  * one call equals two calls chained through (A, S, n);
  * a missing n_in is a zero denominator state: after the first token
    n = alpha-hat.
"""
import numpy as np
import pytest

import oracle


def _inputs(seed, B=2, T=23, H=2, d=8):
    r = np.random.default_rng(seed)
    return {"q": r.standard_normal((B, T, H, d)), "k": r.standard_normal((B, T, H, d)),
            "v": r.standard_normal((B, T, H, d)), "p": r.standard_normal((B, T, H, d)) / np.sqrt(d)}


@pytest.mark.parametrize("d", [4, 8, 32])
def test_ratio_is_plain_over_plain_of_ones(d):
    x = _inputs(11 + d, d=d)
    r = np.random.default_rng(5)
    A0 = np.eye(d) * 0.9 + 0.0
    A0 = np.broadcast_to(A0, (2, 2, d, d)).copy()
    S0 = r.standard_normal((2, 2, d, d)) * 0.3
    n0 = r.standard_normal((2, 2, d)) * 0.1
    y, A, S, n = oracle.vla_forward_ratio(x["q"], x["k"], x["v"], x["p"], A_in=A0, S_in=S0, n_in=n0)
    y_num, A_p, S_p = oracle.vla_forward(x["q"], x["k"], x["v"], x["p"], A_in=A0, S_in=S0)
    ones = np.ones_like(x["v"])
    N0 = np.repeat(n0[:, :, None, :], d, axis=2)  # every value row starts at n0
    y_den, _, N = oracle.vla_forward(x["q"], x["k"], ones, x["p"], A_in=A0, S_in=N0)
    np.testing.assert_allclose(y_den, y_den[..., :1] * np.ones(d), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(y, y_num / y_den, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(A, A_p, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S, S_p, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(n, N[:, :, 0, :], rtol=1e-12, atol=1e-13)


def test_orthonormal_keys_recall_exactly():
    """Raw keys +30 on channel t and -30 elsewhere: ELU+1 gives 31 e_t plus
    e^-30 on the other channels, so k-hat_t = e_t to ~1e-13."""
    d, T = 16, 12
    k = np.full((1, T, 1, d), -30.0)
    for t in range(T):
        k[0, t, 0, t] = 30.0
    v = np.random.default_rng(3).standard_normal((1, T, 1, d))
    p = np.zeros((1, T, 1, d))
    y, A, _, n = oracle.vla_forward_ratio(k, k, v, p)
    np.testing.assert_allclose(y, v, rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(A[0, 0], np.eye(d), atol=1e-15)
    # the denominator memory holds 1 along every written key and 0 elsewhere
    want = np.zeros(d)
    want[:T] = 1.0
    np.testing.assert_allclose(n[0, 0], want, atol=1e-10)


@pytest.mark.parametrize("T1", [1, 9, 16])
def test_chained_calls(T1):
    x = _inputs(21, T=31)
    y, A, S, n = oracle.vla_forward_ratio(x["q"], x["k"], x["v"], x["p"])
    a = {k_: v_[:, :T1] for k_, v_ in x.items()}
    b = {k_: v_[:, T1:] for k_, v_ in x.items()}
    y1, A1, S1, n1 = oracle.vla_forward_ratio(a["q"], a["k"], a["v"], a["p"])
    y2, A2, S2, n2 = oracle.vla_forward_ratio(b["q"], b["k"], b["v"], b["p"], A_in=A1, S_in=S1, n_in=n1)
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), y, rtol=1e-12, atol=1e-13)
    for got, ref in ((A2, A), (S2, S), (n2, n)):
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_first_token_denominator_is_alpha_hat():
    x = _inputs(31, T=1)
    _, _, _, n = oracle.vla_forward_ratio(x["q"], x["k"], x["v"], x["p"])
    _, _, _, diag = oracle.vla_forward(x["q"], x["k"], x["v"], x["p"], diagnostics=True)
    np.testing.assert_allclose(n, diag["ahat"][:, 0], rtol=1e-13, atol=1e-14)
