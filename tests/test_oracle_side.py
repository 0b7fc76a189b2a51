"""Pins of the oracle's cross-layer routing outputs ("Mechanisms, trade-offs
and cross-layer routing of linear-attention architectures", "Methodology"
and "Technical details": CLER routes the delta-rule residual r, CLVR the
write value, through a zero-initialised projection P added to the residual
stream).

The residual is pinned to the state trajectory, which the forward pins fix
independently: the write of token t is W_t - W~_t = beta_t r_t k_t^T, so r_t
= (W_t - W~_t) k_t / (beta_t |k_t|^2), with W~_t the decayed W_{t-1} formed
here from the stored states.  The routing product is pinned by P = 0, by an
identity projection and by a brute-force loop.
"""
import numpy as np
import pytest

import oracle

VARIANTS = ["deltanet", "gdn", "kda", "gdn2"]


def _inputs(seed, variant, B=2, T=9, H=2, dk=5, dv=4):
    r = np.random.default_rng(seed)
    x = {"q": r.standard_normal((B, T, H, dk)), "k": r.standard_normal((B, T, H, dk)) * 0.7,
         "v": r.standard_normal((B, T, H, dv)), "beta": r.uniform(0.2, 0.9, (B, T, H)),
         "state_in": r.standard_normal((B, H, dv, dk)) * 0.5}
    if variant == "kda":
        x["alpha"] = r.uniform(0.4, 1.0, (B, T, H, dk))
    elif variant != "deltanet":
        x["alpha"] = r.uniform(0.4, 1.0, (B, T, H))
    if variant == "gdn2":
        x["erase_b"] = r.uniform(0.1, 1.0, (B, T, H, dk))
        x["write_w"] = r.uniform(0.1, 1.0, (B, T, H, dv))
    return x


def _fwd(variant, x, **kw):
    return oracle.delta_forward(variant, x["q"], x["k"], x["v"], x["beta"], alpha=x.get("alpha"),
                                erase_b=x.get("erase_b"), write_w=x.get("write_w"),
                                state_in=x.get("state_in"), **kw)


def _states(variant, x):
    """W_0 .. W_T of every chain, one oracle call per prefix length."""
    B, T, H, _ = x["q"].shape
    sts = [x["state_in"]]
    for t in range(1, T + 1):
        xs = {k_: (v_ if k_ == "state_in" else v_[:, :t]) for k_, v_ in x.items()}
        sts.append(_fwd(variant, xs)[1])
    return sts


def _decay(variant, x, W, t):
    if variant in ("gdn", "gdn2"):
        return W * x["alpha"][:, t][:, :, None, None]
    if variant == "kda":
        return W * x["alpha"][:, t][:, :, None, :]
    return W


@pytest.mark.parametrize("variant", VARIANTS)
def test_residual_is_the_written_update(variant):
    x = _inputs(21 + VARIANTS.index(variant), variant)
    _, _, r = _fwd(variant, x, side="residual")
    sts = _states(variant, x)
    for t in range(x["q"].shape[1]):
        dW = sts[t + 1] - _decay(variant, x, sts[t], t)          # [B,H,dv,dk]
        kt = x["k"][:, t]                                          # [B,H,dk]
        want = np.einsum("bhij,bhj->bhi", dW, kt) / (x["beta"][:, t] * np.sum(kt * kt, -1))[..., None]
        np.testing.assert_allclose(r[:, t], want, rtol=1e-9, atol=1e-11, err_msg=f"{variant} t={t}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_residual_with_nothing_written_is_target_minus_decayed_prediction(variant):
    """beta = 0: the memory only decays, so r_t = z_t - (decay_1..t W_0) e_t,
    formed here from the inputs alone."""
    x = _inputs(31, variant)
    x["beta"][:] = 0.0
    _, _, r = _fwd(variant, x, side="residual")
    W = x["state_in"].copy()
    for t in range(x["q"].shape[1]):
        W = _decay(variant, x, W, t)
        e = x["k"][:, t] * (x["erase_b"][:, t] if variant == "gdn2" else 1.0)
        z = x["v"][:, t] * (x["write_w"][:, t] if variant == "gdn2" else 1.0)
        np.testing.assert_allclose(r[:, t], z - np.einsum("bhij,bhj->bhi", W, e), rtol=1e-12, atol=1e-13)


def test_residual_of_a_rewrite_along_one_key():
    """DeltaNet from a zero memory, unit key, beta = 1: token 0 writes v0
    (r = v0); token 1 on the same key finds v0 there, so r = v1 - v0."""
    k = np.zeros((1, 2, 1, 4))
    k[..., 1] = 1.0
    v = np.array([[[[1.0, 2.0, 3.0]], [[0.5, -1.0, 4.0]]]])
    _, _, r = oracle.delta_forward("deltanet", np.ones((1, 2, 1, 4)), k, v, np.ones((1, 2, 1)),
                                   side="residual")
    np.testing.assert_array_equal(r[0, 0, 0], [1.0, 2.0, 3.0])
    np.testing.assert_array_equal(r[0, 1, 0], [-0.5, -3.0, 1.0])


@pytest.mark.parametrize("variant", VARIANTS)
def test_value_side_output_is_the_write_target(variant):
    x = _inputs(41, variant)
    out0, st0 = _fwd(variant, x)
    out, st, z = _fwd(variant, x, side="value")
    want = x["v"] * (x["write_w"] if variant == "gdn2" else 1.0)
    np.testing.assert_array_equal(z, want)
    # the side output changes nothing else
    np.testing.assert_array_equal(out, out0)
    np.testing.assert_array_equal(st, st0)


def test_route_zero_projection_leaves_the_stream():
    r = np.random.default_rng(3)
    h, s = r.standard_normal((2, 5, 6)), r.standard_normal((2, 5, 2, 3))
    np.testing.assert_array_equal(oracle.route(h, s, np.zeros((6, 6))), h)


def test_route_identity_projection_adds_the_signal():
    r = np.random.default_rng(4)
    h, s = r.standard_normal((2, 5, 6)), r.standard_normal((2, 5, 2, 3))
    np.testing.assert_allclose(oracle.route(h, s, np.eye(6)), h + s.reshape(2, 5, 6), rtol=0, atol=0)


def test_route_brute_force():
    r = np.random.default_rng(5)
    B, T, H, dv, D = 2, 3, 2, 3, 4
    h, s, P = r.standard_normal((B, T, D)), r.standard_normal((B, T, H, dv)), r.standard_normal((D, H * dv))
    want = h.copy()
    for b in range(B):
        for t in range(T):
            for d in range(D):
                for hh in range(H):
                    for i in range(dv):
                        want[b, t, d] += P[d, hh * dv + i] * s[b, t, hh, i]
    np.testing.assert_allclose(oracle.route(h, s, P), want, rtol=1e-13, atol=1e-13)
