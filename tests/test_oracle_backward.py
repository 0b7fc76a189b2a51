"""Pins of the oracle's backward pass (the adjoint of the delta-rule scan).

The pages give only the forward rule ("Mechanisms, trade-offs and
cross-layer routing of linear-attention architectures", "Technical
details"), so the adjoint is pinned to something independent of its own
derivation: central finite differences of the forward oracle, element by
element, on tiny inputs in fp64, for every gradient of every variant; plus
structural cases (beta = 0 writes nothing, so no gradient reaches v; Gated
DeltaNet at alpha = 1 is DeltaNet).
"""
import numpy as np
import pytest

import oracle

VARIANTS = ["deltanet", "gdn", "kda", "gdn2"]


def _inputs(seed, variant, B=1, T=5, H=2, dk=3, dv=2):
    r = np.random.default_rng(seed)
    x = {
        "q": r.standard_normal((B, T, H, dk)),
        "k": r.standard_normal((B, T, H, dk)) * 0.6,
        "v": r.standard_normal((B, T, H, dv)),
        "beta": r.uniform(0.1, 0.9, (B, T, H)),
        "state_in": r.standard_normal((B, H, dv, dk)) * 0.5,
    }
    if variant == "kda":
        x["alpha"] = r.uniform(0.3, 1.0, (B, T, H, dk))
    elif variant != "deltanet":
        x["alpha"] = r.uniform(0.3, 1.0, (B, T, H))
    if variant == "gdn2":
        x["erase_b"] = r.uniform(0.1, 1.0, (B, T, H, dk))
        x["write_w"] = r.uniform(0.1, 1.0, (B, T, H, dv))
    seeds = np.random.default_rng(seed + 1)
    dout = seeds.standard_normal((B, T, H, dv))
    dstate = seeds.standard_normal((B, H, dv, dk))
    return x, dout, dstate


def _loss(variant, x, dout, dstate):
    out, st = oracle.delta_forward(variant, x["q"], x["k"], x["v"], x["beta"], alpha=x.get("alpha"),
                                   erase_b=x.get("erase_b"), write_w=x.get("write_w"),
                                   state_in=x["state_in"])
    return float(np.sum(out * dout) + np.sum(st * dstate))


def _grads(variant, x, dout, dstate):
    return oracle.delta_backward(variant, x["q"], x["k"], x["v"], x["beta"], dout, alpha=x.get("alpha"),
                                 erase_b=x.get("erase_b"), write_w=x.get("write_w"),
                                 state_in=x["state_in"], dstate_out=dstate)


NAMES = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "alpha": "dalpha", "erase_b": "derase_b",
         "write_w": "dwrite_w", "state_in": "dstate_in"}


@pytest.mark.parametrize("variant", VARIANTS)
def test_adjoint_matches_central_differences(variant):
    """Every gradient element against (L(x + h) - L(x - h)) / 2h, h = 1e-6:
    a dropped term, a wrong sign or a transposed operand in the adjoint
    changes some element by far more than the differencing error (~1e-9)."""
    x, dout, dstate = _inputs(11 + VARIANTS.index(variant), variant)
    g = _grads(variant, x, dout, dstate)
    h = 1e-6
    for name, arr in x.items():
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = _loss(variant, x, dout, dstate)
            arr[idx] = keep - h
            lm = _loss(variant, x, dout, dstate)
            arr[idx] = keep
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[NAMES[name]], num, rtol=1e-6, atol=1e-8, err_msg=f"{variant} {name}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_zero_beta_sends_no_gradient_to_the_values(variant):
    """beta = 0: nothing is written, so v (and w) cannot affect the loss."""
    x, dout, dstate = _inputs(31, variant)
    x["beta"][:] = 0.0
    g = _grads(variant, x, dout, dstate)
    assert np.all(g["dv"] == 0.0)
    if variant == "gdn2":
        assert np.all(g["dwrite_w"] == 0.0)


def test_gated_deltanet_at_unit_decay_is_deltanet():
    x, dout, dstate = _inputs(41, "gdn")
    x["alpha"][:] = 1.0
    g1 = _grads("gdn", x, dout, dstate)
    g0 = _grads("deltanet", {k_: v_ for k_, v_ in x.items() if k_ != "alpha"}, dout, dstate)
    for n in ("dq", "dk", "dv", "dbeta", "dstate_in"):
        np.testing.assert_allclose(g1[n], g0[n], rtol=1e-13, atol=1e-14, err_msg=n)


def test_read_only_gradient_closed_form():
    """One token from a zero memory: y = beta (k . q) v, so dq = beta (v . dout) k,
    dv = beta (k . q) dout and dbeta = (k . q)(v . dout)."""
    r = np.random.default_rng(5)
    q, k = r.standard_normal((1, 1, 1, 4)), r.standard_normal((1, 1, 1, 4))
    v, dout = r.standard_normal((1, 1, 1, 3)), r.standard_normal((1, 1, 1, 3))
    beta = np.full((1, 1, 1), 0.7)
    g = oracle.delta_backward("deltanet", q, k, v, beta, dout)
    kq, vd = float(np.sum(k * q)), float(np.sum(v * dout))
    np.testing.assert_allclose(g["dq"], 0.7 * vd * k, rtol=1e-14)
    np.testing.assert_allclose(g["dv"], 0.7 * kq * dout, rtol=1e-14)
    np.testing.assert_allclose(g["dbeta"], np.full((1, 1, 1), kq * vd), rtol=1e-14)


@pytest.mark.parametrize("variant", ["deltanet", "gdn", "gdn2"])
@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunked_adjoint_equals_token_adjoint(variant, C):
    """The chunked adjoint (residual form, test-only numpy model) equals the
    oracle's token-by-token adjoint to ~1e-10 relative per gradient, at a
    ragged length spanning several chunks, with W0 and dW_T given."""
    from tests import chunked_model

    r = np.random.default_rng(17)
    B, T, H, dk, dv = 1, 83, 2, 8, 6
    x, dout, dstate = _inputs(19, variant, B=B, T=T, H=H, dk=dk, dv=dv)
    # a slower decay, so chunks carry real state
    if "alpha" in x:
        x["alpha"] = r.uniform(0.85, 1.0, x["alpha"].shape)
    ref = _grads(variant, x, dout, dstate)
    got = chunked_model.delta_chunked_backward(variant, x["q"], x["k"], x["v"], x["beta"], dout,
                                               alpha=x.get("alpha"), erase_b=x.get("erase_b"),
                                               write_w=x.get("write_w"), state_in=x["state_in"],
                                               dstate_out=dstate, C=C)
    for n, g in ref.items():
        scale = max(np.max(np.abs(g)), 1e-30)
        assert np.max(np.abs(got[n] - g)) <= 1e-10 * scale, (n, np.max(np.abs(got[n] - g)) / scale)


@pytest.mark.parametrize("variant", ["deltanet", "gdn", "gdn2"])
@pytest.mark.parametrize("C", [1, 16])
def test_record_form_adjoint_scan(variant, C):
    """The reverse scan in the record form the adjoint kernel runs (Ahat' =
    Tc^T Ahat, (Aq Tc)^T, the decayed query and erase-key operands) gives the
    oracle's dW0 and, through dX, its dv (and dw for Gated DeltaNet-2)."""
    from tests import chunked_model

    r = np.random.default_rng(23)
    x, dout, dstate = _inputs(29, variant, B=1, T=45, H=2, dk=8, dv=6)
    if "alpha" in x:
        x["alpha"] = r.uniform(0.6, 1.0, x["alpha"].shape)
    ref = _grads(variant, x, dout, dstate)
    dX, dS = chunked_model.delta_record_adjoint(variant, x["q"], x["k"], x["v"], x["beta"], dout,
                                                alpha=x.get("alpha"), erase_b=x.get("erase_b"),
                                                write_w=x.get("write_w"), state_in=x["state_in"],
                                                dstate_out=dstate, C=C)
    tol = lambda g: 1e-10 * max(np.max(np.abs(g)), 1e-30)
    assert np.max(np.abs(dS - ref["dstate_in"])) <= tol(ref["dstate_in"])
    if variant == "gdn2":
        assert np.max(np.abs(x["write_w"] * dX - ref["dv"])) <= tol(ref["dv"])
        assert np.max(np.abs(x["v"] * dX - ref["dwrite_w"])) <= tol(ref["dwrite_w"])
    else:
        assert np.max(np.abs(dX - ref["dv"])) <= tol(ref["dv"])


@pytest.mark.parametrize("variant", ["gdn", "gdn2"])
@pytest.mark.parametrize("C", [4, 16])
def test_direct_decay_gradient_form(variant, C):
    """d alpha summed without the cancelling terms (the form the chunked
    gradient kernel uses) equals the oracle's, also under strong decays."""
    from tests import chunked_model

    for lo, hi in ((0.85, 1.0), (0.001, 0.01)):
        r = np.random.default_rng(31)
        x, dout, dstate = _inputs(37, variant, B=1, T=40, H=2, dk=8, dv=6)
        x["alpha"] = r.uniform(lo, hi, x["alpha"].shape)
        ref = _grads(variant, x, dout, dstate)
        got = chunked_model.delta_chunked_backward(variant, x["q"], x["k"], x["v"], x["beta"], dout,
                                                   alpha=x["alpha"], erase_b=x.get("erase_b"),
                                                   write_w=x.get("write_w"), state_in=x["state_in"],
                                                   dstate_out=dstate, C=C, dlog_direct=True)
        g = ref["dalpha"]
        assert np.max(np.abs(got["dalpha"] - g)) <= 1e-9 * np.max(np.abs(g)), (lo, hi)
