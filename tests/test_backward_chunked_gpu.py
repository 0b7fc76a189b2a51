"""GPU parity of the chunked backward (lam_backward with algo "chunked")
against the oracle's fp64 adjoint.

The chunked form evaluates the same adjoint in 16-token chunks on fp32
matrix cores: the forward is recomputed keeping each chunk's start state and
residuals, the state cotangent is carried back chunk by chunk, and each
chunk's gradients are formed in parallel.  Every gradient is held to the
backward's fp32 bar, e_rel = max|g - g_ref| / max|g_ref| <= 1e-4 per tensor.
"""
import numpy as np
import pytest

import oracle
from gated_linear_attention_chunked_amd import inputs as I
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

VARIANTS = ["deltanet", "gdn", "gdn2"]
GRAD_REL = 1e-4
NAMES = ["dq", "dk", "dv", "dbeta", "dstate_in", "dalpha", "derase_b", "dwrite_w"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch

    import gated_linear_attention_chunked_amd as lam

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lam.library()


def _w(variant, dtype, B, T, H, dk, dv, seed, gate_mu=-1.0):
    return I.Workload(f"bwdc_{variant}_{dtype}_B{B}_T{T}_H{H}_dk{dk}_dv{dv}", variant, dtype, B, T, H,
                      dk, dv, seed=seed, gate_mu=gate_mu)


def _run(w, x, dout, dstate, s0, algo="chunked", with_dstate_in=True):
    import torch

    import gated_linear_attention_chunked_amd as lam

    g = I.to_device(x, w.dtype, "cuda")
    dy = I.to_device({"d": dout}, w.dtype, "cuda")["d"]
    f32 = lambda a: None if a is None else torch.from_numpy(a.astype(np.float32)).cuda()
    r = lam.backward(w.variant, g["q"], g["k"], g["v"], g["beta"], dy, alpha=g.get("alpha"),
                     erase_b=g.get("erase_b"), write_w=g.get("write_w"), state_in=f32(s0),
                     dstate_out=f32(dstate), algo=algo, with_dstate_in=with_dstate_in)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy().astype(np.float64)) for k, v in r.items()}


def _ref(w, x, dout, dstate, s0):
    return oracle.delta_backward(w.variant, x["q"], x["k"], x["v"], x["beta"], dout, alpha=x.get("alpha"),
                                 erase_b=x.get("erase_b"), write_w=x.get("write_w"), state_in=s0,
                                 dstate_out=dstate)


def _check(got, ref, label):
    for n in NAMES:
        if n not in ref or got.get(n) is None:
            continue
        assert got[n].shape == ref[n].shape, f"{label} {n} shape"
        assert np.all(np.isfinite(got[n])), f"{label} {n} non-finite"
        e_abs, e_rel = U.errs(got[n], ref[n])
        assert e_rel <= GRAD_REL, f"{label} {n} e_rel={e_rel:.3e} (e_abs={e_abs:.3e})"


def _case(w, seed=7, with_state=True):
    x = I.make_inputs(w)
    dout, dstate = I.make_cotangents(w, seed)
    s0 = None
    if with_state:
        s0 = np.random.default_rng(seed + 1).standard_normal((w.B, w.H, w.dv, w.dk)) * 0.2
        s0 = s0.astype(np.float32).astype(np.float64)
    else:
        dstate = None
    return x, dout, dstate, s0


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (96, 96), (128, 128), (128, 32), (32, 128), (96, 64)])
def test_every_gradient(variant, dtype, dk, dv):
    """Every element of every gradient: a ragged length over several chunks,
    an initial state and a final-state cotangent."""
    w = _w(variant, dtype, 2, 83, 2, dk, dv, seed=9900 + dk + 3 * dv)
    x, dout, dstate, s0 = _case(w)
    _check(_run(w, x, dout, dstate, s0), _ref(w, x, dout, dstate, s0), w.name)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("T", [1, 15, 16, 17, 32, 200])
def test_lengths(variant, T):
    """One token, a chunk less or more by one, whole chunks."""
    w = _w(variant, "bf16", 1, T, 3, 64, 64, seed=9910 + T)
    x, dout, dstate, s0 = _case(w)
    _check(_run(w, x, dout, dstate, s0), _ref(w, x, dout, dstate, s0), w.name)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("with_dstate_in", [True, False])
def test_without_state(variant, with_dstate_in):
    """No initial state and no final-state cotangent (both taken as zero);
    the initial state's cotangent asked for or not."""
    w = _w(variant, "f32", 2, 70, 2, 128, 128, seed=9920)
    x, dout, dstate, s0 = _case(w, with_state=False)
    got = _run(w, x, dout, dstate, s0, with_dstate_in=with_dstate_in)
    assert (got["dstate_in"] is None) == (not with_dstate_in)
    _check(got, _ref(w, x, dout, dstate, s0), w.name)


@pytest.mark.parametrize("variant,gate_mu", [("gdn", -4.0), ("gdn2", -4.0), ("deltanet", 0.0), ("gdn", 6.0)])
def test_long(variant, gate_mu):
    """600 tokens (38 chunks): weak decays carry the state cotangent across
    many chunks; strong ones drive the in-chunk decays far below one."""
    w = _w(variant, "f32", 1, 600, 2, 128, 64, seed=9930, gate_mu=gate_mu)
    x, dout, dstate, s0 = _case(w)
    _check(_run(w, x, dout, dstate, s0), _ref(w, x, dout, dstate, s0), f"{w.name} mu={gate_mu}")


@pytest.mark.parametrize("variant", ["gdn", "gdn2"])
def test_zero_and_unit_decays(variant):
    """alpha = 1 runs and a chunk with beta = 0 (writes nothing); alpha is kept
    away from zero, where its gradient divides by alpha."""
    w = _w(variant, "f32", 1, 150, 2, 64, 64, seed=9940)
    x, dout, dstate, s0 = _case(w)
    x["alpha"][:, 70:90] = 1.0
    x["alpha"][:, 10:13] = 1e-3
    x["beta"][:, 96:112] = 0.0
    _check(_run(w, x, dout, dstate, s0), _ref(w, x, dout, dstate, s0), "zero/unit " + variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_bitwise_reproducible(variant):
    """No atomics: two calls give the same bits."""
    w = _w(variant, "bf16", 2, 130, 4, 128, 128, seed=9950)
    x, dout, dstate, s0 = _case(w)
    r1 = _run(w, x, dout, dstate, s0)
    r2 = _run(w, x, dout, dstate, s0)
    for n in r1:
        if r1[n] is not None:
            np.testing.assert_array_equal(r1[n], r2[n], err_msg=n)


def test_full_grid_every_gradient():
    """B8 H8: 64 heads (the scans' XCD-grouped block map), every element."""
    w = _w("gdn", "bf16", 8, 50, 8, 128, 128, seed=9960)
    x, dout, dstate, s0 = _case(w)
    _check(_run(w, x, dout, dstate, s0), _ref(w, x, dout, dstate, s0), w.name)


@pytest.mark.parametrize("name", ["gdn_bf16_B8_T4096_H8_d128", "gdn2_bf16_B8_T4096_H8_d128"])
def test_full_size_sampled(name):
    """The forward's throughput shape (the backward bench line's launch),
    full grid; three (b, h) chains checked against the oracle one by one (the
    gradients of a chain depend on that chain alone)."""
    w = I.WORKLOADS[name]
    x = I.make_inputs(w)
    dout, dstate = I.make_cotangents(w, 11)
    got = _run(w, x, dout, dstate, None)
    for b, h in [(0, 0), (3, 5), (7, 7)]:
        sl = lambda a: None if a is None else a[b:b + 1, :, h:h + 1]
        xs = {k: sl(v) for k, v in x.items()}
        ref = _ref(w, xs, sl(dout), dstate[b:b + 1, h:h + 1], None)
        mine = {}
        for n, v in got.items():
            if v is not None:
                mine[n] = v[b:b + 1, h:h + 1] if n == "dstate_in" else v[b:b + 1, :, h:h + 1]
        _check(mine, ref, f"{name} chain ({b},{h})")


def test_kda_chunked_is_unsupported():
    import gated_linear_attention_chunked_amd as lam

    w = _w("kda", "bf16", 1, 20, 1, 64, 64, seed=1)
    x, dout, dstate, s0 = _case(w)
    with pytest.raises(lam.LamError) as e:
        _run(w, x, dout, dstate, s0)
    assert e.value.status == 2


def test_empty_sequence_passes_the_state_cotangent():
    w = _w("gdn", "f32", 2, 0, 2, 64, 64, seed=9970)
    x, dout, dstate, s0 = _case(w)
    got = _run(w, x, dout, dstate, s0, algo="auto")
    np.testing.assert_array_equal(got["dstate_in"], dstate.astype(np.float32).astype(np.float64))
