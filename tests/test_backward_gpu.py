"""GPU parity of the token-recurrent backward pass (lam_backward through the
C ABI with algo "recurrent", the only form for Kimi Delta) against the
oracle's fp64 adjoint on the same seeded inputs and cotangents.  The chunked
backward, the default for the other three variants, has its own tests in
test_backward_chunked_gpu.py.

The kernel computes in fp32 from the stored inputs (bf16 storage included),
recomputing the forward states from fp32 checkpoints, so every gradient is
held to e_rel = max|g - g_ref| / max|g_ref| <= 1e-4 per tensor, the bar of
the fp32 forward scan: the adjoint takes the same kind of fp32 sums (length
dk or dv per row, dv rows per cross-row sum) over the same number of tokens.
"""
import numpy as np
import pytest

import oracle
from gated_linear_attention_chunked_amd import inputs as I
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

DELTA = ["deltanet", "gdn", "kda", "gdn2"]
GRAD_REL = 1e-4
NAMES = ["dq", "dk", "dv", "dbeta", "dstate_in", "dalpha", "derase_b", "dwrite_w"]


def _w(variant, dtype, B, T, H, dk, dv, seed, gate_mu=-1.0):
    return I.Workload(f"bwd_{variant}_{dtype}_B{B}_T{T}_H{H}_dk{dk}_dv{dv}", variant, dtype, B, T, H,
                      dk, dv, seed=seed, gate_mu=gate_mu)


def _gpu(w, x, dout, dstate, state_in, with_dstate_in=True, algo="recurrent"):
    import torch

    import gated_linear_attention_chunked_amd as lam

    g = I.to_device(x, w.dtype, "cuda")
    dy = I.to_device({"d": dout}, w.dtype, "cuda")["d"]
    f32 = lambda a: None if a is None else torch.from_numpy(a.astype(np.float32)).cuda()
    r = lam.backward(w.variant, g["q"], g["k"], g["v"], g["beta"], dy, alpha=g.get("alpha"),
                     erase_b=g.get("erase_b"), write_w=g.get("write_w"), state_in=f32(state_in),
                     dstate_out=f32(dstate), with_dstate_in=with_dstate_in, algo=algo)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy().astype(np.float64)) for k, v in r.items()}


def _oracle(w, x, dout, dstate, state_in):
    return oracle.delta_backward(w.variant, x["q"], x["k"], x["v"], x["beta"], dout, alpha=x.get("alpha"),
                                 erase_b=x.get("erase_b"), write_w=x.get("write_w"), state_in=state_in,
                                 dstate_out=dstate)


def _check(got, ref, label):
    rep = {}
    for n in NAMES:
        if n not in ref or got.get(n) is None:
            continue
        assert got[n].shape == ref[n].shape, f"{label} {n} shape"
        e_abs, e_rel = U.errs(got[n], ref[n])
        rep[n] = e_rel
        assert np.all(np.isfinite(got[n])), f"{label} {n} non-finite"
        assert e_rel <= GRAD_REL, f"{label} {n} e_rel={e_rel:.3e} (e_abs={e_abs:.3e})"
    return rep


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


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch

    import gated_linear_attention_chunked_amd as lam

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lam.library()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", DELTA)
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (96, 96), (128, 128), (128, 64), (64, 128), (32, 96)])
def test_backward_small(variant, dtype, dk, dv):
    """Every element of every gradient; 83 tokens = five 16-token checkpoint
    chunks and a ragged tail; initial state and final-state adjoint given."""
    w = _w(variant, dtype, 2, 83, 3, dk, dv, seed=3000 + dk + dv)
    x, dout, dstate, s0 = _case(w)
    _check(_gpu(w, x, dout, dstate, s0), _oracle(w, x, dout, dstate, s0), w.name)


@pytest.mark.parametrize("variant", DELTA)
@pytest.mark.parametrize("T", [1, 8, 9, 15, 16, 17, 32, 33])
def test_backward_lengths(variant, T):
    """Chunk and flush boundaries (16-token checkpoints, sums flushed every 8)."""
    w = _w(variant, "bf16", 1, T, 2, 128, 128, seed=3100 + T)
    x, dout, dstate, s0 = _case(w)
    _check(_gpu(w, x, dout, dstate, s0), _oracle(w, x, dout, dstate, s0), w.name)


@pytest.mark.parametrize("variant", DELTA)
def test_backward_without_state(variant):
    """No initial state, no final-state adjoint, dstate_in not requested."""
    w = _w(variant, "f32", 2, 40, 2, 64, 64, seed=3200)
    x, dout, _, _ = _case(w, with_state=False)
    got = _gpu(w, x, dout, None, None, with_dstate_in=False)
    assert got["dstate_in"] is None
    _check(got, _oracle(w, x, dout, None, None), w.name)


@pytest.mark.parametrize("variant", DELTA)
def test_backward_weak_decay_long(variant):
    """alpha ~ 0.98 over 600 tokens: adjoints travel back hundreds of tokens,
    through dozens of checkpoints."""
    w = _w(variant, "bf16", 1, 600, 2, 64, 64, seed=3300, gate_mu=-4.0)
    x, dout, dstate, s0 = _case(w)
    _check(_gpu(w, x, dout, dstate, s0), _oracle(w, x, dout, dstate, s0), w.name)


def test_backward_empty_sequence_passes_the_state_adjoint():
    """T = 0: state_out = state_in, so dstate_in = dstate_out."""
    import torch

    import gated_linear_attention_chunked_amd as lam

    dst = torch.randn(2, 3, 64, 64, device="cuda")
    e = lambda *s: torch.empty(*s, device="cuda", dtype=torch.bfloat16)
    r = lam.backward("gdn", e(2, 0, 3, 64), e(2, 0, 3, 64), e(2, 0, 3, 64), e(2, 0, 3), e(2, 0, 3, 64),
                     alpha=e(2, 0, 3), dstate_out=dst, algo="recurrent")
    torch.cuda.synchronize()
    assert torch.equal(r["dstate_in"], dst)
    r = lam.backward("gdn", e(2, 0, 3, 64), e(2, 0, 3, 64), e(2, 0, 3, 64), e(2, 0, 3), e(2, 0, 3, 64),
                     alpha=e(2, 0, 3), algo="recurrent")
    torch.cuda.synchronize()
    assert torch.count_nonzero(r["dstate_in"]).item() == 0


def test_backward_row_local_gradients_are_reproducible():
    """dv, dwrite_w and dstate_in are written by one lane each: bitwise equal
    across runs; the atomically summed ones agree to the parity bar."""
    w = _w("gdn2", "bf16", 2, 70, 4, 128, 128, seed=3400)
    x, dout, dstate, s0 = _case(w)
    a, b = _gpu(w, x, dout, dstate, s0), _gpu(w, x, dout, dstate, s0)
    for n in ("dv", "dwrite_w", "dstate_in"):
        assert np.array_equal(a[n], b[n]), n
    for n in ("dq", "dk", "dbeta", "dalpha", "derase_b"):
        assert U.errs(a[n], b[n])[1] <= GRAD_REL, n


@pytest.mark.parametrize("name", ["gdn_bf16_B8_T4096_H8_d128", "gdn2_bf16_B8_T4096_H8_d128"])
def test_backward_full_size_sampled(name):
    """The forward's throughput shape, full grid; three (b, h) chains checked
    against the oracle one by one (the gradients of a chain depend on that
    chain alone)."""
    w = I.WORKLOADS[name]
    x = I.make_inputs(w)
    dout, dstate = I.make_cotangents(w, 11)
    got = _gpu(w, x, dout, dstate, None)
    for b, h in [(0, 0), (3, 5), (7, 7)]:
        sl = lambda a: None if a is None else a[b:b + 1, :, h:h + 1]
        xs = {k: sl(v) for k, v in x.items()}
        ds = dstate[b:b + 1, h:h + 1]
        ref = oracle.delta_backward(w.variant, xs["q"], xs["k"], xs["v"], xs["beta"], sl(dout),
                                    alpha=xs.get("alpha"), erase_b=xs.get("erase_b"),
                                    write_w=xs.get("write_w"), dstate_out=ds)
        mine = {}
        for n, v in got.items():
            if v is None:
                continue
            mine[n] = v[b:b + 1, h:h + 1] if n == "dstate_in" else v[b:b + 1, :, h:h + 1]
        _check(mine, ref, f"{name} chain ({b},{h})")
