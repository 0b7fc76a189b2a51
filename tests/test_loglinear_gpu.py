"""GPU parity of the log-linear (Fenwick-tree) readout and its level-weight
MLP ("Technical summary: adaptive memory decay for log-linear attention",
"Problem definition" and "Methodology") against the fp64 oracle.

The readout computes in fp32 end to end from the stored inputs, so `out`
takes the forward's gates (fp32: e_rel <= 1e-4; bf16: the one rounding of
`out`, e_abs <= 2e-2 with an e_rel <= 1e-2 tripwire) and the fp32 level
memories e_rel <= 1e-4 for either storage dtype.  The MLP is fp32 with a
softplus from the fp32 exp and log1p: e_rel <= 1e-5.
"""
import numpy as np
import pytest

import oracle
from gated_linear_attention_chunked_amd import inputs as I
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

DELTA = ["deltanet", "gdn", "kda", "gdn2"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch

    import gated_linear_attention_chunked_amd as lam

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lam.library()


def _case(variant, dtype, B, T, H, dk, dv, seed, nL=None, t0=0, gate_mu=-1.0):
    w = I.Workload(f"ll_{variant}_{dtype}_B{B}_T{T}_H{H}_dk{dk}_dv{dv}_t0{t0}", variant, dtype, B, T, H, dk, dv,
                   seed=seed, gate_mu=gate_mu)
    x = I.make_inputs(w)
    nL = nL or oracle.loglinear_levels(t0 + T - 1)
    r = np.random.default_rng(seed + 1)
    lam = I.round_f32(r.uniform(0.2, 1.5, (B, T, H, nL))).astype(np.float64)
    return w, x, lam


def _gpu(w, x, lam, state_in=None, t0=0):
    import torch

    import gated_linear_attention_chunked_amd as lam_

    g = I.to_device(x, w.dtype, "cuda")
    f32 = lambda a: None if a is None else torch.from_numpy(a.astype(np.float32)).cuda()
    out, st = lam_.loglinear_forward(w.variant, g["q"], g["k"], g["v"], g["beta"], f32(lam), alpha=g.get("alpha"),
                                     erase_b=g.get("erase_b"), write_w=g.get("write_w"), state_in=f32(state_in),
                                     t0=t0)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), st.cpu().numpy().astype(np.float64)


def _oracle(w, x, lam, state_in=None, t0=0):
    return oracle.loglinear_forward(w.variant, x["q"], x["k"], x["v"], x["beta"], lam, alpha=x.get("alpha"),
                                    erase_b=x.get("erase_b"), write_w=x.get("write_w"), state_in=state_in, t0=t0)


def _check(w, got, ref, label):
    U.check(w, got, ref, label=label, exact_f32=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", DELTA)
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (96, 96), (128, 128), (128, 64), (32, 96)])
def test_loglinear_small(variant, dtype, dk, dv):
    """Every element; 83 tokens (8 levels, merges up to level 7, ragged
    16-token tiles)."""
    w, x, lam = _case(variant, dtype, 2, 83, 3, dk, dv, seed=5000 + dk + dv)
    _check(w, _gpu(w, x, lam), _oracle(w, x, lam), w.name)


@pytest.mark.parametrize("variant", DELTA)
@pytest.mark.parametrize("t0", [1, 37, 64, 1000])
def test_loglinear_offset_and_levels_in(variant, t0):
    """Starting mid-sequence (absolute positions t0 ..) from given level
    memories, with more levels than needed."""
    w, x, lam = _case(variant, "bf16", 1, 50, 2, 64, 64, seed=5100 + t0, t0=t0,
                      nL=oracle.loglinear_levels(t0 + 49) + 2)
    nL = lam.shape[3]
    s0 = (np.random.default_rng(t0).standard_normal((1, 2, nL, 64, 64)) * 0.1).astype(np.float32).astype(np.float64)
    _check(w, _gpu(w, x, lam, state_in=s0, t0=t0), _oracle(w, x, lam, state_in=s0, t0=t0), w.name)


@pytest.mark.parametrize("variant", DELTA)
def test_loglinear_unit_weights_is_the_plain_scan(variant):
    """lambda = 1: the kernel reproduces the plain scan's output and its
    levels sum to the plain scan's memory (both computed on the GPU)."""
    import torch

    import gated_linear_attention_chunked_amd as lam_

    w, x, lam = _case(variant, "f32", 2, 100, 2, 128, 128, seed=5200)
    lam[:] = 1.0
    out, lv = _gpu(w, x, lam)
    g = I.to_device(x, "f32", "cuda")
    ref, st = lam_.forward(variant, g["q"], g["k"], g["v"], g["beta"], alpha=g.get("alpha"),
                           erase_b=g.get("erase_b"), write_w=g.get("write_w"), algo="recurrent")
    torch.cuda.synchronize()
    ref, st = ref.cpu().numpy(), st.cpu().numpy()
    assert U.errs(out, ref)[1] <= 1e-5
    assert U.errs(lv.sum(axis=2), st)[1] <= 1e-5


@pytest.mark.parametrize("variant", DELTA)
def test_loglinear_decode_steps_match_one_call(variant):
    """Streaming decode: T = 1 calls at t0 = 0, 1, 2, ... with the levels
    updated in place give the one-call result (O(log T) state)."""
    import torch

    import gated_linear_attention_chunked_amd as lam_

    w, x, lam = _case(variant, "bf16", 2, 40, 2, 64, 64, seed=5300, nL=oracle.loglinear_levels(39))
    full_out, full_st = _gpu(w, x, lam)
    g = I.to_device(x, "bf16", "cuda")
    lg = torch.from_numpy(lam.astype(np.float32)).cuda()
    st = torch.zeros((2, 2, lam.shape[3], 64, 64), device="cuda")
    outs = []
    for t in range(40):
        sl = lambda a: None if a is None else a[:, t:t + 1].contiguous()
        o, _ = lam_.loglinear_forward(variant, sl(g["q"]), sl(g["k"]), sl(g["v"]), sl(g["beta"]), sl(lg),
                                      alpha=sl(g.get("alpha")), erase_b=sl(g.get("erase_b")),
                                      write_w=sl(g.get("write_w")), state_in=st, state_out=st, t0=t)
        outs.append(o)
    torch.cuda.synchronize()
    step_out = torch.cat(outs, 1).float().cpu().numpy()
    # the same fp32 arithmetic in the same order, token by token
    np.testing.assert_array_equal(step_out, full_out)
    np.testing.assert_array_equal(st.cpu().numpy(), full_st)


@pytest.mark.parametrize("name", ["gdn_bf16_B8_T4096_H8_d128"])
def test_loglinear_full_size_sampled(name):
    """B8 T4096 H8 d128 (13 levels), full grid; two (b, h) chains checked
    against the oracle."""
    w, x, lam = _case("gdn", "bf16", 8, 4096, 8, 128, 128, seed=5400, gate_mu=2.0)
    out, lv = _gpu(w, x, lam)
    for b, h in [(0, 0), (6, 5)]:
        sl = lambda a: None if a is None else a[b:b + 1, :, h:h + 1]
        xs = {k: sl(v) for k, v in x.items()}
        ref = _oracle(w.replace(B=1, H=1), xs, sl(lam))
        _check(w, (out[b:b + 1, :, h:h + 1], lv[b:b + 1, h:h + 1]), ref, f"{name} chain ({b},{h})")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_loglinear_lambda_mlp(dtype):
    """Every row of the level-weight MLP (13 levels, hidden 26), and the
    page's initialisation (W2 = 0, b = 0.54) gives softplus(0.54) everywhere."""
    import torch

    import gated_linear_attention_chunked_amd as lam_

    r = np.random.default_rng(7)
    nL, nh = 13, 26
    d = I.round_f32(r.standard_normal((3, 333, 2, nL))).astype(np.float64)
    if dtype == "bf16":
        d = I.round_bf16(d.astype(np.float32)).astype(np.float64)
    W1, W2 = I.round_f32(r.standard_normal((nL, nh)) * 0.3), I.round_f32(r.standard_normal((nh, nL)) * 0.3)
    b = I.round_f32(r.standard_normal(nL))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda a: torch.from_numpy(np.asarray(a, np.float32)).cuda()
    got = lam_.loglinear_lambda(dev(d).to(tdt), dev(W1), dev(W2), dev(b))
    torch.cuda.synchronize()
    ref = oracle.loglinear_lambda(d, W1.astype(np.float64), W2.astype(np.float64), b.astype(np.float64))
    assert U.errs(got.cpu().numpy(), ref)[1] <= 1e-5
    init = lam_.loglinear_lambda(dev(d).to(tdt), dev(W1), dev(np.zeros((nh, nL))), dev(np.full(nL, 0.54)))
    torch.cuda.synchronize()
    np.testing.assert_allclose(init.cpu().numpy(), np.log1p(np.exp(0.54)), rtol=1e-6)
