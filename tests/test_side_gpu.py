"""GPU parity of the cross-layer routing outputs ("Mechanisms, trade-offs and
cross-layer routing of linear-attention architectures", "Methodology" and
"Technical details"): lam_forward_side's per-token residual (CLER) and write
value (CLVR), and lam_route's h + s P^T, against the oracle on the same
seeded inputs.

Gates (derived from where each path rounds):
  * residual, fp32 storage (fp32 arithmetic end to end): e_rel <= 1e-4, the
    forward's fp32 bar;
  * residual, bf16 storage: the value is rounded to bf16 once (and, on the
    chunked schedule, carried through bf16 matrix-core operands like `out`):
    the forward's bf16 bar on `out`, e_abs <= 2e-2 with an e_rel <= 1e-2
    tripwire;
  * write value: v itself is emitted bit for bit; Gated DeltaNet-2's w * v is
    one fp32 product, rounded to the storage dtype: |err| <= 2^-8 |ref|
    (bf16) or 2^-23 |ref| (fp32) per element;
  * route: the bf16 products are exact in fp32 and summed in fp32, then
    h + sum is rounded once to bf16: |err| <= 2^-8 |ref| + 1e-4 per element
    (the 1e-4 bounds the fp32 sum of up to 1024 products of size ~0.6)
    (fp32: 1e-5 of max |ref|).
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


def _w(variant, dtype, B, T, H, dk, dv, seed, gate_mu=-1.0):
    return I.Workload(f"side_{variant}_{dtype}_B{B}_T{T}_H{H}_dk{dk}_dv{dv}", variant, dtype, B, T, H, dk, dv,
                      seed=seed, gate_mu=gate_mu)


def _gpu(w, x, side, algo="auto", state_in=None):
    import torch

    import gated_linear_attention_chunked_amd as lam

    g = I.to_device(x, w.dtype, "cuda")
    si = None if state_in is None else torch.from_numpy(state_in.astype(np.float32)).cuda()
    kw = dict(alpha=g.get("alpha"), erase_b=g.get("erase_b"), write_w=g.get("write_w"), state_in=si, algo=algo)
    out, st, sd = lam.forward(w.variant, g["q"], g["k"], g["v"], g["beta"], side=side, **kw)
    out0, st0 = lam.forward(w.variant, g["q"], g["k"], g["v"], g["beta"], **kw)
    torch.cuda.synchronize()
    # asking for the side output changes nothing else
    assert torch.equal(out, out0) and torch.equal(st, st0), "side output changed the scan"
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return f(out), f(st), f(sd)


def _oracle(w, x, side, state_in=None):
    return oracle.delta_forward(w.variant, x["q"], x["k"], x["v"], x["beta"], alpha=x.get("alpha"),
                                erase_b=x.get("erase_b"), write_w=x.get("write_w"), state_in=state_in, side=side)


def _check_side(w, side, got, ref, label):
    if side == "value":
        if w.variant != "gdn2":
            np.testing.assert_array_equal(got, ref, err_msg=label)
        else:
            tol = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -23
            assert np.all(np.abs(got - ref) <= tol * np.abs(ref)), label
        return
    e_abs, e_rel = U.errs(got, ref)
    if w.dtype == "f32":
        assert e_rel <= U.F32_REL, f"{label} residual e_rel={e_rel:.3e}"
    else:
        assert e_abs <= U.BF16_ABS, f"{label} residual e_abs={e_abs:.3e}"
        assert e_rel <= U.BF16_REL_TRIPWIRE, f"{label} residual e_rel={e_rel:.3e}"


@pytest.mark.parametrize("side", ["residual", "value"])
@pytest.mark.parametrize("algo", ["recurrent", "auto"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", DELTA)
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (32, 96), (128, 64)])
def test_side_small(variant, dtype, algo, side, dk, dv):
    """Every element; 83 tokens (two 64-token chunks, five 16-token
    sub-chunks, ragged tail), non-zero initial state."""
    w = _w(variant, dtype, 2, 83, 3, dk, dv, seed=4000 + dk + dv)
    x = I.make_inputs(w)
    s0 = (np.random.default_rng(9).standard_normal((2, 3, dv, dk)) * 0.2).astype(np.float32).astype(np.float64)
    out, st, sd = _gpu(w, x, side, algo=algo, state_in=s0)
    ro, rs, rsd = _oracle(w, x, side, state_in=s0)
    U.check(w, (out, st), (ro, rs), label=w.name, exact_f32=(algo == "recurrent"))
    _check_side(w, side, sd, rsd, f"{w.name} {algo} {side}")


@pytest.mark.parametrize("variant", DELTA)
def test_residual_at_zero_beta(variant):
    """beta = 0 on some tokens: nothing is written there, yet r is still the
    target minus the decayed prediction (the chunked scan carries r itself,
    not beta r)."""
    w = _w(variant, "bf16", 1, 130, 2, 128, 128, seed=4100)
    x = I.make_inputs(w)
    x["beta"][:, ::3] = 0.0
    out, st, sd = _gpu(w, x, "residual")
    ro, rs, rsd = _oracle(w, x, "residual")
    U.check(w, (out, st), (ro, rs), label=w.name)
    _check_side(w, "residual", sd, rsd, w.name)


@pytest.mark.parametrize("name", ["gdn_bf16_B8_T4096_H8_d128", "gdn2_bf16_B8_T4096_H8_d128"])
def test_residual_full_size_sampled(name):
    w = I.WORKLOADS[name]
    x = I.make_inputs(w)
    got = _gpu(w, x, "residual")
    chains = [(0, 0), (5, 3), (7, 7)]
    ref = U.run_oracle(w, x, chains=chains)
    sel = lambda a: np.concatenate([a[b:b + 1, :, h:h + 1] for b, h in chains], 0)
    xs = {k: sel(v) for k, v in x.items()}
    rsd = oracle.delta_forward(w.variant, xs["q"], xs["k"], xs["v"], xs["beta"], alpha=xs.get("alpha"),
                               erase_b=xs.get("erase_b"), write_w=xs.get("write_w"), side="residual")[2]
    U.check(w, U.pick_chains(got[:2], chains), ref, label=name)
    _check_side(w, "residual", sel(got[2]), rsd, name)


def _route_case(dtype, B, T, H, dv, D, seed, zero_p=False):
    import torch

    import gated_linear_attention_chunked_amd as lam

    r = np.random.default_rng(seed)
    N = H * dv
    h = I.round_f32(r.standard_normal((B, T, D))).astype(np.float64)
    s = I.round_f32(r.standard_normal((B, T, H, dv))).astype(np.float64)
    P = np.zeros((D, N)) if zero_p else I.round_f32(r.standard_normal((D, N)) / np.sqrt(N)).astype(np.float64)
    if dtype == "bf16":
        h, s, P = (I.round_bf16(a.astype(np.float32)).astype(np.float64) for a in (h, s, P))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda a: torch.from_numpy(a.astype(np.float32)).cuda().to(tdt)
    hg = dev(h)
    lam.route(hg, dev(s), dev(P))
    torch.cuda.synchronize()
    return hg.float().cpu().numpy().astype(np.float64), h, s, P


def _check_route(dtype, got, ref, label):
    if dtype == "bf16":
        bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + 1e-4
        assert not bad.any(), f"{label}: {bad.sum()} elements off, max err {np.max(np.abs(got - ref)):.3e}"
    else:
        assert U.errs(got, ref)[1] <= 1e-5, label


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,T,H,dv,D", [(1, 1, 1, 32, 16), (2, 83, 3, 64, 48), (1, 300, 8, 128, 1024),
                                         (3, 257, 2, 96, 272)])
def test_route_small(dtype, B, T, H, dv, D):
    """Every element: ragged token counts (tiles of 256), widths not a
    multiple of the 128-column tile, signal widths not a multiple of the
    reduction step."""
    got, h, s, P = _route_case(dtype, B, T, H, dv, D, seed=B * 1000 + T + D)
    _check_route(dtype, got, oracle.route(h, s, P), f"route {dtype} {B}x{T} N={H * dv} D={D}")


def test_route_zero_projection_is_identity():
    """P = 0 (its initial value): the stream passes through bit for bit."""
    got, h, _, _ = _route_case("bf16", 2, 130, 8, 128, 1024, seed=7, zero_p=True)
    np.testing.assert_array_equal(got, h)


def test_route_full_size_sampled():
    """B8 T4096 H8 dv128 into a 1024-wide stream (the pages' 350M-class
    width), every column of 97 sampled tokens."""
    got, h, s, P = _route_case("bf16", 8, 4096, 8, 128, 1024, seed=11)
    idx = np.random.default_rng(1).choice(8 * 4096, 97, replace=False)
    hb, sb = h.reshape(-1, 1024)[idx][None], s.reshape(8 * 4096, 8, 128)[idx][None]
    _check_route("bf16", got.reshape(-1, 1024)[idx][None], oracle.route(hb, sb, P), "route full size")
