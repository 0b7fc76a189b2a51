"""GPU parity of VLA with the output read as a ratio of two recurrences
(lam_vla_forward_ratio, lam_vla_step_ratio; "Technical summary: Variational
Linear Attention (VLA)", section 2.3) against the fp64 oracle.

The kernel is the token-recurrent VLA scan, fp32 throughout, with the
denominator n carried beside S: out, A, S and n are held to the fp32 gate
(e_rel <= 1e-4 per tensor; bf16 storage: out takes the bf16 gates, the fp32
states keep 1e-4).  On these inputs the denominator n . qhat stays within
about [0.6, 1.2], so the division does not amplify the fp32 error.
"""
import numpy as np
import pytest

import oracle
from gated_linear_attention_chunked_amd import inputs as I
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch

    import gated_linear_attention_chunked_amd as lam

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lam.library()


def _gpu(x, dtype, A_in=None, S_in=None, n_in=None):
    import torch

    import gated_linear_attention_chunked_amd as lam

    g = I.to_device(x, dtype, "cuda")
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    r = lam.vla_forward_ratio(g["q"], g["k"], g["v"], g["p"], A_in=f32(A_in), S_in=f32(S_in), n_in=f32(n_in))
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in r)


def _check(got, ref, dtype, label):
    names = ("out", "A", "S", "n")
    for nm, g, r in zip(names, got, ref):
        e_abs, e_rel = U.errs(g, r)
        if nm == "out" and dtype == "bf16":
            assert e_abs <= U.BF16_ABS and e_rel <= U.BF16_REL_TRIPWIRE, (label, nm, e_abs, e_rel)
        else:
            assert e_rel <= 1e-4, (label, nm, e_rel)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
def test_vla_ratio_small(d, dtype):
    """Every element; 75 tokens (several 16-token tiles and a ragged one)."""
    w = I.Workload(f"vla_{dtype}_B2_T75_H3_d{d}", "vla", dtype, 2, 75, 3, d, d, seed=7000 + d)
    x = I.make_inputs(w)
    ref = oracle.vla_forward_ratio(x["q"], x["k"], x["v"], x["p"])
    _check(_gpu(x, dtype), ref, dtype, w.name)


@pytest.mark.parametrize("d", [32, 96])
@pytest.mark.parametrize("T1", [1, 16, 37])
def test_vla_ratio_chained(d, T1):
    """Two calls chained through (A, S, n) give the one-call result."""
    w = I.Workload(f"vla_f32_B1_T70_H2_d{d}", "vla", "f32", 1, 70, 2, d, d, seed=7100 + d)
    x = I.make_inputs(w)
    ref = oracle.vla_forward_ratio(x["q"], x["k"], x["v"], x["p"])
    a = {k: v[:, :T1] for k, v in x.items()}
    b = {k: v[:, T1:] for k, v in x.items()}
    y1, A1, S1, n1 = _gpu(a, "f32")
    y2, A2, S2, n2 = _gpu(b, "f32", A_in=A1, S_in=S1, n_in=n1)
    _check((np.concatenate([y1, y2], 1), A2, S2, n2), ref, "f32", f"chained at {T1}")


@pytest.mark.parametrize("d", [32, 96])
def test_vla_ratio_step_matches_scan(d):
    """lam_vla_step_ratio over the tokens one at a time (A, S, n in place)
    is the same fp32 arithmetic as one scan over them."""
    import torch

    import gated_linear_attention_chunked_amd as lam

    w = I.Workload(f"vla_f32_B3_T20_H2_d{d}", "vla", "f32", 3, 20, 2, d, d, seed=7200 + d)
    x = I.make_inputs(w)
    full = _gpu(x, "f32")
    g = I.to_device(x, "f32", "cuda")
    A = torch.eye(d, device="cuda").repeat(3, 2, 1, 1).contiguous()
    S = torch.zeros((3, 2, d, d), device="cuda")
    n = torch.zeros((3, 2, d), device="cuda")
    outs = [lam.vla_step_ratio(g["q"][:, t].contiguous(), g["k"][:, t].contiguous(), g["v"][:, t].contiguous(),
                               g["p"][:, t].contiguous(), A, S, n) for t in range(20)]
    torch.cuda.synchronize()
    got = (torch.stack(outs, 1).cpu().numpy(), A.cpu().numpy(), S.cpu().numpy(), n.cpu().numpy())
    for a_, b_ in zip(got, full):
        np.testing.assert_allclose(a_, b_, rtol=1e-5, atol=1e-6)


def test_vla_ratio_step_decode_shape():
    """One step at the decode bench shape (256 streams x 8 heads, d = 96)
    from loaded states (identity penalty, a random memory, a uniform
    denominator), every element against the oracle."""
    import torch

    import gated_linear_attention_chunked_amd as lam

    w = I.DECODE_WORKLOADS["vla_ratio_step_f32_N256_H8_d96"]
    x = I.make_inputs(w)
    r = np.random.default_rng(w.seed)
    A0 = np.broadcast_to(np.eye(96), (256, 8, 96, 96)).copy()
    S0 = (r.standard_normal((256, 8, 96, 96)) * 0.1).astype(np.float32).astype(np.float64)
    n0 = np.full((256, 8, 96), 0.8 / np.sqrt(96)).astype(np.float32).astype(np.float64)
    ref = oracle.vla_forward_ratio(x["q"], x["k"], x["v"], x["p"], A_in=A0, S_in=S0, n_in=n0)
    g = I.to_device(x, "f32", "cuda")
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    A, S, n = f32(A0), f32(S0), f32(n0)
    out = lam.vla_step_ratio(g["q"][:, 0].contiguous(), g["k"][:, 0].contiguous(), g["v"][:, 0].contiguous(),
                             g["p"][:, 0].contiguous(), A, S, n)
    torch.cuda.synchronize()
    got = (out.cpu().numpy()[:, None].astype(np.float64), A.cpu().numpy(), S.cpu().numpy(), n.cpu().numpy())
    _check(got, ref, "f32", w.name)
