"""GPU parity of the fp32 chunked delta-rule schedule against the fp64 oracle.

The schedule works on 16-token chunks with fp32 matrix-core products: an
intra-chunk pass builds each chunk's record (the unit-lower inverse of the
chunk's key Gram matrix under decay and write strength, the transformed keys
and queries, the decay-scaled write keys), then one workgroup per (b, h,
16-column value slice) carries the state across chunks.  It takes DeltaNet,
Gated DeltaNet and Gated DeltaNet-2 with fp32 storage at every head size, and
with bf16 storage at the key widths the bf16 schedule does not take (32, 96).
Every case here asks for it explicitly (algo "chunked").
"""
import numpy as np
import pytest

from gated_linear_attention_chunked_amd import inputs as I
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

VARIANTS = ["deltanet", "gdn", "gdn2"]


def _w(variant, dtype, B, T, H, dk, dv, seed, gate_mu=2.0):
    return I.Workload(f"{variant}_{dtype}_B{B}_T{T}_H{H}_dk{dk}_dv{dv}", variant, dtype, B, T, H,
                      dk, dv, seed=seed, gate_mu=gate_mu)


def _s0(seed, B, H, dk, dv):
    s = np.random.default_rng(seed).standard_normal((B, H, dv, dk)) * 0.2
    return s.astype(np.float32).astype(np.float64)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    import gated_linear_attention_chunked_amd as lam

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lam.library()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 64), (96, 96), (128, 128), (128, 32), (32, 128),
                                   (96, 64)])
@pytest.mark.parametrize("T,gate_mu", [(1, 2.0), (16, -4.0), (17, 0.0), (83, -1.0), (300, 2.0)])
def test_f32_every_element(variant, dk, dv, T, gate_mu):
    """fp32 storage, every element: a single token, one whole chunk, a chunk
    plus one, ragged lengths over several chunks; strong and weak decays;
    non-zero initial state."""
    w = _w(variant, "f32", 2, T, 2, dk, dv, seed=9000 + T + dk + 3 * dv, gate_mu=gate_mu)
    x = I.make_inputs(w)
    s0 = _s0(T + dk, 2, 2, dk, dv)
    got = U.run_gpu(w, x, algo="chunked", state_in=s0)
    U.check(w, got, U.run_oracle(w, x, state_in=s0), label=w.name)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dk,dv", [(32, 32), (96, 96), (32, 128), (96, 64)])
@pytest.mark.parametrize("T", [17, 200])
def test_bf16_narrow_keys(variant, dk, dv, T):
    """bf16 storage at key widths 32 and 96 (the bf16 schedule takes 64 and
    128 only): loads widen to fp32, the output rounds to bf16."""
    w = _w(variant, "bf16", 2, T, 3, dk, dv, seed=9100 + T + dk + dv, gate_mu=-1.0)
    x = I.make_inputs(w)
    s0 = _s0(T + 1, 2, 3, dk, dv)
    got = U.run_gpu(w, x, algo="chunked", state_in=s0)
    U.check(w, got, U.run_oracle(w, x, state_in=s0), label=w.name)


@pytest.mark.parametrize("variant,dk", [("deltanet", 128), ("gdn", 128), ("gdn2", 96), ("gdn", 32)])
def test_long_weak_decay(variant, dk):
    """alpha ~ 0.98 over 2,000 tokens (125 chunks): the state carried across
    chunks dominates the output, so an error in the carry accumulates where
    the gate sees it."""
    w = _w(variant, "f32", 1, 2000, 2, dk, dk, seed=9200 + dk, gate_mu=-4.0)
    x = I.make_inputs(w)
    got = U.run_gpu(w, x, algo="chunked")
    U.check(w, got, U.run_oracle(w, x), label=w.name)


@pytest.mark.parametrize("variant", ["gdn", "gdn2"])
@pytest.mark.parametrize("gate_mu", [8.0, 30.0])
def test_strong_decay(variant, gate_mu):
    """alpha ~ 3e-4 and ~ 1e-13: the cumulative decay inside one chunk falls
    far below the fp32 range; the clamped per-token logarithm keeps every
    exponent difference finite and the products small, not NaN."""
    w = _w(variant, "f32", 1, 150, 2, 64, 64, seed=9300, gate_mu=gate_mu)
    x = I.make_inputs(w)
    s0 = _s0(3, 1, 2, 64, 64)
    got = U.run_gpu(w, x, algo="chunked", state_in=s0)
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1]))
    U.check(w, got, U.run_oracle(w, x, state_in=s0), label=f"{w.name} mu={gate_mu}")


@pytest.mark.parametrize("variant", ["gdn", "gdn2"])
def test_zero_and_unit_decays(variant):
    """alpha = 0 (the memory cleared) and alpha = 1 mixed inside chunks, and a
    chunk whose write strengths are all zero."""
    w = _w(variant, "f32", 1, 150, 2, 128, 128, seed=9400, gate_mu=-2.0)
    x = I.make_inputs(w)
    x["alpha"][:, 10:13] = 0.0
    x["alpha"][:, 37] = 0.0
    x["alpha"][:, 70:90] = 1.0
    x["beta"][:, 96:112] = 0.0
    got = U.run_gpu(w, x, algo="chunked")
    U.check(w, got, U.run_oracle(w, x), label="zero/unit decays " + variant)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dtype,dk", [("f32", 128), ("bf16", 96)])
def test_chained_in_place(variant, dtype, dk):
    """[0, T) in one call against three calls chained through the state at
    cuts inside chunks, the later calls updating the state in place."""
    import torch

    import gated_linear_attention_chunked_amd as lam

    w = _w(variant, dtype, 2, 300, 2, dk, 64, seed=9500 + dk, gate_mu=-3.0)
    x = I.make_inputs(w)
    g = I.to_device(x, w.dtype, "cuda")
    ks = [k for k in ("q", "k", "v", "beta", "alpha", "erase_b", "write_w") if k in g]
    outs, st = [], None
    for lo, hi in ((0, 77), (77, 78), (78, 300)):
        part = {k: g[k][:, lo:hi].contiguous() for k in ks}
        if st is None:
            o, st = lam.forward(variant, **part, algo="chunked")
        else:
            o, st2 = lam.forward(variant, **part, state_in=st, state_out=st, algo="chunked")
            assert st2.data_ptr() == st.data_ptr()
        outs.append(o)
    torch.cuda.synchronize()
    got = (torch.cat(outs, 1).float().cpu().numpy().astype(np.float64),
           st.cpu().numpy().astype(np.float64))
    U.check(w, got, U.run_oracle(w, x), label=f"chained {variant} {dtype}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_bitwise_reproducible(variant):
    w = _w(variant, "f32", 2, 301, 3, 96, 96, seed=9600, gate_mu=0.0)
    x = I.make_inputs(w)
    r1 = U.run_gpu(w, x, algo="chunked")
    r2 = U.run_gpu(w, x, algo="chunked")
    for a, b in zip(r1, r2):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("variant,dk", [("gdn", 128), ("gdn2", 96), ("deltanet", 32)])
def test_full_grid(variant, dk):
    """B8 H8: 64 heads times the value slices; every element (two whole
    chunks of 64 and a ragged tail)."""
    w = _w(variant, "f32", 8, 141, 8, dk, dk, seed=9700 + dk, gate_mu=0.0)
    x = I.make_inputs(w)
    U.check(w, U.run_gpu(w, x, algo="chunked"), U.run_oracle(w, x), label=w.name)


def test_full_size_sampled():
    """Gated DeltaNet with fp32 storage at B8 T4096 H8 d128, sampled chains."""
    w = _w("gdn", "f32", 8, 4096, 8, 128, 128, seed=2, gate_mu=2.0)
    x = I.make_inputs(w)
    chains = [(0, 0), (4, 3), (7, 7)]
    got = U.pick_chains(U.run_gpu(w, x, algo="chunked"), chains)
    U.check(w, got, U.run_oracle(w, x, chains=chains), label=w.name)


@pytest.mark.parametrize("variant", VARIANTS)
def test_non_finite_inputs_propagate(variant):
    """A NaN in chain (0, 1) at token 100 and +Inf in chain (1, 0) at token 70:
    the clean chains match the oracle, every output the oracle makes
    non-finite is non-finite, and rows before the planted token's 16-token
    chunk stay finite and match."""
    w = _w(variant, "f32", 2, 150, 2, 64, 64, seed=9800)
    x = {k_: v_.copy() for k_, v_ in I.make_inputs(w).items()}
    if variant == "deltanet":
        x["k"][0, 100, 1, 3] = np.nan
    else:
        x["alpha"][0, 100, 1] = np.nan
    x["v"][1, 70, 0, 5] = np.inf
    got = U.run_gpu(w, x, algo="chunked")
    ref = U.run_oracle(w, x)
    clean = [(0, 0), (1, 1)]
    U.check(w, U.pick_chains(got, clean), U.pick_chains(ref, clean), label=w.name + " clean")
    for (b, h), t_bad in (((0, 1), 100), ((1, 0), 70)):
        y, yr = got[0][b, :, h], ref[0][b, :, h]
        bad_ref = ~np.isfinite(yr)
        assert bad_ref[t_bad:].any() and not bad_ref[:t_bad].any()
        assert np.all(~np.isfinite(y[bad_ref])), (b, h)
        first = (t_bad // 16) * 16
        assert np.all(np.isfinite(y[:first]))
        e = np.max(np.abs(y[:first] - yr[:first])) / np.max(np.abs(yr[:first]))
        assert e <= U.F32_REL
        s, sr = got[1][b, h], ref[1][b, h]
        assert np.all(~np.isfinite(s[~np.isfinite(sr)]))
