"""GPU parity: the HIP scan (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Small cases compare every element; the full-size
workloads run at their real shapes and compare sampled (b, h) chains, which
the oracle computes one by one.
"""
import numpy as np
import pytest

from gated_linear_attention_chunked_amd import inputs as I
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

DELTA = ["deltanet", "gdn", "kda", "gdn2"]
SHAPES = [(32, 32), (64, 64), (96, 96), (128, 128), (128, 64), (64, 128), (32, 96)]


def _w(variant, dtype, B, T, H, dk, dv, seed, gate_mu=2.0):
    return I.Workload(f"{variant}_{dtype}_B{B}_T{T}_H{H}_dk{dk}_dv{dv}", variant, dtype, B, T, H,
                      dk, dv, seed=seed, gate_mu=gate_mu)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    import gated_linear_attention_chunked_amd as lam

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lam.library()


@pytest.mark.parametrize("algo", ["recurrent", "auto"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", DELTA)
@pytest.mark.parametrize("dk,dv", SHAPES)
def test_delta_small(variant, dtype, dk, dv, algo):
    """Every element, ragged length spanning several tiles, weak and strong
    decays mixed across heads by the seed, non-zero initial state."""
    w = _w(variant, dtype, 2, 83, 3, dk, dv, seed=1000 + dk + dv, gate_mu=-1.0)
    x = I.make_inputs(w)
    s0 = np.random.default_rng(5).standard_normal((2, 3, dv, dk)) * 0.2
    s0 = s0.astype(np.float32).astype(np.float64)
    got = U.run_gpu(w, x, algo=algo, state_in=s0)
    ref = U.run_oracle(w, x, state_in=s0)
    U.check(w, got, ref, label=w.name, exact_f32=(algo == "recurrent"))


@pytest.mark.parametrize("variant", DELTA)
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 130])
def test_delta_lengths(variant, T):
    w = _w(variant, "bf16", 1, T, 2, 128, 128, seed=2000 + T, gate_mu=-4.0)
    x = I.make_inputs(w)
    U.check(w, U.run_gpu(w, x), U.run_oracle(w, x), label=w.name)


@pytest.mark.parametrize("variant", DELTA)
def test_weak_decay_long(variant):
    """alpha ~ 0.98: the memory spans hundreds of tokens, so a dropped or
    mis-ordered state carry cannot hide behind fast forgetting."""
    w = _w(variant, "bf16", 2, 700, 2, 128, 128, seed=3000, gate_mu=-4.0)
    x = I.make_inputs(w)
    U.check(w, U.run_gpu(w, x), U.run_oracle(w, x), label=w.name)


@pytest.mark.parametrize("variant", DELTA)
def test_empty_sequence_copies_state(variant):
    import torch

    import gated_linear_attention_chunked_amd as lam

    w = _w(variant, "f32", 2, 0, 2, 64, 64, seed=1)
    x = I.make_inputs(w)
    g = I.to_device(x, "f32", "cuda")
    s0 = torch.randn(2, 2, 64, 64, device="cuda")
    out, st = lam.forward(variant, g["q"], g["k"], g["v"], g["beta"], alpha=g.get("alpha"),
                          erase_b=g.get("erase_b"), write_w=g.get("write_w"), state_in=s0)
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 2, 64)
    assert torch.equal(st, s0)


@pytest.mark.parametrize("variant", DELTA)
def test_chained_calls_and_in_place_state(variant):
    """[0, T) in one call equals two calls chained through the state, with the
    second call updating its state buffer in place."""
    import torch

    import gated_linear_attention_chunked_amd as lam

    w = _w(variant, "bf16", 2, 200, 2, 128, 128, seed=4000, gate_mu=-3.0)
    x = I.make_inputs(w)
    g = I.to_device(x, w.dtype, "cuda")
    ks = [k for k in ("q", "k", "v", "beta", "alpha", "erase_b", "write_w") if k in g]
    full_out, full_st = lam.forward(variant, **{k: g[k] for k in ks})
    a = {k: g[k][:, :77].contiguous() for k in ks}
    b = {k: g[k][:, 77:].contiguous() for k in ks}
    o1, st = lam.forward(variant, **a)
    o2, st2 = lam.forward(variant, **b, state_in=st, state_out=st)
    torch.cuda.synchronize()
    assert st2.data_ptr() == st.data_ptr()
    got = (torch.cat([o1, o2], 1).float().cpu().numpy().astype(np.float64),
           st.cpu().numpy().astype(np.float64))
    ref = U.run_oracle(w, x)
    U.check(w, got, ref, label="chained " + variant)
    d = (torch.cat([o1, o2], 1).float() - full_out.float()).abs().max().item()
    assert d <= 2e-2


@pytest.mark.parametrize("variant", DELTA)
def test_bitwise_reproducible(variant):
    import torch

    w = _w(variant, "bf16", 2, 300, 4, 128, 128, seed=5000, gate_mu=0.0)
    x = I.make_inputs(w)
    r1 = U.run_gpu(w, x)
    r2 = U.run_gpu(w, x)
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("variant,T,dk", [("gdn", 1024, 128), ("gdn", 1093, 64), ("deltanet", 1100, 128),
                                          ("gdn2", 1030, 128), ("gdn", 2047, 128),
                                          ("kda", 1280, 128), ("kda", 1297, 64)])
def test_chunked_long_sequences(variant, T, dk):
    """Sixteen chunks and more, even and odd chunk counts, a ragged tail and
    a carried-in state; two runs agree bit for bit.  Kimi Delta: 40 pairs of
    16-token sub-chunks, and 41 pairs whose last ends in a padded odd
    sub-chunk, many times round the producers' slot ring."""
    w = _w(variant, "bf16", 1, T, 2, dk, 64, seed=7700 + T)
    x = I.make_inputs(w)
    s0 = (np.random.default_rng(T).standard_normal((1, 2, 64, dk)) * 0.2).astype(np.float64)
    got = U.run_gpu(w, x, algo="chunked", state_in=s0)
    again = U.run_gpu(w, x, algo="chunked", state_in=s0)
    for a_, b_ in zip(got, again):
        assert np.array_equal(a_, b_)
    ref = U.run_oracle(w, x, state_in=s0)
    U.check(w, got, ref, label=w.name)


@pytest.mark.parametrize("variant,dtype", [("gdn", "bf16"), ("gdn2", "bf16"), ("kda", "bf16"),
                                           ("gdn", "f32"), ("gdn2", "f32"), ("deltanet", "f32")])
def test_chunked_workspaces_streams_and_threads(variant, dtype):
    """The caller owns the workspace.  Calls queued on two streams with a
    workspace each, a small call reusing a large call's workspace on one
    stream, and calls from two host threads on one stream (each with a
    workspace from torch's allocator) must all give the results of isolated
    calls, bit for bit (fp32 storage: the fp32 chunked form)."""
    import threading

    import torch

    import gated_linear_attention_chunked_amd as lam

    shapes = [(2, 900, 4, 128, 128), (3, 130, 2, 64, 64)]
    ws = [_w(variant, dtype, *sh, seed=5100 + i) for i, sh in enumerate(shapes)]
    xs = [I.make_inputs(w) for w in ws]
    alone = [U.run_gpu(w, x, algo="chunked") for w, x in zip(ws, xs)]
    gs = [I.to_device(x, dtype, "cuda") for x in xs]

    def call(g, **kw):
        return lam.forward(variant, g["q"], g["k"], g["v"], g["beta"], alpha=g.get("alpha"),
                           erase_b=g.get("erase_b"), write_w=g.get("write_w"), algo="chunked", **kw)

    def same(res, ref):
        out, st = res
        assert np.array_equal(out.float().cpu().numpy().astype(np.float64), ref[0])
        assert np.array_equal(st.cpu().numpy().astype(np.float64), ref[1])

    need = [lam.workspace_size(variant, dtype, *sh, algo="chunked") for sh in shapes]
    assert need[0] > need[1] > 0
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.empty(n, dtype=torch.uint8, device="cuda") for n in need]
    torch.cuda.synchronize()
    res = []
    for rep in range(3):
        for g, st, w_ in zip(gs, streams, wss):
            with torch.cuda.stream(st):
                res.append(call(g, stream=st, workspace=w_))
    torch.cuda.synchronize()
    for i, r in enumerate(res):
        same(r, alone[i % 2])
    # one workspace, a large call then a small one on the same stream
    big = torch.empty(need[0], dtype=torch.uint8, device="cuda")
    r0 = call(gs[0], workspace=big)
    r1 = call(gs[1], workspace=big)
    torch.cuda.synchronize()
    same(r0, alone[0])
    same(r1, alone[1])
    # two host threads on the current stream, each call with its own workspace
    out = [None] * 6
    errs = []

    def worker(j):
        try:
            for i in range(3):
                out[3 * j + i] = call(gs[(i + j) % 2])
        except Exception as e:  # reported below
            errs.append(e)

    th = [threading.Thread(target=worker, args=(j,)) for j in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for j in range(2):
        for i in range(3):
            same(out[3 * j + i], alone[(i + j) % 2])


def test_workspace_too_small_is_rejected():
    import torch

    import gated_linear_attention_chunked_amd as lam

    w = _w("gdn", "bf16", 1, 200, 2, 128, 128, seed=5)
    g = I.to_device(I.make_inputs(w), "bf16", "cuda")
    need = lam.workspace_size("gdn", "bf16", 1, 200, 2, 128, 128)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        lam.forward("gdn", g["q"], g["k"], g["v"], g["beta"], alpha=g["alpha"], workspace=small)
    # through the C ABI directly (the binding's own size check bypassed)
    lib = lam.library()
    out = torch.empty_like(g["v"])
    rc = lib.lam_forward(1, 1, 1, 200, 2, 128, 128, g["q"].data_ptr(), g["k"].data_ptr(),
                         g["v"].data_ptr(), g["alpha"].data_ptr(), None, None, g["beta"].data_ptr(),
                         None, out.data_ptr(), None, small.data_ptr(), small.numel(), 0,
                         torch.cuda.current_stream().cuda_stream)
    assert rc == 1  # LAM_ERR_INVALID_ARG, before any work is enqueued


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
def test_vla_small(d, dtype, algo):
    w = I.Workload(f"vla_{dtype}_B2_T75_H3_d{d}", "vla", dtype, 2, 75, 3, d, d, seed=6000 + d)
    x = I.make_inputs(w)
    got = U.run_gpu(w, x, algo=algo)
    ref = U.run_oracle(w, x)
    if dtype == "f32":
        U.check(w, got, ref, label=w.name)
    else:
        e_abs, e_rel = U.errs(got[0], ref[0])
        assert e_abs <= U.BF16_ABS and e_rel <= U.BF16_REL_TRIPWIRE, (e_abs, e_rel)
        for g, r in zip(got[1:], ref[1:]):
            assert U.errs(g, r)[1] <= 1e-4


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
@pytest.mark.parametrize("d", [32, 96])
def test_vla_initial_state_and_chaining(d, algo):
    """Two calls chained through (A, S): a ragged split (40 + 50 tokens), so
    the second call starts from a non-identity penalty inverse and a non-zero
    state."""
    w = I.Workload(f"vla_f32_B1_T90_H2_d{d}", "vla", "f32", 1, 90, 2, d, d, seed=6100 + d)
    x = I.make_inputs(w)
    ref = U.run_oracle(w, x)
    first = {k: v[:, :40] for k, v in x.items()}
    second = {k: v[:, 40:] for k, v in x.items()}
    w1, w2 = w.replace(T=40), w.replace(T=50)
    g1 = U.run_gpu(w1, first, algo=algo)
    g2 = U.run_gpu(w2, second, A_in=g1[1], S_in=g1[2], algo=algo)
    got = (np.concatenate([g1[0], g2[0]], 1), g2[1], g2[2])
    U.check(w, got, ref, label="vla chained " + algo)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 48, 301])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
def test_vla_chunked_lengths(d, T):
    """The 16-token chunked schedule: a single token, one short and one full
    chunk, a ragged tail, several chunks."""
    w = I.Workload(f"vla_f32_B1_T{T}_H2_d{d}", "vla", "f32", 1, T, 2, d, d, seed=6200 + T + d)
    x = I.make_inputs(w)
    U.check(w, U.run_gpu(w, x, algo="chunked"), U.run_oracle(w, x), label=w.name)


# ------------------------------------------------------------ full sizes
FULL_CHAINS = {
    "deltanet_f32_B1_T256_H2_d32": None,                        # every chain
    "gdn_bf16_B8_T4096_H8_d128": [(0, 0), (3, 5), (7, 7), (5, 2)],
    "kda_bf16_B2_T32768_H8_d128": [(0, 3), (1, 6)],
    "gdn2_bf16_B8_T4096_H8_d128": [(0, 1), (6, 4), (7, 7)],
    "vla_f32_B4_T4096_H8_d32": [(0, 0), (2, 5), (3, 7)],
    "vla_f32_B4_T4096_H8_d96": [(1, 1), (3, 6)],
}


@pytest.mark.parametrize("name", list(FULL_CHAINS))
def test_full_workload(name):
    """The real shapes, in the launch configuration the benchmark times
    (algo auto), compared on sampled chains."""
    w = I.WORKLOADS[name]
    x = I.make_inputs(w)
    got = U.run_gpu(w, x)
    chains = FULL_CHAINS[name]
    ref = U.run_oracle(w, x, chains=chains)
    if chains is not None:
        got = U.pick_chains(got, chains)
    rep = U.check(w, got, ref, label=name)
    print(name, rep)


# ---------------------------------------------------- chunked schedule
CHUNKED = ["deltanet", "gdn", "kda", "gdn2"]


@pytest.mark.parametrize("variant", CHUNKED)
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 32), (64, 96), (128, 64)])
@pytest.mark.parametrize("T,gate_mu", [(1, 2.0), (63, -4.0), (64, 2.0), (65, -4.0), (200, 0.0),
                                       (1000, -4.0)])
def test_chunked_every_element(variant, dk, dv, T, gate_mu):
    """The matrix-core chunked schedule, every element, ragged tails, strong
    and weak decays, non-zero initial state."""
    w = _w(variant, "bf16", 2, T, 2, dk, dv, seed=7000 + T + dk, gate_mu=gate_mu)
    x = I.make_inputs(w)
    s0 = (np.random.default_rng(T).standard_normal((2, 2, dv, dk)) * 0.2).astype(np.float32)
    s0 = s0.astype(np.float64)
    got = U.run_gpu(w, x, algo="chunked", state_in=s0)
    ref = U.run_oracle(w, x, state_in=s0)
    U.check(w, got, ref, label=w.name)


@pytest.mark.parametrize("variant", ["gdn", "kda", "gdn2"])
def test_chunked_zero_and_unit_decays(variant):
    """alpha = 0 (memory cleared) and alpha = 1 tokens mixed into one chunk;
    for Kimi Delta also single channels cleared while the rest decay slowly."""
    w = _w(variant, "bf16", 1, 150, 2, 128, 128, seed=7100, gate_mu=-2.0)
    x = I.make_inputs(w)
    x["alpha"][:, 10:13] = 0.0
    x["alpha"][:, 70:90] = 1.0
    if variant == "kda":
        x["alpha"][:, 40, :, 3] = 0.0
        x["alpha"][:, 100:104, 1, 60:70] = 0.0
    got = U.run_gpu(w, x, algo="chunked")
    ref = U.run_oracle(w, x)
    U.check(w, got, ref, label="zero/unit decays " + variant)


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 32)])
def test_kda_chunked_long_in_place(dk, dv):
    """Kimi Delta over a long sequence with few scan workgroups: every
    element against the oracle, with a ragged tail and a carried-in state
    updated in place; two calls in a row (the second reusing the first's
    workspace) agree bit for bit."""
    import torch

    import gated_linear_attention_chunked_amd as lam

    w = _w("kda", "bf16", 1, 8213, 4, dk, dv, seed=9100 + dk)
    x = I.make_inputs(w)
    s0 = (np.random.default_rng(dk).standard_normal((1, 4, dv, dk)) * 0.2).astype(np.float64)
    g = I.to_device(x, w.dtype, "cuda")
    wsp = torch.empty(lam.workspace_size("kda", "bf16", 1, 8213, 4, dk, dv), dtype=torch.uint8, device="cuda")
    runs = []
    for _ in range(2):
        st = torch.from_numpy(s0.astype(np.float32)).cuda()
        out, st2 = lam.forward("kda", g["q"], g["k"], g["v"], g["beta"], alpha=g["alpha"], state_in=st,
                               state_out=st, algo="chunked", workspace=wsp)
        torch.cuda.synchronize()
        assert st2.data_ptr() == st.data_ptr()
        runs.append((out.float().cpu().numpy().astype(np.float64), st.cpu().numpy().astype(np.float64)))
    for a_, b_ in zip(runs[0], runs[1]):
        assert np.array_equal(a_, b_)
    ref = U.run_oracle(w, x, state_in=s0)
    U.check(w, runs[0], ref, label=w.name + " long, in place")


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("gate_mu", [6.0, 4.5, 3.0])
def test_kda_chunked_strong_channel_decay(dk, gate_mu):
    """Per-channel decays strong enough that a 16-token chunk decays some
    channels below 2^-100 (every chunk at mu = 6, some at mu = 4.5), which
    the chunked Kimi Delta kernel handles without factoring the decay."""
    w = _w("kda", "bf16", 2, 333, 2, dk, 64, seed=7200 + dk, gate_mu=gate_mu)
    x = I.make_inputs(w)
    s0 = (np.random.default_rng(dk).standard_normal((2, 2, 64, dk)) * 0.2).astype(np.float32)
    s0 = s0.astype(np.float64)
    got = U.run_gpu(w, x, algo="chunked", state_in=s0)
    ref = U.run_oracle(w, x, state_in=s0)
    U.check(w, got, ref, label=w.name + f" mu={gate_mu}")


@pytest.mark.parametrize("B,H,dk,dv", [(1, 2, 128, 96), (2, 3, 64, 32), (8, 8, 128, 128)])
def test_kda_chunked_tile_shapes(B, H, dk, dv):
    """One 16-column value tile per workgroup (grids of fewer than 256
    two-tile slices) and two per workgroup (B8 H8 dv128: 256 slices)."""
    w = _w("kda", "bf16", B, 70, H, dk, dv, seed=7300 + dv, gate_mu=1.0)
    x = I.make_inputs(w)
    s0 = (np.random.default_rng(dv).standard_normal((B, H, dv, dk)) * 0.2).astype(np.float32)
    s0 = s0.astype(np.float64)
    got = U.run_gpu(w, x, algo="chunked", state_in=s0)
    ref = U.run_oracle(w, x, state_in=s0)
    U.check(w, got, ref, label=w.name)


@pytest.mark.parametrize("T", [16, 33, 70, 300])
@pytest.mark.parametrize("dk", [64, 128])
def test_kda_chunked_two_tiles_repeat(T, dk):
    """Two value tiles per workgroup (B8 H8 dv128), chunk counts from one
    to past the slot ring, with and without a decay strong enough to take
    the exact form; each case runs twice and must match bit for bit, since
    the hand-offs between the waves must not change any result."""
    for mu in (1.0, 5.0):
        w = _w("kda", "bf16", 8, T, 8, dk, 128, seed=7500 + T + dk, gate_mu=mu)
        x = I.make_inputs(w)
        s0 = (np.random.default_rng(T).standard_normal((8, 8, 128, dk)) * 0.2).astype(np.float64)
        r1 = U.run_gpu(w, x, algo="chunked", state_in=s0)
        r2 = U.run_gpu(w, x, algo="chunked", state_in=s0)
        for a, b in zip(r1, r2):
            np.testing.assert_array_equal(a, b)
        ref = U.run_oracle(w, x, state_in=s0)
        U.check(w, r1, ref, label=w.name + f" mu={mu}")


def test_chunked_rejects_unsupported():
    import torch

    import gated_linear_attention_chunked_amd as lam

    w = _w("kda", "bf16", 1, 70, 1, 96, 128, seed=1)
    g = I.to_device(I.make_inputs(w), "bf16", "cuda")
    with pytest.raises(lam.LamError) as e:
        lam.forward("kda", g["q"], g["k"], g["v"], g["beta"], alpha=g["alpha"], algo="chunked")
    assert e.value.status == 2
    w = _w("kda", "f32", 1, 70, 1, 128, 128, seed=1)
    g = I.to_device(I.make_inputs(w), "f32", "cuda")
    with pytest.raises(lam.LamError):
        lam.forward("kda", g["q"], g["k"], g["v"], g["beta"], alpha=g["alpha"], algo="chunked")
    torch.cuda.synchronize()


@pytest.mark.parametrize("variant", ["deltanet", "gdn", "gdn2", "kda"])
def test_chunked_every_element_full_grid(variant):
    """B8 H8 at d128: 64 heads, so the scan's XCD-grouped block-to-head map
    takes its grouped branch; every element against the oracle (ragged
    length, two full chunks plus a tail)."""
    w = _w(variant, "bf16", 8, 130, 8, 128, 128, seed=7300, gate_mu=0.0)
    x = I.make_inputs(w)
    U.check(w, U.run_gpu(w, x, algo="chunked"), U.run_oracle(w, x), label=w.name)


def _plant(w, x):
    """A NaN in chain (0, 1) at token 100 (the decay, or the key for
    DeltaNet) and +Inf in chain (1, 0) at token 70, value channel 5."""
    x = {k_: v_.copy() for k_, v_ in x.items()}
    if w.variant == "deltanet":
        x["k"][0, 100, 1, 3] = np.nan
    elif w.variant == "kda":
        x["alpha"][0, 100, 1, 7] = np.nan
    else:
        x["alpha"][0, 100, 1] = np.nan
    x["v"][1, 70, 0, 5] = np.inf
    return x


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
@pytest.mark.parametrize("variant", DELTA)
def test_non_finite_inputs_propagate(variant, algo):
    """Non-finite inputs neither crash nor leak: chains without them match
    the oracle at the usual gates; in a chain with one, every output the
    oracle makes non-finite is non-finite too, and the final state is
    non-finite where the oracle's is.  Rows before the planted token match
    the oracle, except that the chunked schedule may also turn earlier rows
    of the planted token's own 64-token chunk non-finite (its masked
    in-chunk products multiply zeros by the non-finite values)."""
    w = _w(variant, "bf16", 2, 150, 2, 64, 64, seed=7400)
    x = _plant(w, I.make_inputs(w))
    got = U.run_gpu(w, x, algo=algo)
    ref = U.run_oracle(w, x)
    clean = [(0, 0), (1, 1)]
    U.check(w, U.pick_chains(got, clean), U.pick_chains(ref, clean), label=w.name + " clean chains")
    for (b, h), t_bad in (((0, 1), 100), ((1, 0), 70)):
        y, yr = got[0][b, :, h], ref[0][b, :, h]
        bad_ref = ~np.isfinite(yr)
        assert bad_ref[t_bad:].any() and not bad_ref[:t_bad].any()
        assert np.all(~np.isfinite(y[bad_ref])), (b, h)
        first = t_bad if algo == "recurrent" else (t_bad // 64) * 64
        assert np.all(np.isfinite(y[:first]))
        assert np.max(np.abs(y[:first] - yr[:first])) <= U.BF16_ABS
        s, sr = got[1][b, h], ref[1][b, h]
        assert np.all(~np.isfinite(s[~np.isfinite(sr)]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128])
def test_vla_chunked_segments_chained(d, dtype):
    """Sequences long enough for several segments of the inverse-penalty
    chain (each segment past the first starts from an inverted penalty), in
    two calls chained through (A, S), so the second call's segment starts
    also invert the carried-in A; every element against the oracle."""
    w = I.Workload(f"vla_{dtype}_B2_T700_H2_d{d}", "vla", dtype, 2, 700, 2, d, d, seed=6300 + d)
    x = I.make_inputs(w)
    ref = U.run_oracle(w, x)
    first = {k: v[:, :290] for k, v in x.items()}
    second = {k: v[:, 290:] for k, v in x.items()}
    g1 = U.run_gpu(w.replace(T=290), first, algo="chunked")
    g2 = U.run_gpu(w.replace(T=410), second, A_in=g1[1], S_in=g1[2], algo="chunked")
    got = (np.concatenate([g1[0], g2[0]], 1), g2[1], g2[2])
    # fp32 arithmetic throughout: A and S are held to the fp32 gate for
    # either storage dtype; bf16 outputs take the bf16 gates
    U.check(w, got, ref, label=w.name + " chained", exact_f32=True)


def _step_run(w, x, s0):
    """lam.step over the T tokens of x one at a time (state in place)."""
    import torch

    import gated_linear_attention_chunked_amd as lam

    g = I.to_device(x, w.dtype, "cuda")
    state = torch.from_numpy(s0.astype(np.float32)).cuda()
    outs = []
    for t in range(w.T):
        sl = lambda n: None if g.get(n) is None else g[n][:, t].contiguous()
        outs.append(lam.step(w.variant, sl("q"), sl("k"), sl("v"), sl("beta"), alpha=sl("alpha"),
                             erase_b=sl("erase_b"), write_w=sl("write_w"), state=state))
    torch.cuda.synchronize()
    return (torch.stack(outs, 1).float().cpu().numpy().astype(np.float64),
            state.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", DELTA)
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (32, 96), (96, 64), (128, 32)])
def test_step_matches_scan(variant, dtype, dk, dv):
    """The decode step, one token at a time for N streams with the memory
    updated in place, against the oracle's scan over the same tokens from the
    same initial memory; every element.  dk = 96 takes the token-recurrent
    kernel, the others the dedicated step kernel."""
    w = _w(variant, dtype, 5, 12, 3, dk, dv, seed=7600 + dk + dv, gate_mu=0.0)
    x = I.make_inputs(w)
    s0 = (np.random.default_rng(dk + dv).standard_normal((5, 3, dv, dk)) * 0.2).astype(np.float32)
    got = _step_run(w, x, s0)
    ref = U.run_oracle(w, x, state_in=s0.astype(np.float64))
    U.check(w, got, ref, label=w.name + " step", exact_f32=True)


@pytest.mark.parametrize("variant", ["gdn", "kda"])
def test_step_full_decode_shape(variant):
    """One step at the decode bench shape (256 streams x 8 heads, d = 128,
    bf16 tokens) from a random fp32 memory: every element."""
    w = _w(variant, "bf16", 256, 1, 8, 128, 128, seed=7650, gate_mu=2.0)
    x = I.make_inputs(w)
    s0 = (np.random.default_rng(3).standard_normal((256, 8, 128, 128)) * 0.1).astype(np.float32)
    got = _step_run(w, x, s0)
    ref = U.run_oracle(w, x, state_in=s0.astype(np.float64))
    U.check(w, got, ref, label=w.name + " step", exact_f32=True)


@pytest.mark.parametrize("d", [32, 64, 96, 128])
def test_vla_step_matches_scan(d):
    """lam_vla_step, one token at a time for N streams with A and S updated
    in place, against the oracle's VLA scan; every element."""
    import torch

    import gated_linear_attention_chunked_amd as lam

    w = I.Workload(f"vla_f32_B3_T10_H2_d{d}", "vla", "f32", 3, 10, 2, d, d, seed=7700 + d)
    x = I.make_inputs(w)
    g = I.to_device(x, "f32", "cuda")
    A = torch.eye(d, device="cuda").expand(3, 2, d, d).contiguous()
    S = torch.zeros(3, 2, d, d, device="cuda")
    outs = [lam.vla_step(*(g[n][:, t].contiguous() for n in ("q", "k", "v", "p")), A, S)
            for t in range(w.T)]
    torch.cuda.synchronize()
    got = (torch.stack(outs, 1).cpu().numpy().astype(np.float64), A.cpu().numpy().astype(np.float64),
           S.cpu().numpy().astype(np.float64))
    U.check(w, got, U.run_oracle(w, x), label=w.name + " step")
