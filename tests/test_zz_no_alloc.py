"""lam_forward_noalloc (the entry point that allocates nothing: its workspace
is a fixed device array inside the library) against lam_forward, called
through the C ABI: two calls in a row, the second with a smaller input, each
compared with lam_forward on the same inputs (bit for bit: same kernels) and
with the oracle at the bf16 gates; a call needing more than the array holds
is refused before any work is enqueued."""
import numpy as np
import pytest

from gated_linear_attention_chunked_amd import inputs as I
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SCRATCH_LIMIT = 4
SCRATCH_BYTES = 32 << 20


def _call_noalloc(lib, w, g, out, st_out, algo=0):
    import torch

    var = {"deltanet": 0, "gdn": 1, "kda": 2, "gdn2": 3}[w.variant]
    dt = {"f32": 0, "bf16": 1}[w.dtype]
    p = lambda t: None if t is None else t.data_ptr()
    return lib.lam_forward_noalloc(var, dt, w.B, w.T, w.H, w.dk, w.dv, p(g["q"]), p(g["k"]), p(g["v"]),
                                   p(g.get("alpha")), p(g.get("erase_b")), p(g.get("write_w")),
                                   p(g["beta"]), None, p(out), p(st_out), algo,
                                   torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("variant", ["gdn", "gdn2"])
def test_noalloc_matches_forward(variant):
    import torch

    import gated_linear_attention_chunked_amd as lam

    lib = lam.library()
    big = I.Workload(f"{variant}_bf16_B8_T1000_H4_d128", variant, "bf16", 8, 1000, 4, 128, 128, seed=8800)
    small = I.Workload(f"{variant}_bf16_B2_T77_H2_d64", variant, "bf16", 2, 77, 2, 64, 64, seed=8801)
    for w in (big, small):  # the second call is smaller than the first
        assert 0 < lam.workspace_size(w.variant, "bf16", w.B, w.T, w.H, w.dk, w.dv) <= SCRATCH_BYTES
        x = I.make_inputs(w)
        g = I.to_device(x, "bf16", "cuda")
        out = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
        st = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
        assert _call_noalloc(lib, w, g, out, st) == 0
        torch.cuda.synchronize()
        got = (out.float().cpu().numpy().astype(np.float64), st.cpu().numpy().astype(np.float64))
        ref_fwd = U.run_gpu(w, x)
        assert np.array_equal(got[0], ref_fwd[0]) and np.array_equal(got[1], ref_fwd[1]), w.name
        U.check(w, got, U.run_oracle(w, x), label=w.name + " noalloc")


def test_noalloc_refuses_calls_beyond_its_scratch():
    import torch

    import gated_linear_attention_chunked_amd as lam

    lib = lam.library()
    w = I.Workload("kda_bf16_B2_T4096_H8_d128", "kda", "bf16", 2, 4096, 8, 128, 128, seed=3)
    assert lam.workspace_size("kda", "bf16", 2, 4096, 8, 128, 128) > SCRATCH_BYTES
    fake = torch.empty(16, dtype=torch.bfloat16, device="cuda")  # never touched: refused first
    g = {k_: fake for k_ in ("q", "k", "v", "alpha", "beta")}
    assert _call_noalloc(lib, w, g, fake, None, algo=2) == SCRATCH_LIMIT
    assert b"scratch" in lib.lam_status_string(SCRATCH_LIMIT)


def test_noalloc_auto_beyond_its_scratch_runs_recurrent():
    """With algo auto, a call whose fp32 chunk records outgrow the array runs
    the recurrent schedule: bit for bit lam_forward's recurrent result, and the
    oracle's at the fp32 gate on sampled chains; a smaller call after it takes
    the chunked schedule through the array again."""
    import torch

    import gated_linear_attention_chunked_amd as lam

    lib = lam.library()
    big = I.Workload("gdn_f32_B2_T4096_H4_d128", "gdn", "f32", 2, 4096, 4, 128, 128, seed=8802)
    small = I.Workload("gdn_f32_B1_T99_H2_d64", "gdn", "f32", 1, 99, 2, 64, 64, seed=8803)
    assert lam.workspace_size("gdn", "f32", 2, 4096, 4, 128, 128) > SCRATCH_BYTES
    assert 0 < lam.workspace_size("gdn", "f32", 1, 99, 2, 64, 64) <= SCRATCH_BYTES
    for w, algo, chains in ((big, "recurrent", [(0, 1), (1, 3)]), (small, "chunked", None)):
        x = I.make_inputs(w)
        g = I.to_device(x, "f32", "cuda")
        out = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
        st = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
        assert _call_noalloc(lib, w, g, out, st) == 0
        torch.cuda.synchronize()
        got = (out.cpu().numpy().astype(np.float64), st.cpu().numpy().astype(np.float64))
        ref_fwd = U.run_gpu(w, x, algo=algo)
        assert np.array_equal(got[0], ref_fwd[0]) and np.array_equal(got[1], ref_fwd[1]), w.name
        if chains is not None:
            got = U.pick_chains(got, chains)
        U.check(w, got, U.run_oracle(w, x, chains=chains), label=w.name + " noalloc auto")
