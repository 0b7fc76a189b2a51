"""Helpers for the GPU parity tests: run a workload through the C ABI and
compare it with the fp64 oracle on the same seeded inputs.

Error measures (per output tensor, each compared separately):
  e_abs = max |y - y_ref|
  e_rel = max |y - y_ref| / max |y_ref|
Gates: fp32 storage -> e_rel <= 1e-4 on every output; bf16 storage ->
e_abs <= 2e-2 on `out` and on the fp32 final state (both of order one), plus
an e_rel <= 1e-2 tripwire on each.  ``exact_f32=True`` (schedules whose
arithmetic is fp32 end to end, such as the token-recurrent one) holds the
final state of bf16 workloads to e_rel <= 1e-4 as well.
"""
from __future__ import annotations

import numpy as np

import oracle
from gated_linear_attention_chunked_amd import inputs as I

F32_REL = 1e-4
BF16_ABS = 2e-2
BF16_REL_TRIPWIRE = 1e-2
STATE_REL = 1e-4


def errs(y, ref):
    y = np.asarray(y, np.float64)
    d = np.max(np.abs(y - ref)) if ref.size else 0.0
    m = np.max(np.abs(ref)) if ref.size else 1.0
    return float(d), float(d / m) if m > 0 else float(d)


def run_gpu(w: I.Workload, x: dict, algo="auto", state_in=None, A_in=None, S_in=None):
    import torch

    import gated_linear_attention_chunked_amd as lam

    g = I.to_device(x, w.dtype, "cuda")
    if w.variant == "vla":
        Ai = None if A_in is None else torch.from_numpy(A_in.astype(np.float32)).cuda()
        Si = None if S_in is None else torch.from_numpy(S_in.astype(np.float32)).cuda()
        out, A, S = lam.vla_forward(g["q"], g["k"], g["v"], g["p"], Ai, Si, algo=algo)
        torch.cuda.synchronize()
        return (out.float().cpu().numpy().astype(np.float64),
                A.cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64))
    si = None if state_in is None else torch.from_numpy(state_in.astype(np.float32)).cuda()
    out, st = lam.forward(w.variant, g["q"], g["k"], g["v"], g["beta"], alpha=g.get("alpha"),
                          erase_b=g.get("erase_b"), write_w=g.get("write_w"), state_in=si,
                          algo=algo)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), st.cpu().numpy().astype(np.float64)


def run_oracle(w: I.Workload, x: dict, chains=None, state_in=None, A_in=None, S_in=None):
    """Oracle on all chains, or on the listed (b, h) chains (results stacked
    along a leading axis, one [T, dv] output and one state per chain)."""
    if chains is None:
        if w.variant == "vla":
            return oracle.vla_forward(x["q"], x["k"], x["v"], x["p"], A_in=A_in, S_in=S_in)
        return oracle.delta_forward(w.variant, x["q"], x["k"], x["v"], x["beta"], alpha=x.get("alpha"),
                                    erase_b=x.get("erase_b"), write_w=x.get("write_w"),
                                    state_in=state_in)
    # gather the chains into one batch so the oracle runs them in parallel
    idx = list(chains)
    cat = lambda a: None if a is None else np.concatenate([a[b:b + 1, :, h:h + 1] for b, h in idx], 0)
    cats = lambda a: None if a is None else np.concatenate([a[b:b + 1, h:h + 1] for b, h in idx], 0)
    if w.variant == "vla":
        return oracle.vla_forward(cat(x["q"]), cat(x["k"]), cat(x["v"]), cat(x["p"]),
                                  A_in=cats(A_in), S_in=cats(S_in))
    return oracle.delta_forward(w.variant, cat(x["q"]), cat(x["k"]), cat(x["v"]), cat(x["beta"]),
                                alpha=cat(x.get("alpha")), erase_b=cat(x.get("erase_b")),
                                write_w=cat(x.get("write_w")), state_in=cats(state_in))


def pick_chains(gpu_res, chains):
    """Select the same chains from full GPU results (out [B,T,H,d], states [B,H,..])."""
    out = np.concatenate([gpu_res[0][b:b + 1, :, h:h + 1] for b, h in chains], 0)
    sts = [np.concatenate([s[b:b + 1, h:h + 1] for b, h in chains], 0) for s in gpu_res[1:]]
    return (out, *sts)


def check(w: I.Workload, got, ref, label="", exact_f32=False):
    """Assert the gates; return a dict of the measured errors."""
    rep = {}
    e_abs, e_rel = errs(got[0], ref[0])
    rep["out"] = (e_abs, e_rel, float(np.max(np.abs(ref[0]))) if ref[0].size else 0.0)
    if w.dtype == "f32":
        assert e_rel <= F32_REL, f"{label} out e_rel={e_rel:.3e}"
    else:
        assert e_abs <= BF16_ABS, f"{label} out e_abs={e_abs:.3e}"
        assert e_rel <= BF16_REL_TRIPWIRE, f"{label} out e_rel={e_rel:.3e}"
    names = ["A", "S"] if w.variant == "vla" else ["state"]
    for n, g, r in zip(names, got[1:], ref[1:]):
        sa, sr = errs(g, r)
        rep[n] = (sa, sr)
        if w.dtype == "f32" or exact_f32:
            assert sr <= STATE_REL, f"{label} {n} e_rel={sr:.3e}"
        else:
            assert sa <= BF16_ABS, f"{label} {n} e_abs={sa:.3e}"
            assert sr <= BF16_REL_TRIPWIRE, f"{label} {n} e_rel={sr:.3e}"
    return rep
