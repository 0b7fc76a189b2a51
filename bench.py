"""Throughput benchmark of the recurrent-memory forward scan on one MI355X.

Default workload: Gated DeltaNet, bf16 token streams, fp32 state,
B=8 T=4096 H=8 dk=dv=128 (one 350M-class layer's heads at sequence 4096).
A step is one full forward scan of that batch (one lam_forward call) with
its inputs already resident in HBM.  W untimed warm-up steps are followed by
exactly K timed steps between two device synchronisations.  Steps rotate
over three copies of the inputs (3 x 270 MB > the 256 MB last-level cache), so
no step is served from cache by its predecessor.

Printed: one JSON line with tokens/s (tokens = B*T), the roofline object of
the scan kernel (algorithmic bytes per launch / mean launch time from HIP
events on the launch stream, against 8 TB/s HBM) and the fp64 oracle timed
on host cores on a bounded sample of the same workload.

Other lines (``--workload NAME``): the other forward workloads, the decode
step, and the paths beside the forward scan on the same B8 T4096 H8 d128
Gated DeltaNet shapes -- its backward pass, the forward with the per-token
residual side output, the routing product into a 1024-wide stream, the
log-linear readout (13 levels) and its level-weight MLP.  Each reports its
own roofline and its own oracle baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # dense bf16 matrix-core peak
FP32_PEAK_TFS = 157.3


def algorithmic_bytes(w, decode=False) -> int:
    """Every input read once, out and the final state written once (no
    initial state), in the storage dtype.  A decode step also reads the
    state it updates (VLA's decode step, with the ratio read: A, S and the
    denominator n, each read and written)."""
    es = 2 if w.dtype == "bf16" else 4
    n_th = w.B * w.T * w.H
    if decode and w.variant == "vla":
        return n_th * 5 * w.dk * es + 2 * w.B * w.H * (2 * w.dk * w.dk + w.dk) * 4
    if decode:
        return algorithmic_bytes(w) + w.B * w.H * w.dv * w.dk * 4
    if w.variant == "vla":
        per = 5 * w.dk * es                                   # q, k, v, p, out
        state = 2 * w.B * w.H * w.dk * w.dk * 4               # A_out, S_out
        return n_th * per + state
    per = (2 * w.dk + 2 * w.dv + 1) * es                     # q, k, v, out, beta
    if w.variant in ("gdn", "gdn2"):
        per += es                                            # scalar alpha
    if w.variant == "kda":
        per += w.dk * es                                     # per-channel alpha
    if w.variant == "gdn2":
        per += (w.dk + w.dv) * es                            # erase, write
    return n_th * per + w.B * w.H * w.dv * w.dk * 4          # + state_out


def algorithmic_flops(w) -> int:
    """The recurrence's own work per token-head: predict (2 dk dv), decay +
    write (3 dk dv), read (2 dk dv); VLA 12 d^2."""
    n_th = w.B * w.T * w.H
    if w.variant == "vla":
        return n_th * 12 * w.dk * w.dk
    return n_th * 7 * w.dk * w.dv


# Paths beside the forward scan, benchmarked on a forward workload's shapes:
# name -> (kind, forward workload, extra parameters)
JOBS = {
    "gdn_bwd_bf16_B8_T4096_H8_d128": ("backward", "gdn_bf16_B8_T4096_H8_d128", {}),
    "gdn_side_bf16_B8_T4096_H8_d128": ("side", "gdn_bf16_B8_T4096_H8_d128", {}),
    "route_bf16_B8_T4096_N1024_D1024": ("route", "gdn_bf16_B8_T4096_H8_d128", {"D": 1024}),
    "gdn_loglinear_bf16_B8_T4096_H8_d128": ("loglinear", "gdn_bf16_B8_T4096_H8_d128", {}),
    "loglinear_lambda_bf16_B8_T4096_H8_L13": ("lambda", "gdn_bf16_B8_T4096_H8_d128", {"nh": 26}),
    # the throughput workload's forward with fp32 storage (the fp32 chunked form)
    "gdn_f32_B8_T4096_H8_d128": ("forward", "gdn_bf16_B8_T4096_H8_d128", {"dtype": "f32"}),
}


def loglinear_levels(T: int) -> int:
    """Fenwick levels through position T - 1: floor(log2(T - 1)) + 2."""
    return 1 if T - 1 < 1 else (T - 1).bit_length() + 1


def loglinear_occupancy(T: int) -> int:
    """Sum over positions t < T of the levels the readout touches at t: the
    levels holding earlier tokens (one per set bit of t) plus level 0."""
    return sum(bin(t).count("1") + 1 for t in range(T))


def job_counts(kind: str, w, extra=None):
    """(algorithmic bytes, algorithmic flops) of one call of a job.

    backward: reads the forward's inputs and dout in the storage dtype,
      writes every gradient in fp32 (dq, dk, dv, dbeta, dalpha, Gated
      DeltaNet-2's derase_b and dwrite_w, and dstate_in); flops 14 dk dv per
      token-head (each of the forward's 7 dk dv matched by its adjoint twice:
      the reverse sweep's products, recomputation not counted).
    side: the forward's, plus the residual written once in the storage dtype.
    route: s, P and h read once, h written once; flops 2 M N D.
    loglinear: the forward's inputs and out, the level weights (fp32, nL per
      token-head) and nL final level memories; flops 7 dk dv per occupied
      level and token-head.
    lambda: d read in the storage dtype, lambda written in fp32 (weights
      negligible); flops 4 nL nh per row (two products).
    """
    extra = extra or {}
    es = 2 if w.dtype == "bf16" else 4
    n_th = w.B * w.T * w.H
    state = w.B * w.H * w.dv * w.dk * 4
    if kind == "backward":
        nin = (2 * w.dk + 2 * w.dv + 1) * es                 # q, k, v, dout, beta
        nout = (2 * w.dk + w.dv + 1) * 4                     # dq, dk, dv, dbeta
        if w.variant in ("gdn", "gdn2"):
            nin, nout = nin + es, nout + 4
        if w.variant == "kda":
            nin, nout = nin + w.dk * es, nout + w.dk * 4
        if w.variant == "gdn2":
            nin, nout = nin + (w.dk + w.dv) * es, nout + (w.dk + w.dv) * 4
        return n_th * (nin + nout) + state, n_th * 14 * w.dk * w.dv
    if kind == "side":
        return algorithmic_bytes(w) + n_th * w.dv * es, algorithmic_flops(w)
    if kind == "route":
        M, N, D = w.B * w.T, w.H * w.dv, extra["D"]
        return (M * N + D * N + 2 * M * D) * es, 2 * M * N * D
    if kind == "loglinear":
        nL = loglinear_levels(w.T)
        nbytes = algorithmic_bytes(w) - state + n_th * nL * 4 + nL * state
        return nbytes, w.B * w.H * loglinear_occupancy(w.T) * 7 * w.dk * w.dv
    if kind == "lambda":
        nL, nh = loglinear_levels(w.T), extra["nh"]
        return n_th * nL * (es + 4), n_th * 4 * nL * nh
    raise ValueError(kind)


KERNEL_SOURCES = {  # schedule -> kernel source per variant family
    ("chunked", "delta"): "delta_chunked.hip",
    ("chunked", "delta_f32"): "delta_chunked_f32.hip",
    ("chunked", "kda"): "kda_chunked.hip",
    ("chunked", "vla"): "vla_chunked.hip",
    ("recurrent", "delta"): "delta_recurrent.hip",
    ("recurrent", "kda"): "delta_recurrent.hip",
    ("recurrent", "vla"): "vla_recurrent.hip",
    ("step", "delta"): "delta_step.hip",
    ("step", "vla"): "vla_recurrent.hip",
    ("backward", "delta"): "delta_backward.hip",
    ("backward_chunked", "delta"): "delta_chunked_f32.hip",
    ("route", "delta"): "route.hip",
    ("loglinear", "delta"): "loglin_recurrent.hip",
    ("lambda", "delta"): "loglin_recurrent.hip",
}
SHARED_HEADERS = ("chunk_common.h", "chunk_f32.h", "device_common.h", "lam_internal.h")


def bf16_matrix_schedule(w) -> bool:
    """The delta-rule chunked schedules that feed bf16 operands to the matrix
    cores: bf16 storage at dk 64 or 128 (every other delta-rule shape takes
    the fp32 chunked form)."""
    return w.dtype == "bf16" and w.dk in (64, 128)


def kernel_source_hash(ran: str, w):
    """(source file name, sha256 over that source, the shared headers and
    the source's own compiler flags, if it has any)."""
    import hashlib

    from gated_linear_attention_chunked_amd.build import SOURCE_FLAGS

    variant = w.variant
    fam = variant if variant in ("kda", "vla") else "delta"
    if ran == "chunked" and fam == "delta" and not bf16_matrix_schedule(w):
        fam = "delta_f32"
    name = KERNEL_SOURCES.get((ran, fam)) or KERNEL_SOURCES[(ran, "delta")]
    csrc = os.path.join(ROOT, "gated_linear_attention_chunked_amd", "csrc")
    h = hashlib.sha256()
    for f in (name,) + SHARED_HEADERS:
        h.update(open(os.path.join(csrc, f), "rb").read())
    if SOURCE_FLAGS.get(name):
        h.update(" ".join(SOURCE_FLAGS[name]).encode())
    return name, h.hexdigest()


def measured_traffic(w, ran: str, name=None):
    """HBM bytes per launch from the committed rocprofv3 counter record
    (profiles/traffic.json), or None when there is no record for this
    workload and schedule, or it was taken on a different revision of the
    kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))["workloads"][name or w.name]
        name, sha = kernel_source_hash(ran, w)
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("schedule") != ran or rec.get("source") != name or rec.get("sha256") != sha:
        return None
    return float(rec["bytes_per_launch"])


def cpu_threads(chains: int) -> int:
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    cap = int(os.environ.get("OMP_NUM_THREADS", avail) or avail)
    return max(1, min(avail, cap, chains))


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, batch_rows: int, min_seconds: float):
    """The fp64 oracle on the first `batch_rows` batch rows (all heads, all
    tokens) of the same inputs, repeated until at least `min_seconds` of
    wall time have passed (one pass of the whole workload takes well under a
    second on a many-core host); tokens/s over all repetitions."""
    import oracle

    sl = {k: v[:batch_rows] for k, v in x.items()}
    chains = batch_rows * w.H
    th = cpu_threads(chains)
    reps, dt = 0, 0.0
    while reps == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        if w.variant == "vla" and "n_in" in sl:  # decode with the ratio read, from the same states
            oracle.vla_forward_ratio(sl["q"], sl["k"], sl["v"], sl["p"], A_in=sl["A_in"], S_in=sl["S_in"],
                                     n_in=sl["n_in"], nthreads=th)
        elif w.variant == "vla":
            oracle.vla_forward(sl["q"], sl["k"], sl["v"], sl["p"], nthreads=th)
        else:
            oracle.delta_forward(w.variant, sl["q"], sl["k"], sl["v"], sl["beta"], alpha=sl.get("alpha"),
                                 erase_b=sl.get("erase_b"), write_w=sl.get("write_w"),
                                 state_in=sl.get("state_in"), nthreads=th)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": reps * batch_rows * w.T / dt, "unit": "tokens/s", "cores": th, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"fp64 token-by-token oracle on batch rows 0..{batch_rows - 1} of {w.B} "
                      f"(all {w.H} heads, all {w.T} tokens: {chains} chains, "
                      f"{batch_rows * w.T} tokens) of the same inputs, {reps} pass{'es' if reps > 1 else ''} "
                      f"in {dt:.1f} s wall"}


def cpu_baseline_job(kind, w, x, extra, batch_rows: int, min_seconds: float, tokens: int = None):
    """The oracle of a job on the first `batch_rows` batch rows (all heads;
    the first `tokens` tokens when given), repeated for at least
    `min_seconds`; tokens/s over all repetitions."""
    import numpy as np

    import oracle

    T = tokens or w.T
    sl = {k: v[:batch_rows, :T] for k, v in x.items()}
    chains = batch_rows * w.H
    th = cpu_threads(chains)
    r = np.random.default_rng(w.seed + 17)
    if kind == "backward":
        dout = r.standard_normal(sl["v"].shape)
        run = lambda: oracle.delta_backward(w.variant, sl["q"], sl["k"], sl["v"], sl["beta"], dout,
                                            alpha=sl.get("alpha"), erase_b=sl.get("erase_b"),
                                            write_w=sl.get("write_w"), nthreads=th)
        what = "fp64 token-by-token adjoint oracle"
    elif kind == "side":
        run = lambda: oracle.delta_forward(w.variant, sl["q"], sl["k"], sl["v"], sl["beta"], alpha=sl.get("alpha"),
                                           erase_b=sl.get("erase_b"), write_w=sl.get("write_w"), nthreads=th,
                                           side="residual")
        what = "fp64 token-by-token oracle with the residual side output"
    elif kind == "loglinear":
        nL = loglinear_levels(w.T)
        lamw = r.uniform(0.5, 1.5, sl["beta"].shape + (nL,))
        run = lambda: oracle.loglinear_forward(w.variant, sl["q"], sl["k"], sl["v"], sl["beta"], lamw,
                                               alpha=sl.get("alpha"), erase_b=sl.get("erase_b"),
                                               write_w=sl.get("write_w"), nthreads=th)
        what = f"fp64 token-by-token log-linear oracle ({nL} levels)"
    elif kind == "lambda":
        nL, nh = loglinear_levels(w.T), extra["nh"]
        d = r.standard_normal(sl["beta"].shape + (nL,))
        W1, W2, b = r.standard_normal((nL, nh)), r.standard_normal((nh, nL)), r.standard_normal(nL)
        run = lambda: oracle.loglinear_lambda(d, W1, W2, b)
        what, th = "fp64 level-weight MLP (numpy)", 1
    elif kind == "route":
        D = extra["D"]
        hh = r.standard_normal((batch_rows, T, D))
        P = r.standard_normal((D, w.H * w.dv))
        run = lambda: oracle.route(hh, sl["v"], P)
        what, th = "fp64 routing product (numpy matmul)", os.cpu_count()
    else:
        raise ValueError(kind)
    reps, dt = 0, 0.0
    while reps == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        run()
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": reps * batch_rows * T / dt, "unit": "tokens/s", "cores": th, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"{what} on batch rows 0..{batch_rows - 1} of {w.B}, tokens 0..{T - 1} of {w.T} "
                      f"(all {w.H} heads), {reps} pass{'es' if reps > 1 else ''} in {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: Gated DeltaNet B8 T4096 H8 d128)")
    ap.add_argument("--algo", default="auto", choices=["auto", "recurrent", "chunked"])
    ap.add_argument("--copies", type=int, default=3, help="input copies rotated across steps")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="batch rows timed on the CPU oracle (default: the whole workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle baseline until this much wall time has passed")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up steps, so the device clocks settle")
    ap.add_argument("--copy-probe-mib", type=int, default=1024,
                    help="size of the plain device copy timed beside the scan (0 = skip)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the scan shards over (batch, head) chains with no communication between them)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_linear_attention_chunked_amd as lam
    from gated_linear_attention_chunked_amd import inputs as I

    if not os.path.exists(lam.LIB_PATH):
        from gated_linear_attention_chunked_amd import build as _b

        _b.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    name = args.workload or I.METRIC_WORKLOAD
    decode = name in I.DECODE_WORKLOADS
    job = JOBS.get(name)
    if job is None and not decode and name not in I.WORKLOADS:
        print(f"bench.py: unknown workload {name}; known: "
              f"{sorted(I.WORKLOADS) + sorted(I.DECODE_WORKLOADS) + sorted(JOBS)}", file=sys.stderr)
        sys.exit(2)
    kind, extra = (job[0], job[2]) if job else ("decode" if decode else "forward", {})
    w = I.DECODE_WORKLOADS[name] if decode else I.WORKLOADS[job[1] if job else name]
    if extra.get("dtype"):  # a forward workload's shapes with another storage dtype
        w = w.replace(name=name, dtype=extra["dtype"])
    x = I.make_inputs(w)
    dev = torch.device("cuda:0")
    copies = [I.to_device(x, w.dtype, dev) for _ in range(max(1, args.copies))]
    jr = np.random.default_rng(w.seed + 29)   # the jobs' extra seeded inputs
    tdt = copies[0]["q"].dtype
    if decode:  # one token per stream: [N, 1, H, d] -> [N, H, d]
        copies = [{n: t[:, 0].contiguous() for n, t in g.items()} for g in copies]
        s0 = np.random.default_rng(w.seed).standard_normal((w.B, w.H, w.dv, w.dk)) * 0.1
        x["state_in"] = s0.astype(np.float32).astype(np.float64)
        if w.variant == "vla":  # fresh penalty, a loaded memory and denominator
            x["A_in"] = np.broadcast_to(np.eye(w.dk), (w.B, w.H, w.dk, w.dk)).copy()
            x["S_in"] = x.pop("state_in")
            x["n_in"] = np.full((w.B, w.H, w.dk), 0.8 / np.sqrt(w.dk))
    outs = []
    for g in copies:
        if kind == "backward":
            g["dout"] = torch.from_numpy(jr.standard_normal((w.B, w.T, w.H, w.dv)).astype(np.float32)).to(dev).to(tdt)
            outs.append(None)
        elif kind == "side":
            outs.append((torch.empty((w.B, w.T, w.H, w.dv), dtype=tdt, device=dev),
                         torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev),
                         torch.empty((w.B, w.T, w.H, w.dv), dtype=tdt, device=dev)))
        elif kind == "route":
            D, N = extra["D"], w.H * w.dv
            g["h"] = torch.from_numpy(jr.standard_normal((w.B, w.T, D)).astype(np.float32)).to(dev).to(tdt)
            g["P"] = torch.from_numpy((jr.standard_normal((D, N)) / np.sqrt(N)).astype(np.float32)).to(dev).to(tdt)
            outs.append(None)
        elif kind == "loglinear":
            nL = loglinear_levels(w.T)
            g["lam"] = torch.from_numpy(jr.uniform(0.5, 1.5, (w.B, w.T, w.H, nL)).astype(np.float32)).to(dev)
            outs.append((torch.empty((w.B, w.T, w.H, w.dv), dtype=tdt, device=dev),
                         torch.empty((w.B, w.H, nL, w.dv, w.dk), dtype=torch.float32, device=dev)))
        elif kind == "lambda":
            nL, nh = loglinear_levels(w.T), extra["nh"]
            g["d"] = torch.from_numpy(jr.standard_normal((w.B, w.T, w.H, nL)).astype(np.float32)).to(dev).to(tdt)
            g["W1"] = torch.from_numpy((jr.standard_normal((nL, nh)) * 0.3).astype(np.float32)).to(dev)
            g["W2"] = torch.from_numpy((jr.standard_normal((nh, nL)) * 0.3).astype(np.float32)).to(dev)
            g["b"] = torch.full((nL,), 0.54, dtype=torch.float32, device=dev)
            outs.append(torch.empty((w.B, w.T, w.H, nL), dtype=torch.float32, device=dev))
        elif decode and w.variant == "vla":
            f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
            outs.append((torch.empty((w.B, w.H, w.dv), dtype=g["q"].dtype, device=dev),
                         f32(x["A_in"]), f32(x["S_in"]), f32(x["n_in"])))
        elif decode:
            outs.append((torch.empty((w.B, w.H, w.dv), dtype=g["q"].dtype, device=dev),
                         torch.from_numpy(x["state_in"].astype(np.float32)).to(dev)))
        elif w.variant == "vla":
            outs.append((torch.empty((w.B, w.T, w.H, w.dv), dtype=g["q"].dtype, device=dev),
                         torch.empty((w.B, w.H, w.dk, w.dk), dtype=torch.float32, device=dev),
                         torch.empty((w.B, w.H, w.dk, w.dk), dtype=torch.float32, device=dev)))
        else:
            outs.append((torch.empty((w.B, w.T, w.H, w.dv), dtype=g["q"].dtype, device=dev),
                         torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)))
    stream = torch.cuda.current_stream()
    # one caller-owned workspace for every step: the steps run in order on
    # one stream, so each may reuse it
    if kind == "backward":
        nws = lam.backward_workspace_size(w.variant, w.dtype, w.B, w.T, w.H, w.dk, w.dv, algo=args.algo)
    elif decode or kind in ("route", "loglinear", "lambda"):
        nws = 0
    elif w.variant == "vla":
        nws = lam.vla_workspace_size(w.dtype, w.B, w.T, w.H, w.dk, algo=args.algo)
    else:
        nws = lam.workspace_size(w.variant, w.dtype, w.B, w.T, w.H, w.dk, w.dv, algo=args.algo)
    wsp = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None

    def step(i):
        g, o = copies[i % len(copies)], outs[i % len(outs)]
        if kind == "backward":
            lam.backward(w.variant, g["q"], g["k"], g["v"], g["beta"], g["dout"], alpha=g.get("alpha"),
                         erase_b=g.get("erase_b"), write_w=g.get("write_w"), algo=args.algo, workspace=wsp)
        elif kind == "side":
            lam.forward(w.variant, g["q"], g["k"], g["v"], g["beta"], alpha=g.get("alpha"), erase_b=g.get("erase_b"),
                        write_w=g.get("write_w"), algo=args.algo, out=o[0], state_out=o[1], workspace=wsp,
                        side="residual", side_out=o[2])
        elif kind == "route":
            lam.route(g["h"], g["v"], g["P"])
        elif kind == "loglinear":
            lam.loglinear_forward(w.variant, g["q"], g["k"], g["v"], g["beta"], g["lam"], alpha=g.get("alpha"),
                                  erase_b=g.get("erase_b"), write_w=g.get("write_w"), out=o[0], state_out=o[1])
        elif kind == "lambda":
            lam.loglinear_lambda(g["d"], g["W1"], g["W2"], g["b"], out=o)
        elif decode and w.variant == "vla":
            lam.vla_step_ratio(g["q"], g["k"], g["v"], g["p"], o[1], o[2], o[3], out=o[0])
        elif decode:
            lam.step(w.variant, g["q"], g["k"], g["v"], g["beta"], alpha=g.get("alpha"),
                     erase_b=g.get("erase_b"), write_w=g.get("write_w"), state=o[1], out=o[0])
        elif w.variant == "vla":
            lam.vla_forward(g["q"], g["k"], g["v"], g["p"], algo=args.algo, out=o[0], A_out=o[1],
                            S_out=o[2], workspace=wsp)
        else:
            lam.forward(w.variant, g["q"], g["k"], g["v"], g["beta"], alpha=g.get("alpha"),
                        erase_b=g.get("erase_b"), write_w=g.get("write_w"), algo=args.algo,
                        out=o[0], state_out=o[1], workspace=wsp)

    # Clock settling: the device raises its clocks only after some
    # milliseconds of sustained work, so before the W warm-up steps the step
    # runs untimed for --settle-s seconds (synchronising every few steps, so
    # the time is device time, not host submission time).
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(8):
            step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps between one pair of HIP events on the launch
    # stream (events between the steps would add their own gaps to the
    # wall time); mean launch = event time / K.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_launch_ms = e0.elapsed_time(e1) / args.steps
    # Spread of single calls, from a separate untimed pass with an event
    # pair around each call.
    nspread = min(args.steps, 20)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nspread)]
    for i in range(nspread):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = [a.elapsed_time(b) for a, b in ev]

    tokens = w.B * w.T
    value = tokens * args.steps / wall
    if kind == "backward":
        # the chunked adjoint (fp32 matrix cores) for every variant but Kimi Delta, unless told otherwise
        chunked_bwd = w.variant != "kda" and w.T > 0 and args.algo != "recurrent"
        ran = "backward_chunked" if chunked_bwd else "backward"
    elif kind in ("route", "loglinear", "lambda"):
        ran = kind
    elif decode:
        ran = "step"
    elif w.variant == "vla":
        # the VLA entry point runs the chunked schedule for any T > 0 unless told otherwise
        ran = args.algo if args.algo != "auto" else ("chunked" if w.T > 0 else "recurrent")
    else:
        ran = args.algo if args.algo != "auto" else lam.select_algo(w.variant, w.dtype, w.T, w.dk, w.dv)
    # arithmetic type: the recurrent schedules and fp32 storage compute in
    # fp32; the delta-rule chunked schedules on bf16 storage at dk 64 / 128
    # feed bf16 operands to the matrix cores (fp32 accumulate, fp32 state);
    # the VLA chunked schedule and the fp32 chunked delta form (every other
    # shape) use fp32 matrix-core products
    if ran == "route":
        arith_dtype = "bf16" if w.dtype == "bf16" else "f32"
    elif ran == "chunked" and w.variant != "vla" and bf16_matrix_schedule(w):
        arith_dtype = "bf16"
    else:
        arith_dtype = "f32"
    mean_launch_s = mean_launch_ms / 1e3
    if job and kind != "forward":
        abytes, aflops = job_counts(kind, w, extra)
    else:
        abytes = algorithmic_bytes(w, decode)
        aflops = algorithmic_flops(w)
    achieved_gbs = abytes / mean_launch_s / 1e9
    # the binding roofline: HBM bytes, or the algorithmic flops on the unit
    # the schedule computes them with (matrix cores for the chunked schedules,
    # the fp32 vector ALU for the recurrent ones), whichever takes longer
    if ran in ("chunked", "route", "backward_chunked"):
        cpeak, cbound = (MFMA_BF16_PEAK_TFS if arith_dtype == "bf16" else FP32_PEAK_TFS), "mfma"
    elif ran == "step":
        cpeak, cbound = FP32_PEAK_TFS, "alu"
    else:
        cpeak, cbound = FP32_PEAK_TFS, "alu"
    achieved_tfs = aflops / mean_launch_s / 1e12
    if aflops / (cpeak * 1e12) > abytes / (HBM_PEAK_GBS * 1e9):
        roofline = {"bound": cbound, "achieved": achieved_tfs, "peak": cpeak, "unit": "TFLOP/s",
                    "frac": achieved_tfs / cpeak}
    else:
        roofline = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved_gbs / HBM_PEAK_GBS}
    roofline.update({"traffic": measured_traffic(w, ran, name),
                "algorithmic_bytes_per_launch": abytes,
                "mean_launch_us": mean_launch_s * 1e6,
                "single_call_median_us": float(np.median(launch_ms)) * 1e3,
                "single_call_min_us": float(np.min(launch_ms)) * 1e3,
                "single_call_p90_us": float(np.percentile(launch_ms, 90)) * 1e3,
                "workspace_bytes": nws,
                "achieved_GBps": achieved_gbs,
                "algorithmic_tflops": achieved_tfs})

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(10)]
        for a, b in ce:
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
        torch.cuda.synchronize()
        cms = float(np.median([a.elapsed_time(b) for a, b in ce]))
        roofline["copy_probe"] = {"bytes": 2 * n * 4, "median_us": cms * 1e3,
                                  "GB/s": 2 * n * 4 / (cms / 1e3) / 1e9}
        del src, dst

    cpu = None
    if not args.no_cpu_baseline and job and kind != "forward":
        rows = min(w.B, args.cpu_rows or 1)
        cpu = cpu_baseline_job(kind, w, x, extra, rows, args.cpu_seconds)
    elif not args.no_cpu_baseline:
        rows = min(w.B, args.cpu_rows or w.B)
        cpu = cpu_baseline(w, x, rows, args.cpu_seconds)
        if decode:
            cpu["sample"] = cpu["sample"].replace("tokens)", "tokens, one decode step each from the same state)")

    job_metric = {
        "backward": f"{w.variant} backward tokens/s (all gradients), {name}",
        "side": f"{w.variant} fwd tokens/s with the per-token residual side output, {name}",
        "route": f"routing product h += s P^T tokens/s, {name}",
        "loglinear": f"{w.variant} log-linear readout tokens/s, {name}",
        "lambda": f"log-linear level-weight MLP tokens/s, {name}",
    }
    line = {
        "metric": "gated delta-rule fwd tokens/s, B8 T4096 H8 d128; % of HBM/MFMA roofline"
        if name == I.METRIC_WORKLOAD else (job_metric[kind] if kind in job_metric else
                                           (f"{w.variant} decode tokens/s (one token per stream per call"
                                            f"{', ratio read' if w.variant == 'vla' else ''}), {name}"
                                            if decode else f"{w.variant} fwd tokens/s, {name}")),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle_s,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arith_dtype,
        "data": "synthetic (seeded Gaussian activations, no dataset)",
        "config": dict({"workload": name, "variant": w.variant, "B": w.B, "T": w.T, "H": w.H,
                        "dk": w.dk, "dv": w.dv, "state": "fp32", "algo": ran, "storage": w.dtype,
                        "parallelism": "single GPU"}, **extra,
                       **({"levels": loglinear_levels(w.T)} if kind in ("loglinear", "lambda") else {})),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
