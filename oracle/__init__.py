"""Python binding of the fp64 CPU oracle (``oracle/lam_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path (the HIP
library and its binding) never imports this package, and this package never
imports the product path: the two share only the seeded input generator.

The oracle is plain C compiled with gcc (no HIP).  ``build()`` compiles two
copies of the same source: ``liblam_oracle.so`` computes in double, and
``liblam_oracle_f32.so`` computes in float (used only to measure how far
single precision can drift from double on a given input).

What the oracle computes, and from which passage of the pages, is stated in
the header comment of ``lam_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lam_oracle.c")
_LIBS = {
    "f64": os.path.join(_HERE, "liblam_oracle.so"),
    "f32": os.path.join(_HERE, "liblam_oracle_f32.so"),
}
# LAM_ORACLE_LIB / LAM_ORACLE_LIB_F32 name other builds of the same source
# (the sanitizer tests run the pins against an ASan/UBSan build); they are
# loaded as they are, never rebuilt.
_OVERRIDE = {"f64": os.environ.get("LAM_ORACLE_LIB"), "f32": os.environ.get("LAM_ORACLE_LIB_F32")}
_lock = threading.Lock()
_loaded: dict[str, ctypes.CDLL] = {}

DELTANET, GATED_DELTANET, KIMI_DELTA, GATED_DELTANET2 = 0, 1, 2, 3
VARIANTS = {
    "deltanet": DELTANET,
    "gdn": GATED_DELTANET,
    "kda": KIMI_DELTA,
    "gdn2": GATED_DELTANET2,
}


def build(force: bool = True) -> None:
    """Compile both oracle libraries with gcc + OpenMP (no fast-math, no FMA
    contraction, so every operation rounds exactly as written)."""
    for prec, out in _LIBS.items():
        if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
            continue
        real = "double" if prec == "f64" else "float"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               f"-DLAM_ORACLE_REAL={real}", _SRC, "-o", out + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)


def _lib(prec: str = "f64") -> ctypes.CDLL:
    with _lock:
        if prec not in _loaded:
            path = _OVERRIDE[prec] or _LIBS[prec]
            if not _OVERRIDE[prec] and (not os.path.exists(path) or
                                        os.path.getmtime(path) < os.path.getmtime(_SRC)):
                build(force=False)
            lib = ctypes.CDLL(path)
            dp = ctypes.c_void_p
            L = ctypes.c_long
            lib.oracle_delta_forward.argtypes = [ctypes.c_int, L, L, L, L, L] + [dp] * 10 + [ctypes.c_int, ctypes.c_int]
            lib.oracle_delta_forward.restype = ctypes.c_int
            lib.oracle_delta_forward_side.argtypes = ([ctypes.c_int, L, L, L, L, L] + [dp] * 10 +
                                                      [ctypes.c_int, dp, ctypes.c_int, ctypes.c_int])
            lib.oracle_delta_forward_side.restype = ctypes.c_int
            lib.oracle_vla_forward.argtypes = [L, L, L, L] + [dp] * 13 + [ctypes.c_int]
            lib.oracle_vla_forward.restype = ctypes.c_int
            lib.oracle_vla_forward_ratio.argtypes = [L, L, L, L] + [dp] * 11 + [ctypes.c_int]
            lib.oracle_vla_forward_ratio.restype = ctypes.c_int
            lib.oracle_delta_backward.argtypes = [ctypes.c_int, L, L, L, L, L] + [dp] * 18 + [ctypes.c_int]
            lib.oracle_delta_backward.restype = ctypes.c_int
            lib.oracle_loglinear_forward.argtypes = [ctypes.c_int, L, L, L, L, L, L, L] + [dp] * 11 + [ctypes.c_int]
            lib.oracle_loglinear_forward.restype = ctypes.c_int
            lib.oracle_real_bytes.restype = ctypes.c_int
            _loaded[prec] = lib
        return _loaded[prec]


def _in(x, shape=None):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


SIDES = {"residual": 1, "value": 2}


def delta_forward(variant, q, k, v, beta, alpha=None, erase_b=None, write_w=None,
                  state_in=None, drop_delta=False, nthreads=0, precision="f64", side=None):
    """Delta-rule family forward scan.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H]; alpha: [B,T,H] (gdn, gdn2)
    or [B,T,H,dk] (kda) or None (deltanet); erase_b: [B,T,H,dk] and write_w:
    [B,T,H,dv] (gdn2 only); state_in: [B,H,dv,dk] or None (zero memory).
    Returns (out [B,T,H,dv], state_out [B,H,dv,dk]) as float64 arrays, and
    with ``side`` = "residual" or "value" a third array [B,T,H,dv]: the
    per-token residual r (CLER) or write value (CLVR).
    ``drop_delta`` replaces the residual by the plain write target (test hook).
    """
    var = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    q = _in(q)
    B, T, H, dk = q.shape
    k = _in(k, (B, T, H, dk))
    v = _in(v)
    dv = v.shape[3]
    if v.shape[:3] != (B, T, H):
        raise ValueError("v shape")
    beta = _in(beta, (B, T, H))
    if var == DELTANET:
        alpha = None
    elif var == KIMI_DELTA:
        alpha = _in(alpha, (B, T, H, dk))
    else:
        alpha = _in(alpha, (B, T, H))
    if var == GATED_DELTANET2:
        erase_b = _in(erase_b, (B, T, H, dk))
        write_w = _in(write_w, (B, T, H, dv))
    else:
        erase_b = write_w = None
    state_in = _in(state_in, (B, H, dv, dk))
    out = np.zeros((B, T, H, dv), np.float64)
    state_out = np.zeros((B, H, dv, dk), np.float64)
    if side is None:
        rc = _lib(precision).oracle_delta_forward(
            var, B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase_b),
            _ptr(write_w), _ptr(beta), _ptr(state_in), _ptr(out), _ptr(state_out),
            int(bool(drop_delta)), int(nthreads))
        if rc != 0:
            raise RuntimeError("oracle_delta_forward failed")
        return out, state_out
    sd = np.zeros((B, T, H, dv), np.float64)
    rc = _lib(precision).oracle_delta_forward_side(
        var, B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase_b),
        _ptr(write_w), _ptr(beta), _ptr(state_in), _ptr(out), _ptr(state_out),
        int(bool(drop_delta)), _ptr(sd), SIDES[side], int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_delta_forward_side failed")
    return out, state_out, sd


def loglinear_levels(last_position: int) -> int:
    """Levels the Fenwick readout needs through absolute position
    ``last_position``: floor(log2(t)) + 2 for t >= 1 (1 for t = 0)."""
    return 1 if last_position < 1 else int(last_position).bit_length() + 1


def loglinear_forward(variant, q, k, v, beta, lam, alpha=None, erase_b=None, write_w=None,
                      state_in=None, t0=0, nthreads=0, precision="f64"):
    """Log-linear (Fenwick-tree) readout of the delta-rule family
    ("Technical summary: adaptive memory decay for log-linear attention",
    "Problem definition"); the readings are stated in lam_oracle.c.

    Inputs as ``delta_forward``; lam [B,T,H,nL] (the per-level weights);
    state_in [B,H,nL,dv,dk] or None (empty levels); t0 = absolute position of
    token 0.  Returns (out [B,T,H,dv], level states [B,H,nL,dv,dk])."""
    var = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    q = _in(q)
    B, T, H, dk = q.shape
    k = _in(k, (B, T, H, dk))
    v = _in(v)
    dv = v.shape[3]
    beta = _in(beta, (B, T, H))
    lam = _in(lam)
    nL = lam.shape[3]
    if lam.shape[:3] != (B, T, H):
        raise ValueError("lam shape")
    if var == DELTANET:
        alpha = None
    elif var == KIMI_DELTA:
        alpha = _in(alpha, (B, T, H, dk))
    else:
        alpha = _in(alpha, (B, T, H))
    if var == GATED_DELTANET2:
        erase_b = _in(erase_b, (B, T, H, dk))
        write_w = _in(write_w, (B, T, H, dv))
    else:
        erase_b = write_w = None
    state_in = _in(state_in, (B, H, nL, dv, dk))
    out = np.zeros((B, T, H, dv), np.float64)
    state_out = np.zeros((B, H, nL, dv, dk), np.float64)
    rc = _lib(precision).oracle_loglinear_forward(
        var, B, T, H, dk, dv, nL, int(t0), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase_b),
        _ptr(write_w), _ptr(beta), _ptr(lam), _ptr(state_in), _ptr(out), _ptr(state_out), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_loglinear_forward failed (too few levels?)")
    return out, state_out


def loglinear_lambda(d, W1, W2, b):
    """Adaptive level weights ("Technical summary: adaptive memory decay for
    log-linear attention", "Methodology", LambdaMLPSoftplus): two linear
    layers and a softplus, h = d W1, lambda = softplus(h W2 + b), for every
    token, head and level.  d: [..., nL]; W1: [nL, nh]; W2: [nh, nL];
    b: [nL].  softplus(x) = log(1 + e^x), evaluated as
    max(x, 0) + log1p(e^-|x|)."""
    d, W1, W2, b = (np.asarray(a, np.float64) for a in (d, W1, W2, b))
    x = (d @ W1) @ W2 + b
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def route(h, s, P):
    """Cross-layer routing epilogue ([LA-arch] "Technical details", the CLVR
    implementation): each token's signal s_t (all heads, [H*dv]) is mapped to
    the model width by P [D, H*dv] and added to the residual stream,
    h_t + P s_t.  h: [B,T,D]; s: [B,T,H,dv].  Returns float64 [B,T,D]."""
    h = _in(h)
    s = _in(s)
    P = _in(P)
    B, T, D = h.shape
    n = s.shape[2] * s.shape[3]
    if s.shape[:2] != (B, T) or P.shape != (D, n):
        raise ValueError("route: shapes")
    return h + s.reshape(B, T, n) @ P.T


def delta_backward(variant, q, k, v, beta, dout, alpha=None, erase_b=None, write_w=None,
                   state_in=None, dstate_out=None, nthreads=0, precision="f64"):
    """Gradients of sum(dout * out) + sum(dstate_out * state_out) for the
    forward of ``delta_forward`` on the same inputs (reverse-mode adjoint,
    token by token).  Returns a dict of float64 arrays: dq, dk, dv, dbeta,
    dalpha (gated variants), derase_b and dwrite_w (gdn2), dstate_in."""
    var = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    q = _in(q)
    B, T, H, dk = q.shape
    k = _in(k, (B, T, H, dk))
    v = _in(v)
    dv = v.shape[3]
    beta = _in(beta, (B, T, H))
    dout = _in(dout, (B, T, H, dv))
    if var == DELTANET:
        alpha = None
    elif var == KIMI_DELTA:
        alpha = _in(alpha, (B, T, H, dk))
    else:
        alpha = _in(alpha, (B, T, H))
    if var == GATED_DELTANET2:
        erase_b = _in(erase_b, (B, T, H, dk))
        write_w = _in(write_w, (B, T, H, dv))
    else:
        erase_b = write_w = None
    state_in = _in(state_in, (B, H, dv, dk))
    dstate_out = _in(dstate_out, (B, H, dv, dk))
    g = {"dq": np.zeros((B, T, H, dk)), "dk": np.zeros((B, T, H, dk)), "dv": np.zeros((B, T, H, dv)),
         "dbeta": np.zeros((B, T, H)), "dstate_in": np.zeros((B, H, dv, dk))}
    if alpha is not None:
        g["dalpha"] = np.zeros(alpha.shape)
    if var == GATED_DELTANET2:
        g["derase_b"] = np.zeros((B, T, H, dk))
        g["dwrite_w"] = np.zeros((B, T, H, dv))
    rc = _lib(precision).oracle_delta_backward(
        var, B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase_b), _ptr(write_w),
        _ptr(beta), _ptr(state_in), _ptr(dout), _ptr(dstate_out), _ptr(g["dq"]), _ptr(g["dk"]),
        _ptr(g["dv"]), _ptr(g.get("dalpha")), _ptr(g.get("derase_b")), _ptr(g.get("dwrite_w")),
        _ptr(g["dbeta"]), _ptr(g["dstate_in"]), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_delta_backward failed")
    return g


def vla_forward(q, k, v, p, A_in=None, S_in=None, diagnostics=False, nthreads=0,
                precision="f64"):
    """VLA forward scan on raw q, k (ELU+1 features and unit norms inside).

    q, k, v, p: [B,T,H,d]; A_in, S_in: [B,H,d,d] or None (identity, zero).
    Returns (out, A_out, S_out) and, with ``diagnostics``, a dict holding the
    per-token k-hat, q-hat, alpha-hat [B,T,H,d] and the Sherman-Morrison
    denominator 1 + p^T z [B,T,H].
    """
    q = _in(q)
    B, T, H, d = q.shape
    k, v, p = (_in(x, (B, T, H, d)) for x in (k, v, p))
    A_in = _in(A_in, (B, H, d, d))
    S_in = _in(S_in, (B, H, d, d))
    out = np.zeros((B, T, H, d), np.float64)
    A_out = np.zeros((B, H, d, d), np.float64)
    S_out = np.zeros((B, H, d, d), np.float64)
    diag = None
    if diagnostics:
        diag = {n: np.zeros((B, T, H, d), np.float64) for n in ("khat", "qhat", "ahat")}
        diag["den"] = np.zeros((B, T, H), np.float64)
    g = (lambda n: _ptr(diag[n])) if diag else (lambda n: None)
    rc = _lib(precision).oracle_vla_forward(
        B, T, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(p), _ptr(A_in), _ptr(S_in), _ptr(out),
        _ptr(A_out), _ptr(S_out), g("khat"), g("qhat"), g("ahat"), g("den"), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_vla_forward failed")
    if diagnostics:
        return out, A_out, S_out, diag
    return out, A_out, S_out


def vla_forward_ratio(q, k, v, p, A_in=None, S_in=None, n_in=None, nthreads=0, precision="f64"):
    """VLA forward scan with the output read as a ratio of two recurrences:
    the state S and a d-vector n that follows the same write rule with the
    value 1, y = (S q-hat) / (n . q-hat).

    q, k, v, p: [B,T,H,d]; A_in, S_in: [B,H,d,d] or None (identity, zero);
    n_in: [B,H,d] or None (zero).  Returns (out, A_out, S_out, n_out).
    """
    q = _in(q)
    B, T, H, d = q.shape
    k, v, p = (_in(x, (B, T, H, d)) for x in (k, v, p))
    A_in = _in(A_in, (B, H, d, d))
    S_in = _in(S_in, (B, H, d, d))
    n_in = _in(n_in, (B, H, d))
    out = np.zeros((B, T, H, d), np.float64)
    A_out = np.zeros((B, H, d, d), np.float64)
    S_out = np.zeros((B, H, d, d), np.float64)
    n_out = np.zeros((B, H, d), np.float64)
    rc = _lib(precision).oracle_vla_forward_ratio(
        B, T, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(p), _ptr(A_in), _ptr(S_in), _ptr(n_in), _ptr(out),
        _ptr(A_out), _ptr(S_out), _ptr(n_out), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_vla_forward_ratio failed")
    return out, A_out, S_out, n_out


def real_bytes(precision="f64") -> int:
    return _lib(precision).oracle_real_bytes()
