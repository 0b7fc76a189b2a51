"""MI355X-native (gfx950) recurrent-memory linear-attention forward scan.

Thin Python binding of ``liblam.so`` (C ABI in ``include/lam.h``): it checks
and marshals torch tensors into plain device pointers and sizes and calls the
library on torch's current HIP stream.  Every step of the scan runs in the
library's HIP kernels; there is no Python or CPU fallback -- if the library is
not built, or the device is not a GPU, the call raises.

Variants (see ``include/lam.h`` for the rules and their sources): DeltaNet
("deltanet"), Gated DeltaNet ("gdn"), Kimi Delta ("kda"), Gated DeltaNet-2
("gdn2"), and VLA (``vla_forward``).
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["forward", "vla_forward", "step", "vla_step", "select_algo", "workspace_size", "vla_workspace_size",
           "set_device_checks", "library", "LamError", "LamDeviceError", "VARIANTS", "ALGOS",
           "LIB_PATH"]

# LAM_LIBRARY names another build of the same library (the sanitizer tests
# load an ASan/UBSan build of the argument checks through it).
LIB_PATH = os.environ.get("LAM_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "liblam.so")
VARIANTS = {"deltanet": 0, "gdn": 1, "kda": 2, "gdn2": 3}
ALGOS = {"auto": 0, "recurrent": 1, "chunked": 2}
DTYPES = {"f32": 0, "bf16": 1}
STATUS = {0: "LAM_OK", 1: "LAM_ERR_INVALID_ARG", 2: "LAM_ERR_UNSUPPORTED", 3: "LAM_ERR_HIP",
          4: "LAM_ERR_SCRATCH_LIMIT"}

DEVICE_WAIT_TIMEOUT = 0x1   # bit of workspace word 0 (status block)

_lock = threading.Lock()
_lib = None
_device_checks = False


class LamError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} "
                         f"({library().lam_status_string(status).decode()})")


class LamDeviceError(RuntimeError):
    """A call's kernels reported a problem through the workspace status word."""

    def __init__(self, flags: int, what: str):
        self.flags = flags
        super().__init__(f"{what}: device status 0x{flags:x}"
                         + (" (a bounded in-kernel wait ran out)" if flags & DEVICE_WAIT_TIMEOUT else ""))


def set_device_checks(on: bool) -> None:
    """When on, every call synchronises the device after enqueueing its work
    and raises LamDeviceError if the workspace status word is not zero (for
    tests; it serialises the host with the device)."""
    global _device_checks
    _device_checks = bool(on)


def library() -> ctypes.CDLL:
    """The loaded C library (built in-tree by ``build.py``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built; run "
                                   "`python -m gated_linear_attention_chunked_amd.build`")
            lib = ctypes.CDLL(LIB_PATH)
            i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
            sz = ctypes.c_size_t
            lib.lam_forward.argtypes = [ci, ci, i64, i64, i64, i64, i64] + [vp] * 10 + [vp, sz, ci, vp]
            lib.lam_forward.restype = ci
            lib.lam_forward_noalloc.argtypes = [ci, ci, i64, i64, i64, i64, i64] + [vp] * 10 + [ci, vp]
            lib.lam_forward_noalloc.restype = ci
            lib.lam_forward_workspace_size.argtypes = [ci, ci, i64, i64, i64, i64, i64, ci,
                                                       ctypes.POINTER(sz)]
            lib.lam_forward_workspace_size.restype = ci
            lib.lam_vla_forward.argtypes = [ci, i64, i64, i64, i64] + [vp] * 9 + [vp, sz, ci, vp]
            lib.lam_vla_forward.restype = ci
            lib.lam_vla_workspace_size.argtypes = [ci, i64, i64, i64, i64, ci, ctypes.POINTER(sz)]
            lib.lam_vla_workspace_size.restype = ci
            lib.lam_forward_side.argtypes = [ci, ci, i64, i64, i64, i64, i64] + [vp] * 10 + [ci, vp, vp, sz, ci, vp]
            lib.lam_forward_side.restype = ci
            lib.lam_route.argtypes = [ci, i64, i64, i64, vp, vp, vp, vp]
            lib.lam_route.restype = ci
            lib.lam_loglinear_forward.argtypes = [ci, ci, i64, i64, i64, i64, i64, i64, i64] + [vp] * 11 + [vp]
            lib.lam_loglinear_forward.restype = ci
            lib.lam_loglinear_levels.argtypes = [i64]
            lib.lam_loglinear_levels.restype = i64
            lib.lam_loglinear_lambda.argtypes = [ci, i64, i64, i64] + [vp] * 5 + [vp]
            lib.lam_loglinear_lambda.restype = ci
            lib.lam_backward.argtypes = [ci, ci, i64, i64, i64, i64, i64] + [vp] * 18 + [ci, vp, sz, vp]
            lib.lam_backward.restype = ci
            lib.lam_backward_workspace_size.argtypes = [ci, ci, i64, i64, i64, i64, i64, ci, ctypes.POINTER(sz)]
            lib.lam_backward_workspace_size.restype = ci
            lib.lam_step.argtypes = [ci, ci, i64, i64, i64, i64] + [vp] * 9 + [vp]
            lib.lam_step.restype = ci
            lib.lam_vla_step.argtypes = [ci, i64, i64, i64] + [vp] * 7 + [vp]
            lib.lam_vla_step.restype = ci
            lib.lam_vla_forward_ratio.argtypes = [ci, i64, i64, i64, i64] + [vp] * 11 + [vp]
            lib.lam_vla_forward_ratio.restype = ci
            lib.lam_vla_step_ratio.argtypes = [ci, i64, i64, i64] + [vp] * 8 + [vp]
            lib.lam_vla_step_ratio.restype = ci
            lib.lam_status_string.argtypes = [ci]
            lib.lam_status_string.restype = ctypes.c_char_p
            lib.lam_abi_version.restype = ci
            lib.lam_select_algo.argtypes = [ci, ci, i64, i64, i64]
            lib.lam_select_algo.restype = ci
            _lib = lib
        return _lib


def select_algo(variant, dtype, T, dk, dv) -> str:
    """Name of the schedule ``algo="auto"`` runs for these arguments."""
    r = library().lam_select_algo(VARIANTS[variant], DTYPES[dtype], T, dk, dv)
    if r < 0:
        raise ValueError("arguments the library would reject")
    return {v: k for k, v in ALGOS.items()}[r]


def workspace_size(variant, dtype, B, T, H, dk, dv, algo="auto") -> int:
    """Bytes of workspace ``forward`` needs for these arguments (0: none)."""
    n = ctypes.c_size_t(0)
    rc = library().lam_forward_workspace_size(VARIANTS[variant], DTYPES[dtype], B, T, H, dk, dv,
                                              ALGOS[algo], ctypes.byref(n))
    if rc != 0:
        raise LamError(rc, "lam_forward_workspace_size")
    return int(n.value)


def backward_workspace_size(variant, dtype, B, T, H, dk, dv, algo="auto") -> int:
    """Bytes of workspace ``backward`` needs for these arguments."""
    n = ctypes.c_size_t(0)
    rc = library().lam_backward_workspace_size(VARIANTS[variant], DTYPES[dtype], B, T, H, dk, dv,
                                               ALGOS[algo], ctypes.byref(n))
    if rc != 0:
        raise LamError(rc, "lam_backward_workspace_size")
    return int(n.value)


def vla_workspace_size(dtype, B, T, H, d, algo="auto") -> int:
    """Bytes of workspace ``vla_forward`` needs for these arguments (0: none)."""
    n = ctypes.c_size_t(0)
    rc = library().lam_vla_workspace_size(DTYPES[dtype], B, T, H, d, ALGOS[algo], ctypes.byref(n))
    if rc != 0:
        raise LamError(rc, "lam_vla_workspace_size")
    return int(n.value)


def _workspace(nbytes, workspace, device, stream):
    """The caller's workspace (a uint8 tensor of at least nbytes on `device`),
    or a fresh one from torch's allocator, tied to `stream`."""
    import torch

    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.dtype != torch.uint8 or workspace.device != device or not workspace.is_contiguous():
            raise ValueError(f"workspace: expected a contiguous uint8 tensor on {device}")
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace: {workspace.numel()} bytes, the call needs {nbytes}")
        return workspace
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):  # allocated in `stream`'s order, reused only after it
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _after_call(ws, what):
    if not _device_checks:
        return
    import torch

    torch.cuda.synchronize()
    if ws is not None:
        flags = int(ws[:4].view(torch.int32).item())
        if flags:
            raise LamDeviceError(flags, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    import torch

    if t.dtype == torch.float32:
        return DTYPES["f32"]
    if t.dtype == torch.bfloat16:
        return DTYPES["bf16"]
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name}: must be on {device} (a GPU device)")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


SIDES = {None: 0, "residual": 1, "value": 2}


def forward(variant, q, k, v, beta, alpha=None, erase_b=None, write_w=None, state_in=None, *,
            algo="auto", out=None, state_out=None, with_state=True, stream=None, workspace=None,
            side=None, side_out=None):
    """Delta-rule family forward scan.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H]; alpha: [B,T,H]
    ("gdn", "gdn2") or [B,T,H,dk] ("kda"), unused for "deltanet"; erase_b
    [B,T,H,dk] and write_w [B,T,H,dv] for "gdn2".  All per-token tensors share
    one dtype (float32 or bfloat16) and device.  state_in: fp32 [B,H,dv,dk]
    or None (zero memory).  ``workspace``: optional uint8 device tensor of at
    least ``workspace_size(...)`` bytes (default: a fresh one from torch's
    caching allocator).  Returns (out [B,T,H,dv], state_out fp32 [B,H,dv,dk]
    or None), and with ``side`` = "residual" or "value" a third tensor
    [B,T,H,dv] in the streams' dtype: every token's delta-rule residual r
    (CLER) or write value (CLVR), written into ``side_out`` if given.
    """
    import torch

    var = VARIANTS[variant]
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dt, dev = q.dtype, q.device
    _check(q, "q", (B, T, H, dk), dt, dev)
    _check(k, "k", (B, T, H, dk), dt, dev)
    _check(v, "v", (B, T, H, dv), dt, dev)
    _check(beta, "beta", (B, T, H), dt, dev)
    if var == VARIANTS["kda"]:
        _check(alpha, "alpha", (B, T, H, dk), dt, dev)
    elif var != VARIANTS["deltanet"]:
        _check(alpha, "alpha", (B, T, H), dt, dev)
    else:
        alpha = None
    if var == VARIANTS["gdn2"]:
        _check(erase_b, "erase_b", (B, T, H, dk), dt, dev)
        _check(write_w, "write_w", (B, T, H, dv), dt, dev)
    else:
        erase_b = write_w = None
    _check(state_in, "state_in", (B, H, dv, dk), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check(out, "out", (B, T, H, dv), dt, dev)
    if with_state and state_out is None:
        state_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    _check(state_out, "state_out", (B, H, dv, dk), torch.float32, dev)
    nws = ctypes.c_size_t(0)
    rc = library().lam_forward_workspace_size(var, _dtype_code(q), B, T, H, dk, dv, ALGOS[algo],
                                              ctypes.byref(nws))
    if rc != 0:
        raise LamError(rc, "lam_forward_workspace_size")
    ws = _workspace(int(nws.value), workspace, dev, stream)
    if side is None:
        rc = library().lam_forward(var, _dtype_code(q), B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(alpha), _ptr(erase_b), _ptr(write_w), _ptr(beta),
                                   _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(ws),
                                   0 if ws is None else ws.numel(), ALGOS[algo], _stream(stream))
        if rc != 0:
            raise LamError(rc, "lam_forward")
        _after_call(ws, "lam_forward")
        return out, state_out
    if side_out is None:
        side_out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check(side_out, "side_out", (B, T, H, dv), dt, dev)
    rc = library().lam_forward_side(var, _dtype_code(q), B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(alpha), _ptr(erase_b), _ptr(write_w), _ptr(beta),
                                    _ptr(state_in), _ptr(out), _ptr(state_out), SIDES[side],
                                    _ptr(side_out), _ptr(ws), 0 if ws is None else ws.numel(),
                                    ALGOS[algo], _stream(stream))
    if rc != 0:
        raise LamError(rc, "lam_forward_side")
    _after_call(ws, "lam_forward_side")
    return out, state_out, side_out


def loglinear_levels(last_position: int) -> int:
    """Levels the log-linear readout needs through absolute position
    ``last_position`` (floor(log2) + 2; 1 for positions below 1)."""
    return int(library().lam_loglinear_levels(int(last_position)))


def loglinear_forward(variant, q, k, v, beta, lam, alpha=None, erase_b=None, write_w=None, state_in=None,
                      *, t0=0, out=None, state_out=None, with_state=True, stream=None):
    """Log-linear (Fenwick-tree) readout of the delta-rule family.

    Inputs as ``forward``; lam: fp32 [B,T,H,nL] level weights; state_in: fp32
    level memories [B,H,nL,dv,dk] or None; t0: absolute position of token 0.
    Returns (out [B,T,H,dv], level states [B,H,nL,dv,dk] or None).
    """
    import torch

    var = VARIANTS[variant]
    B, T, H, dk = q.shape
    dv = v.shape[3]
    nL = lam.shape[3]
    dt, dev = q.dtype, q.device
    _check(q, "q", (B, T, H, dk), dt, dev)
    _check(k, "k", (B, T, H, dk), dt, dev)
    _check(v, "v", (B, T, H, dv), dt, dev)
    _check(beta, "beta", (B, T, H), dt, dev)
    _check(lam, "lam", (B, T, H, nL), torch.float32, dev)
    if var == VARIANTS["kda"]:
        _check(alpha, "alpha", (B, T, H, dk), dt, dev)
    elif var != VARIANTS["deltanet"]:
        _check(alpha, "alpha", (B, T, H), dt, dev)
    else:
        alpha = None
    if var == VARIANTS["gdn2"]:
        _check(erase_b, "erase_b", (B, T, H, dk), dt, dev)
        _check(write_w, "write_w", (B, T, H, dv), dt, dev)
    else:
        erase_b = write_w = None
    _check(state_in, "state_in", (B, H, nL, dv, dk), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _check(out, "out", (B, T, H, dv), dt, dev)
    if with_state and state_out is None:
        state_out = torch.empty((B, H, nL, dv, dk), dtype=torch.float32, device=dev)
    _check(state_out, "state_out", (B, H, nL, dv, dk), torch.float32, dev)
    rc = library().lam_loglinear_forward(var, _dtype_code(q), B, T, H, dk, dv, nL, int(t0), _ptr(q), _ptr(k),
                                         _ptr(v), _ptr(alpha), _ptr(erase_b), _ptr(write_w), _ptr(beta),
                                         _ptr(lam), _ptr(state_in), _ptr(out), _ptr(state_out),
                                         _stream(stream))
    if rc != 0:
        raise LamError(rc, "lam_loglinear_forward")
    _after_call(None, "lam_loglinear_forward")
    return out, state_out


def loglinear_lambda(d, W1, W2, b, *, out=None, stream=None):
    """Adaptive level weights, softplus((d W1) W2 + b) per row.

    d: [..., nL] (float32 or bfloat16); W1 [nL, nh], W2 [nh, nL], b [nL]
    fp32.  Returns fp32 [..., nL]."""
    import torch

    nL = d.shape[-1]
    nh = W1.shape[1]
    dev = d.device
    if not d.is_contiguous():
        raise ValueError("d: must be contiguous")
    _check(W1, "W1", (nL, nh), torch.float32, dev)
    _check(W2, "W2", (nh, nL), torch.float32, dev)
    _check(b, "b", (nL,), torch.float32, dev)
    if out is None:
        out = torch.empty(d.shape, dtype=torch.float32, device=dev)
    _check(out, "out", tuple(d.shape), torch.float32, dev)
    M = d.numel() // nL
    rc = library().lam_loglinear_lambda(_dtype_code(d), M, nL, nh, _ptr(d), _ptr(W1), _ptr(W2), _ptr(b),
                                        _ptr(out), _stream(stream))
    if rc != 0:
        raise LamError(rc, "lam_loglinear_lambda")
    _after_call(None, "lam_loglinear_lambda")
    return out


def route(h, s, P, *, stream=None):
    """Routing epilogue, in place: h <- h + s P^T per token.

    h: [B,T,D] (the residual stream); s: [B,T,H,dv] (a routing signal from
    ``forward(..., side=...)``); P: [D, H*dv].  One dtype (float32 or
    bfloat16), one device.  Returns h.
    """
    B, T, D = h.shape
    N = s.shape[2] * s.shape[3]
    dt, dev = h.dtype, h.device
    _check(h, "h", (B, T, D), dt, dev)
    _check(s, "s", (B, T, s.shape[2], s.shape[3]), dt, dev)
    _check(P, "P", (D, N), dt, dev)
    rc = library().lam_route(_dtype_code(h), B * T, D, N, _ptr(s), _ptr(P), _ptr(h), _stream(stream))
    if rc != 0:
        raise LamError(rc, "lam_route")
    _after_call(None, "lam_route")
    return h


def backward(variant, q, k, v, beta, dout, alpha=None, erase_b=None, write_w=None, state_in=None,
             dstate_out=None, *, with_dstate_in=True, algo="auto", stream=None, workspace=None):
    """Gradients of sum(dout * out) + sum(dstate_out * state_out) for
    ``forward(variant, q, k, v, beta, alpha, erase_b, write_w, state_in)``.

    Inputs as ``forward``; dout [B,T,H,dv] in their dtype; dstate_out fp32
    [B,H,dv,dk] or None; algo "auto" / "recurrent" / "chunked" as
    ``forward``.  Returns a dict of fp32 tensors: dq, dk, dv, dbeta,
    dstate_in (None unless ``with_dstate_in``), and dalpha ("gdn", "gdn2",
    "kda"), derase_b and dwrite_w ("gdn2").
    """
    import torch

    var = VARIANTS[variant]
    B, T, H, dk = q.shape
    dv = v.shape[3]
    dt, dev = q.dtype, q.device
    _check(q, "q", (B, T, H, dk), dt, dev)
    _check(k, "k", (B, T, H, dk), dt, dev)
    _check(v, "v", (B, T, H, dv), dt, dev)
    _check(beta, "beta", (B, T, H), dt, dev)
    _check(dout, "dout", (B, T, H, dv), dt, dev)
    ashape = None
    if var == VARIANTS["kda"]:
        ashape = (B, T, H, dk)
    elif var != VARIANTS["deltanet"]:
        ashape = (B, T, H)
    if ashape is None:
        alpha = None
    else:
        _check(alpha, "alpha", ashape, dt, dev)
    if var == VARIANTS["gdn2"]:
        _check(erase_b, "erase_b", (B, T, H, dk), dt, dev)
        _check(write_w, "write_w", (B, T, H, dv), dt, dev)
    else:
        erase_b = write_w = None
    _check(state_in, "state_in", (B, H, dv, dk), torch.float32, dev)
    _check(dstate_out, "dstate_out", (B, H, dv, dk), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dq": torch.empty((B, T, H, dk), **f32), "dk": torch.empty((B, T, H, dk), **f32),
         "dv": torch.empty((B, T, H, dv), **f32), "dbeta": torch.empty((B, T, H), **f32),
         "dstate_in": torch.empty((B, H, dv, dk), **f32) if with_dstate_in else None}
    if ashape is not None:
        g["dalpha"] = torch.empty(ashape, **f32)
    if var == VARIANTS["gdn2"]:
        g["derase_b"] = torch.empty((B, T, H, dk), **f32)
        g["dwrite_w"] = torch.empty((B, T, H, dv), **f32)
    ws = _workspace(backward_workspace_size(variant, {torch.float32: "f32", torch.bfloat16: "bf16"}[dt],
                                            B, T, H, dk, dv, algo), workspace, dev, stream)
    rc = library().lam_backward(var, _dtype_code(q), B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(alpha), _ptr(erase_b), _ptr(write_w), _ptr(beta), _ptr(state_in),
                                _ptr(dout), _ptr(dstate_out), _ptr(g["dq"]), _ptr(g["dk"]),
                                _ptr(g["dv"]), _ptr(g.get("dalpha")), _ptr(g.get("derase_b")),
                                _ptr(g.get("dwrite_w")), _ptr(g["dbeta"]), _ptr(g["dstate_in"]),
                                ALGOS[algo], _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    if rc != 0:
        raise LamError(rc, "lam_backward")
    _after_call(ws, "lam_backward")
    return g


def vla_forward(q, k, v, p, A_in=None, S_in=None, *, algo="auto", out=None, A_out=None,
                S_out=None, with_state=True, stream=None, workspace=None):
    """VLA forward scan on raw q, k (ELU+1 features and unit norms inside).

    q, k, v, p: [B,T,H,d] (float32 or bfloat16); A_in, S_in: fp32 [B,H,d,d]
    or None (identity, zero).  Returns (out, A_out, S_out).
    """
    import torch

    B, T, H, d = q.shape
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("p", p)):
        _check(t, n, (B, T, H, d), dt, dev)
    for n, t in (("A_in", A_in), ("S_in", S_in)):
        _check(t, n, (B, H, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, d), dtype=dt, device=dev)
    _check(out, "out", (B, T, H, d), dt, dev)
    if with_state:
        if A_out is None:
            A_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
        if S_out is None:
            S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    for n, t in (("A_out", A_out), ("S_out", S_out)):
        _check(t, n, (B, H, d, d), torch.float32, dev)
    nws = ctypes.c_size_t(0)
    rc = library().lam_vla_workspace_size(_dtype_code(q), B, T, H, d, ALGOS[algo], ctypes.byref(nws))
    if rc != 0:
        raise LamError(rc, "lam_vla_workspace_size")
    ws = _workspace(int(nws.value), workspace, dev, stream)
    rc = library().lam_vla_forward(_dtype_code(q), B, T, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(p),
                                   _ptr(A_in), _ptr(S_in), _ptr(out), _ptr(A_out), _ptr(S_out),
                                   _ptr(ws), 0 if ws is None else ws.numel(), ALGOS[algo],
                                   _stream(stream))
    if rc != 0:
        raise LamError(rc, "lam_vla_forward")
    _after_call(ws, "lam_vla_forward")
    return out, A_out, S_out


def vla_forward_ratio(q, k, v, p, A_in=None, S_in=None, n_in=None, *, out=None, A_out=None, S_out=None,
                      n_out=None, stream=None):
    """VLA forward scan with the output read as a ratio of two recurrences:
    the denominator n [B,H,d] follows the write rule with the value 1 and
    y = (S qhat) / (n . qhat) (token-recurrent kernel).

    q, k, v, p: [B,T,H,d] (float32 or bfloat16); A_in, S_in: fp32 [B,H,d,d]
    or None (identity, zero); n_in: fp32 [B,H,d] or None (zero).  Returns
    (out, A_out, S_out, n_out).
    """
    import torch

    B, T, H, d = q.shape
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("p", p)):
        _check(t, n, (B, T, H, d), dt, dev)
    for n, t in (("A_in", A_in), ("S_in", S_in)):
        _check(t, n, (B, H, d, d), torch.float32, dev)
    _check(n_in, "n_in", (B, H, d), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, d), dtype=dt, device=dev)
    _check(out, "out", (B, T, H, d), dt, dev)
    if A_out is None:
        A_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    if S_out is None:
        S_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    if n_out is None:
        n_out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    for n, t in (("A_out", A_out), ("S_out", S_out)):
        _check(t, n, (B, H, d, d), torch.float32, dev)
    _check(n_out, "n_out", (B, H, d), torch.float32, dev)
    rc = library().lam_vla_forward_ratio(_dtype_code(q), B, T, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(p),
                                         _ptr(A_in), _ptr(S_in), _ptr(n_in), _ptr(out), _ptr(A_out),
                                         _ptr(S_out), _ptr(n_out), _stream(stream))
    if rc != 0:
        raise LamError(rc, "lam_vla_forward_ratio")
    _after_call(None, "lam_vla_forward_ratio")
    return out, A_out, S_out, n_out


def step(variant, q, k, v, beta, alpha=None, erase_b=None, write_w=None, *, state, out=None,
         stream=None):
    """One-token decode step for N streams, the memory updated in place.

    q, k: [N,H,dk]; v: [N,H,dv]; beta: [N,H]; alpha: [N,H] ("gdn", "gdn2") or
    [N,H,dk] ("kda"); erase_b [N,H,dk] and write_w [N,H,dv] for "gdn2";
    state: fp32 [N,H,dv,dk], read and overwritten.  Returns out [N,H,dv].
    """
    import torch

    var = VARIANTS[variant]
    N, H, dk = q.shape
    dv = v.shape[2]
    dt, dev = q.dtype, q.device
    _check(q, "q", (N, H, dk), dt, dev)
    _check(k, "k", (N, H, dk), dt, dev)
    _check(v, "v", (N, H, dv), dt, dev)
    _check(beta, "beta", (N, H), dt, dev)
    if var == VARIANTS["kda"]:
        _check(alpha, "alpha", (N, H, dk), dt, dev)
    elif var != VARIANTS["deltanet"]:
        _check(alpha, "alpha", (N, H), dt, dev)
    else:
        alpha = None
    if var == VARIANTS["gdn2"]:
        _check(erase_b, "erase_b", (N, H, dk), dt, dev)
        _check(write_w, "write_w", (N, H, dv), dt, dev)
    else:
        erase_b = write_w = None
    if state is None:
        raise ValueError("state: required (updated in place)")
    _check(state, "state", (N, H, dv, dk), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=dev)
    _check(out, "out", (N, H, dv), dt, dev)
    rc = library().lam_step(var, _dtype_code(q), N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                            _ptr(erase_b), _ptr(write_w), _ptr(beta), _ptr(state), _ptr(out),
                            _stream(stream))
    if rc != 0:
        raise LamError(rc, "lam_step")
    _after_call(None, "lam_step")
    return out


def vla_step(q, k, v, p, A, S, *, out=None, stream=None):
    """One-token VLA step for N streams: q, k, v, p [N,H,d]; A and S fp32
    [N,H,d,d] updated in place.  Returns out [N,H,d]."""
    import torch

    N, H, d = q.shape
    dt, dev = q.dtype, q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("p", p)):
        _check(t, n, (N, H, d), dt, dev)
    if A is None or S is None:
        raise ValueError("A and S: required (updated in place)")
    _check(A, "A", (N, H, d, d), torch.float32, dev)
    _check(S, "S", (N, H, d, d), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, d), dtype=dt, device=dev)
    _check(out, "out", (N, H, d), dt, dev)
    rc = library().lam_vla_step(_dtype_code(q), N, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(p), _ptr(A),
                                _ptr(S), _ptr(out), _stream(stream))
    if rc != 0:
        raise LamError(rc, "lam_vla_step")
    _after_call(None, "lam_vla_step")
    return out


def vla_step_ratio(q, k, v, p, A, S, n, *, out=None, stream=None):
    """One-token VLA step with the ratio read for N streams: q, k, v, p
    [N,H,d]; A, S fp32 [N,H,d,d] and the denominator n fp32 [N,H,d] updated in
    place.  Returns out [N,H,d]."""
    import torch

    N, H, d = q.shape
    dt, dev = q.dtype, q.device
    for nm, t in (("q", q), ("k", k), ("v", v), ("p", p)):
        _check(t, nm, (N, H, d), dt, dev)
    if A is None or S is None or n is None:
        raise ValueError("A, S and n: required (updated in place)")
    _check(A, "A", (N, H, d, d), torch.float32, dev)
    _check(S, "S", (N, H, d, d), torch.float32, dev)
    _check(n, "n", (N, H, d), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, d), dtype=dt, device=dev)
    _check(out, "out", (N, H, d), dt, dev)
    rc = library().lam_vla_step_ratio(_dtype_code(q), N, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(p), _ptr(A),
                                      _ptr(S), _ptr(n), _ptr(out), _stream(stream))
    if rc != 0:
        raise LamError(rc, "lam_vla_step_ratio")
    _after_call(None, "lam_vla_step_ratio")
    return out
