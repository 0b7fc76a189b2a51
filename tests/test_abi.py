"""C-ABI checks that need no GPU: the library loads, exports every function
include/lam.h declares, and rejects bad arguments before any HIP call.

Pointers passed here are never dereferenced: every call below must fail (or
return early for an empty batch) during host-side validation.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lam.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
FAKE = 0x7F0000000000  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    import gated_linear_attention_chunked_amd as lam

    if not os.path.exists(lam.LIB_PATH):
        from gated_linear_attention_chunked_amd import build

        build.build()
    return lam.library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lam_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"lam_forward", "lam_vla_forward", "lam_forward_workspace_size", "lam_vla_workspace_size",
            "lam_step", "lam_vla_step", "lam_forward_noalloc", "lam_status_string",
            "lam_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_select_algo(lib):
    assert lib.lam_select_algo(9, 1, 100, 128, 128) == -1
    assert lib.lam_select_algo(1, 1, 100, 48, 128) == -1
    assert lib.lam_select_algo(1, 1, 0, 128, 128) == 1          # empty: recurrent (state copy)
    for v in range(4):
        assert lib.lam_select_algo(v, 0, 256, 32, 32) in (1, 2)


def test_status_strings_and_version(lib):
    for s in range(5):
        assert lib.lam_status_string(s)
    assert lib.lam_status_string(99) == b"unknown status"
    assert lib.lam_abi_version() == 201


def _fwd(lib, variant=1, dtype=1, B=2, T=8, H=2, dk=64, dv=64, q=FAKE, k=FAKE + 0x10000000,
         v=FAKE + 0x20000000, alpha=FAKE + 0x30000000, eb=FAKE + 0x40000000,
         ww=FAKE + 0x50000000, beta=FAKE + 0x60000000, sin=None, out=FAKE + 0x70000000,
         sout=None, ws=None, ws_bytes=0, algo=0):
    return lib.lam_forward(variant, dtype, B, T, H, dk, dv, q, k, v, alpha, eb, ww, beta, sin,
                           out, sout, ws, ws_bytes, algo, None)


def test_forward_rejects_bad_enums(lib):
    assert _fwd(lib, variant=4) == INVALID
    assert _fwd(lib, variant=-1) == INVALID
    assert _fwd(lib, dtype=2) == INVALID
    assert _fwd(lib, algo=3) == INVALID


def test_forward_rejects_bad_sizes(lib):
    assert _fwd(lib, B=-1) == INVALID
    assert _fwd(lib, T=-1) == INVALID
    assert _fwd(lib, H=-1) == INVALID
    assert _fwd(lib, dk=0) == INVALID
    assert _fwd(lib, dv=-4) == INVALID
    assert _fwd(lib, dk=48) == UNSUPPORTED
    assert _fwd(lib, dv=256) == UNSUPPORTED
    assert _fwd(lib, B=1 << 40, T=1 << 30) == INVALID       # element count overflows
    assert _fwd(lib, B=1 << 20, H=1 << 10) == INVALID       # too many chains for one grid
    # token-row offsets inside a chunk are 32-bit: H * max(dk, dv) <= 2^24
    assert _fwd(lib, B=1, H=(1 << 17) + 1, dk=128, dv=64) == INVALID
    assert _fwd(lib, B=1, H=(1 << 17) + 1, dk=64, dv=128) == INVALID
    assert _vla(lib, B=1, H=(1 << 17) + 1, d=128) == INVALID


def test_forward_rejects_missing_pointers(lib):
    for name in ("q", "k", "v", "beta", "out"):
        assert _fwd(lib, **{name: None}) == INVALID, name
    assert _fwd(lib, alpha=None) == INVALID                    # gated variant
    assert _fwd(lib, variant=2, alpha=None) == INVALID         # Kimi Delta
    assert _fwd(lib, variant=3, eb=None) == INVALID            # Gated DeltaNet-2
    assert _fwd(lib, variant=3, ww=None) == INVALID


def test_forward_rejects_overlapping_output(lib):
    assert _fwd(lib, out=FAKE + 64) == INVALID                 # out inside q
    assert _fwd(lib, sin=FAKE + 0x70000000 + 128) == INVALID   # state_in inside out
    assert _fwd(lib, sin=FAKE + 0x80000000, sout=FAKE + 0x80000000 + 256) == INVALID


def test_forward_empty_batch_is_a_noop(lib):
    # no work, so no HIP call: returns before touching the device
    assert _fwd(lib, B=0, q=None, k=None, v=None, beta=None, out=None) == OK
    assert _fwd(lib, H=0, q=None, k=None, v=None, beta=None, out=None) == OK
    assert _fwd(lib, T=0, q=None, k=None, v=None, beta=None, out=None, sout=None) == OK


def _vla(lib, dtype=0, B=1, T=8, H=2, d=32, q=FAKE, k=FAKE + 0x10000000, v=FAKE + 0x20000000,
         p=FAKE + 0x30000000, Ain=None, Sin=None, out=FAKE + 0x40000000, Aout=None, Sout=None,
         ws=None, ws_bytes=0, algo=0):
    return lib.lam_vla_forward(dtype, B, T, H, d, q, k, v, p, Ain, Sin, out, Aout, Sout, ws,
                               ws_bytes, algo, None)


def test_vla_rejects_bad_arguments(lib):
    assert _vla(lib, dtype=5) == INVALID
    assert _vla(lib, algo=7) == INVALID
    assert _vla(lib, B=-1) == INVALID
    assert _vla(lib, d=40) == UNSUPPORTED
    assert _vla(lib, d=0) == INVALID
    for name in ("q", "k", "v", "p", "out"):
        assert _vla(lib, **{name: None}) == INVALID, name
    assert _vla(lib, out=FAKE + 4) == INVALID
    assert _vla(lib, Aout=FAKE + 0x50000000, Sout=FAKE + 0x50000000 + 64) == INVALID
    assert _vla(lib, B=0, q=None, k=None, v=None, p=None, out=None) == OK


def _vla_ratio(lib, dtype=0, B=2, T=8, H=2, d=32, q=FAKE, k=FAKE + 0x10000000, v=FAKE + 0x20000000,
               p=FAKE + 0x30000000, Ain=None, Sin=None, nin=None, out=FAKE + 0x40000000, Aout=None, Sout=None,
               nout=None):
    return lib.lam_vla_forward_ratio(dtype, B, T, H, d, q, k, v, p, Ain, Sin, nin, out, Aout, Sout, nout, None)


def test_vla_ratio_rejects_bad_arguments(lib):
    """The ratio read's entry points: the same shape checks as the plain VLA
    scan, plus the denominator state's buffers (none of these reaches HIP)."""
    assert _vla_ratio(lib, dtype=5) == INVALID
    assert _vla_ratio(lib, B=-1) == INVALID
    assert _vla_ratio(lib, d=40) == UNSUPPORTED
    assert _vla_ratio(lib, d=0) == INVALID
    for name in ("q", "k", "v", "p", "out"):
        assert _vla_ratio(lib, **{name: None}) == INVALID, name
    assert _vla_ratio(lib, out=FAKE + 4) == INVALID                              # out over q
    assert _vla_ratio(lib, nout=FAKE + 0x40000000 + 64) == INVALID               # n_out inside out
    S = FAKE + 0x60000000
    assert _vla_ratio(lib, Sin=S, nout=S + 64) == INVALID                        # n_out over S_in
    assert _vla_ratio(lib, nin=S, Aout=S) == INVALID                             # A_out over n_in
    X = FAKE + 0x70000000
    assert _vla_ratio(lib, Aout=X, nout=X + 64) == INVALID                       # two outputs overlap
    assert _vla_ratio(lib, B=0, q=None, k=None, v=None, p=None, out=None) == OK
    A, S2, n, o = FAKE + 0x80000000, FAKE + 0x90000000, FAKE + 0xA0000000, FAKE + 0xB0000000
    assert lib.lam_vla_step_ratio(0, 2, 2, 32, FAKE, FAKE + 0x10000000, FAKE + 0x20000000, FAKE + 0x30000000,
                                  A, S2, None, o, None) == INVALID              # n is updated in place
    assert lib.lam_vla_step_ratio(0, 2, 2, 40, FAKE, FAKE, FAKE, FAKE, A, S2, n, o, None) == UNSUPPORTED
    assert lib.lam_vla_step_ratio(3, 2, 2, 32, FAKE, FAKE, FAKE, FAKE, A, S2, n, o, None) == INVALID


def test_binding_fails_loudly_without_gpu_tensors():
    import torch

    import gated_linear_attention_chunked_amd as lam

    q = torch.zeros(1, 4, 1, 32)
    with pytest.raises(ValueError):
        lam.forward("deltanet", q, q, q, torch.zeros(1, 4, 1))


def _ws_size(lib, variant=1, dtype=1, B=2, T=8, H=2, dk=64, dv=64, algo=0):
    n = ctypes.c_size_t(12345)
    rc = lib.lam_forward_workspace_size(variant, dtype, B, T, H, dk, dv, algo, ctypes.byref(n))
    return rc, n.value


def test_workspace_size_query(lib):
    # chunked delta schedule: 256-byte status block + 5,888 B per (b, h, 64-token chunk)
    assert _ws_size(lib, 1, 1, 8, 4096, 8, 128, 128) == (OK, 256 + 8 * 8 * 64 * 6144)
    assert _ws_size(lib, 3, 1, 8, 4096, 8, 128, 128) == (OK, 256 + 8 * 8 * 64 * 6144)
    assert _ws_size(lib, 0, 1, 1, 65, 1, 128, 128) == (OK, 256 + 2 * 6144)   # ragged: whole chunks
    # Kimi Delta: 14,848 B per 16-token sub-chunk at dk = 128, counted in pairs
    assert _ws_size(lib, 2, 1, 2, 32768, 8, 128, 128) == (OK, 256 + 2 * 8 * 2048 * 14848)
    assert _ws_size(lib, 2, 1, 1, 17, 1, 128, 128) == (OK, 256 + 2 * 14848)
    # fp32 chunked form (any storage at dk 32 / 96, fp32 at every size): one
    # record per (b, h, 16-token chunk), 26,640 B at dk = 128, 8,208 B at dk = 32
    assert _ws_size(lib, 1, 0, 8, 4096, 8, 128, 128) == (OK, 256 + 8 * 8 * 256 * 26640)
    assert _ws_size(lib, 0, 1, 1, 17, 2, 32, 64) == (OK, 256 + 2 * 2 * 8208)
    # schedules with no workspace
    assert _ws_size(lib, 1, 1, 8, 4096, 8, 128, 128, algo=1) == (OK, 0)      # recurrent asked for
    assert _ws_size(lib, 1, 1, 8, 0, 8, 128, 128) == (OK, 0)                 # T = 0: state copy
    assert _ws_size(lib, 1, 1, 0, 100, 8, 128, 128) == (OK, 0)               # empty batch
    # the statuses lam_forward would return
    assert _ws_size(lib, 2, 0, 8, 64, 8, 128, 128, algo=2)[0] == UNSUPPORTED  # Kimi Delta fp32 chunked
    assert _ws_size(lib, 9)[0] == INVALID
    assert _ws_size(lib, dk=48)[0] == UNSUPPORTED
    assert _ws_size(lib, B=-1)[0] == INVALID
    assert lib.lam_forward_workspace_size(1, 1, 1, 8, 1, 64, 64, 0, None) == INVALID
    n = ctypes.c_size_t(7)
    assert lib.lam_vla_workspace_size(0, 4, 4096, 8, 32, 0, ctypes.byref(n)) == OK
    assert lib.lam_vla_workspace_size(0, 4, 4096, 8, 40, 0, ctypes.byref(n)) == UNSUPPORTED


WS = FAKE + 0x90000000  # 256-byte aligned, clear of every other fake argument


def test_forward_rejects_bad_workspace(lib):
    rc, need = _ws_size(lib)
    assert rc == OK and need > 0
    assert _fwd(lib) == INVALID                                     # none given
    assert _fwd(lib, ws=WS, ws_bytes=need - 1) == INVALID           # too small
    assert _fwd(lib, ws=WS + 64, ws_bytes=need) == INVALID          # not 256-byte aligned
    assert _fwd(lib, ws=FAKE, ws_bytes=need) == INVALID             # overlaps q
    assert _fwd(lib, ws=FAKE + 0x70000000, ws_bytes=need) == INVALID  # overlaps out
    assert _fwd(lib, sout=WS + 1024, ws=WS, ws_bytes=need) == INVALID  # overlaps state_out


def _step(lib, variant=1, dtype=1, N=4, H=2, dk=64, dv=64, q=FAKE, k=FAKE + 0x10000000,
          v=FAKE + 0x20000000, alpha=FAKE + 0x30000000, eb=FAKE + 0x40000000, ww=FAKE + 0x50000000,
          beta=FAKE + 0x60000000, state=FAKE + 0x80000000, out=FAKE + 0x70000000):
    return lib.lam_step(variant, dtype, N, H, dk, dv, q, k, v, alpha, eb, ww, beta, state, out, None)


def test_step_rejects_bad_arguments(lib):
    assert _step(lib, variant=7) == INVALID
    assert _step(lib, dtype=3) == INVALID
    assert _step(lib, N=-1) == INVALID
    assert _step(lib, dk=48) == UNSUPPORTED
    assert _step(lib, state=None) == INVALID                   # the state is updated in place
    for name in ("q", "k", "v", "beta", "out"):
        assert _step(lib, **{name: None}) == INVALID, name
    assert _step(lib, alpha=None) == INVALID
    assert _step(lib, variant=3, eb=None) == INVALID
    assert _step(lib, out=FAKE + 0x80000000 + 64) == INVALID   # out inside the state
    assert _step(lib, N=0, q=None, k=None, v=None, beta=None, out=None, state=None) == OK
    assert lib.lam_vla_step(0, 2, 2, 32, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == INVALID
    assert lib.lam_vla_step(0, 2, 2, 40, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == UNSUPPORTED


def _bwd(lib, variant=1, dtype=1, B=2, T=8, H=2, dk=64, dv=64, ws=None, ws_bytes=0, algo=1, **kw):
    p = dict(q=FAKE, k=FAKE + 0x10000000, v=FAKE + 0x20000000, alpha=FAKE + 0x30000000,
             eb=FAKE + 0x40000000, ww=FAKE + 0x50000000, beta=FAKE + 0x60000000, sin=None,
             dout=FAKE + 0x70000000, dsout=None, gq=FAKE + 0x100000000, gk=FAKE + 0x110000000,
             gv=FAKE + 0x120000000, dalpha=FAKE + 0x130000000, deb=FAKE + 0x140000000,
             dww=FAKE + 0x150000000, dbeta=FAKE + 0x160000000, dsin=FAKE + 0x170000000)
    p.update(kw)
    return lib.lam_backward(variant, dtype, B, T, H, dk, dv, p["q"], p["k"], p["v"], p["alpha"], p["eb"],
                            p["ww"], p["beta"], p["sin"], p["dout"], p["dsout"], p["gq"], p["gk"], p["gv"],
                            p["dalpha"], p["deb"], p["dww"], p["dbeta"], p["dsin"], algo, ws, ws_bytes, None)


def test_backward_rejects_bad_arguments(lib):
    n = ctypes.c_size_t(0)
    assert lib.lam_backward_workspace_size(1, 1, 2, 8, 2, 64, 64, 1, ctypes.byref(n)) == OK
    need = n.value
    # recurrent: the forward state every 16 tokens plus the 256-byte status block
    assert need == 256 + 2 * 2 * 1 * 64 * 64 * 4
    assert lib.lam_backward_workspace_size(1, 1, 2, 0, 2, 64, 64, 1, ctypes.byref(n)) == OK and n.value == 256
    assert lib.lam_backward_workspace_size(1, 1, 2, 0, 2, 64, 64, 0, ctypes.byref(n)) == OK and n.value == 256
    # chunked (what auto picks): per (b, h, 16-token chunk) a 14,352-byte forward
    # record and a 13,328-byte adjoint record at dk = 64, the chunk's start
    # state and state cotangent (64 x 64 fp32 each), then U and dX (B*T*H*dv
    # fp32 each); every region starts on a 256-byte boundary
    up = lambda x: (x + 255) // 256 * 256
    chunked = up(up(256 + 4 * 14352) + 4 * 13328) + 2 * 4 * 64 * 64 * 4 + 2 * 2 * 8 * 2 * 64 * 4
    for algo in (0, 2):
        assert lib.lam_backward_workspace_size(1, 1, 2, 8, 2, 64, 64, algo, ctypes.byref(n)) == OK
        assert n.value == chunked, (algo, n.value, chunked)
    assert lib.lam_backward_workspace_size(2, 1, 2, 8, 2, 64, 64, 2, ctypes.byref(n)) == UNSUPPORTED  # Kimi Delta
    assert lib.lam_backward_workspace_size(2, 1, 2, 8, 2, 64, 64, 0, ctypes.byref(n)) == OK           # recurrent
    assert lib.lam_backward_workspace_size(1, 1, 2, 8, 2, 64, 64, 3, ctypes.byref(n)) == INVALID      # algo
    assert lib.lam_backward_workspace_size(1, 1, 2, 8, 2, 48, 64, 1, ctypes.byref(n)) == UNSUPPORTED
    assert lib.lam_backward_workspace_size(9, 1, 2, 8, 2, 64, 64, 1, ctypes.byref(n)) == INVALID
    assert _bwd(lib, algo=0, ws=FAKE + 0x200000000, ws_bytes=chunked - 1) == INVALID   # too small for chunked
    WS = FAKE + 0x200000000
    assert _bwd(lib) == INVALID                                       # no workspace
    assert _bwd(lib, ws=WS, ws_bytes=need - 1) == INVALID             # too small
    for name in ("q", "k", "v", "beta", "dout", "gq", "gk", "gv", "dbeta", "alpha", "dalpha"):
        assert _bwd(lib, ws=WS, ws_bytes=need, **{name: None}) == INVALID, name
    assert _bwd(lib, variant=0, alpha=None, dalpha=None, eb=None, dww=None, ws=WS, ws_bytes=need,
                q=None) == INVALID
    for name in ("eb", "ww", "deb", "dww"):
        assert _bwd(lib, variant=3, ws=WS, ws_bytes=need, **{name: None}) == INVALID, name
    # a gradient inside an input, inside another gradient, or inside the workspace
    assert _bwd(lib, gq=FAKE + 64, ws=WS, ws_bytes=need) == INVALID
    assert _bwd(lib, gk=FAKE + 0x100000000 + 64, ws=WS, ws_bytes=need) == INVALID
    assert _bwd(lib, dsin=WS + 512, ws=WS, ws_bytes=need) == INVALID
    assert _bwd(lib, B=0, ws=None) == OK


def test_forward_side_rejects_bad_arguments(lib):
    def fs(side=1, sout=FAKE + 0x90000000, **kw):
        p = dict(variant=1, dtype=1, B=2, T=8, H=2, dk=64, dv=64)
        p.update(kw)
        return lib.lam_forward_side(p["variant"], p["dtype"], p["B"], p["T"], p["H"], p["dk"], p["dv"], FAKE,
                                    FAKE + 0x10000000, FAKE + 0x20000000, FAKE + 0x30000000, None, None,
                                    FAKE + 0x60000000, None, FAKE + 0x70000000, None, side, sout, None, 0, 1,
                                    None)
    assert fs(side=3) == INVALID
    assert fs(side=-1) == INVALID
    assert fs(sout=None) == INVALID                 # a side output asked for, nowhere to put it
    assert fs(sout=FAKE + 0x70000000 + 2) == INVALID  # inside out
    assert fs(sout=FAKE + 16) == INVALID            # inside q
    assert fs(B=0) == OK


def test_route_rejects_bad_arguments(lib):
    S, P, Hh = FAKE, FAKE + 0x10000000, FAKE + 0x20000000
    assert lib.lam_route(2, 64, 128, 256, S, P, Hh, None) == INVALID   # dtype
    assert lib.lam_route(1, -1, 128, 256, S, P, Hh, None) == INVALID
    assert lib.lam_route(1, 64, 120, 256, S, P, Hh, None) == UNSUPPORTED  # D % 16
    assert lib.lam_route(1, 64, 128, 48, S, P, Hh, None) == UNSUPPORTED   # N % 32
    assert lib.lam_route(1, 64, 128, 256, None, P, Hh, None) == INVALID
    assert lib.lam_route(1, 64, 128, 256, S + 8, P, Hh, None) == INVALID  # not 16-byte aligned
    assert lib.lam_route(1, 64, 128, 256, S, P, S + 64, None) == INVALID  # h inside s
    assert lib.lam_route(1, 0, 128, 256, None, None, None, None) == OK    # no tokens


def test_loglinear_rejects_bad_arguments(lib):
    lib.lam_loglinear_levels.restype = ctypes.c_int64
    lib.lam_loglinear_levels.argtypes = [ctypes.c_int64]
    assert [lib.lam_loglinear_levels(t) for t in (0, 1, 2, 3, 4, 4095, 4096)] == [1, 2, 3, 3, 4, 13, 14]

    def ll(variant=1, dtype=1, B=2, T=8, H=2, dk=64, dv=64, nL=4, t0=0, lam=FAKE + 0x80000000, out=FAKE + 0x70000000,
           sin=None, sout=None, alpha=FAKE + 0x30000000):
        return lib.lam_loglinear_forward(variant, dtype, B, T, H, dk, dv, nL, t0, FAKE, FAKE + 0x10000000,
                                         FAKE + 0x20000000, alpha, None, None, FAKE + 0x60000000, lam, sin, out,
                                         sout, None)
    assert ll(nL=3) == INVALID            # positions 0..7 need 4 levels
    assert ll(t0=8, nL=4) == INVALID      # positions 8..15 need 5
    assert ll(nL=25) == UNSUPPORTED       # more levels than the kernel holds
    assert ll(t0=(1 << 23)) == UNSUPPORTED
    assert ll(t0=-1) == INVALID
    assert ll(lam=None) == INVALID
    assert ll(alpha=None) == INVALID
    assert ll(out=FAKE + 8) == INVALID    # out inside q
    assert ll(sout=FAKE + 0x80000000) == INVALID  # level states inside lam
    assert ll(B=0) == OK
    assert lib.lam_loglinear_lambda(1, 10, 25, 8, FAKE, FAKE, FAKE, FAKE, FAKE + 0x10000000, None) == UNSUPPORTED
    assert lib.lam_loglinear_lambda(1, 10, 4, 65, FAKE, FAKE, FAKE, FAKE, FAKE + 0x10000000, None) == UNSUPPORTED
    assert lib.lam_loglinear_lambda(1, 10, 4, 8, FAKE, FAKE, FAKE, FAKE, FAKE + 8, None) == INVALID  # over d
    assert lib.lam_loglinear_lambda(1, 0, 4, 8, None, None, None, None, None, None) == OK
