"""Seeded synthetic inputs for the recurrent-memory forward scan.

This module is the one piece shared by the HIP path's tests/benchmark and the
CPU oracle's tests.  It holds none of the scan's arithmetic: it only draws
Gaussian activations and applies the input recipe (per-token L2 normalisation
of delta-rule queries and keys, gate squashing), then rounds to the storage
dtype.  The scan itself -- decays, residuals, writes, reads, VLA's feature
maps and Sherman-Morrison downdates -- lives in the HIP kernels and,
independently, in the oracle.

Recipe (the pages run 350M-class layers, hidden 1024 = 8 heads x 128, at
sequence 4k-32k in bf16, on FineWeb-Edu; these Gaussian draws stand in for
those activations -- no dataset is read):
  * generator numpy PCG64(seed); each stream drawn with
    ``standard_normal(shape, float64)`` in the fixed order
    q, k, v, gate-x, beta-x, erase-x, write-x, p (streams a variant does not
    use are not drawn);
  * delta-rule family: q, k L2-normalised per token; v as drawn;
    beta = sigmoid(x_beta); decay alpha = exp(-softplus(x)) = sigmoid(-x),
    x ~ N(gate_mu, 1) (per token-head, or per key channel for Kimi Delta);
    Gated DeltaNet-2 erase b = sigmoid(x_b) per key channel, write
    w = sigmoid(x_w) per value channel;
  * VLA: raw q, k, v ~ N(0, 1) (the feature map is part of the scan);
    penalty direction p ~ N(0, 1/d) (1/d read as the variance);
  * values are computed in float64, rounded to float32 (round to nearest
    even), and for bf16 storage rounded again to bf16 (round to nearest even).
    The returned float64 arrays hold exactly the rounded values the device
    receives, so input quantisation is not part of any comparison.
"""
from __future__ import annotations

import dataclasses

import numpy as np

DELTA_VARIANTS = ("deltanet", "gdn", "kda", "gdn2")
ALL_VARIANTS = DELTA_VARIANTS + ("vla",)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    variant: str          # deltanet | gdn | kda | gdn2 | vla
    dtype: str            # f32 | bf16 (storage dtype of every token stream and of out)
    B: int
    T: int
    H: int
    dk: int
    dv: int
    seed: int
    gate_mu: float = 0.0  # mean of the decay pre-activation x (alpha = sigmoid(-x))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five workloads the method is exercised on, named by what they are.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("deltanet_f32_B1_T256_H2_d32", "deltanet", "f32", 1, 256, 2, 32, 32, seed=1),
        Workload("gdn_bf16_B8_T4096_H8_d128", "gdn", "bf16", 8, 4096, 8, 128, 128, seed=2, gate_mu=2.0),
        Workload("kda_bf16_B2_T32768_H8_d128", "kda", "bf16", 2, 32768, 8, 128, 128, seed=3, gate_mu=3.0),
        Workload("gdn2_bf16_B8_T4096_H8_d128", "gdn2", "bf16", 8, 4096, 8, 128, 128, seed=4, gate_mu=2.0),
        Workload("vla_f32_B4_T4096_H8_d32", "vla", "f32", 4, 4096, 8, 32, 32, seed=5),
        Workload("vla_f32_B4_T4096_H8_d96", "vla", "f32", 4, 4096, 8, 96, 96, seed=6),
    )
}
# The throughput workload: Gated DeltaNet, bf16 streams, fp32 state.
METRIC_WORKLOAD = "gdn_bf16_B8_T4096_H8_d128"

# Decode workloads: one token for each of B streams per call, the fp32 state
# (B x H x dv x dk) resident in HBM and updated in place.
DECODE_WORKLOADS = {
    w.name: w
    for w in (
        Workload("gdn_step_bf16_N256_H8_d128", "gdn", "bf16", 256, 1, 8, 128, 128, seed=9, gate_mu=2.0),
        # VLA decode with the ratio read: A, S and the denominator n carried per stream
        Workload("vla_ratio_step_f32_N256_H8_d96", "vla", "f32", 256, 1, 8, 96, 96, seed=10),
    )
}


def round_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32, round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32 values.
    Inputs here are finite; NaN/Inf are not produced by the recipe."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def _sigmoid(x):
    return np.exp(-np.logaddexp(0.0, -x))


def _l2n(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _store(x64, dtype):
    x32 = round_f32(x64)
    if dtype == "bf16":
        x32 = round_bf16(x32)
    return x32.astype(np.float64)


def make_inputs(w: Workload) -> dict:
    """Host inputs of workload ``w`` as float64 arrays holding the stored values.

    Keys: q, k, v and, by variant, beta, alpha, erase_b, write_w, p.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    n = lambda shape: rng.standard_normal(shape, dtype=np.float64)
    out = {}
    if w.variant == "vla":
        if dk != dv:
            raise ValueError("VLA needs dk == dv")
        q, k, v = n((B, T, H, dk)), n((B, T, H, dk)), n((B, T, H, dv))
        p = n((B, T, H, dk)) / np.sqrt(dk)
        for name, x in (("q", q), ("k", k), ("v", v), ("p", p)):
            out[name] = _store(x, w.dtype)
        return out
    q = _l2n(n((B, T, H, dk)))
    k = _l2n(n((B, T, H, dk)))
    v = n((B, T, H, dv))
    out["q"], out["k"], out["v"] = (_store(x, w.dtype) for x in (q, k, v))
    del q, k, v
    if w.variant in ("gdn", "gdn2"):
        out["alpha"] = _store(_sigmoid(-(n((B, T, H)) + w.gate_mu)), w.dtype)
    elif w.variant == "kda":
        out["alpha"] = _store(_sigmoid(-(n((B, T, H, dk)) + w.gate_mu)), w.dtype)
    out["beta"] = _store(_sigmoid(n((B, T, H))), w.dtype)
    if w.variant == "gdn2":
        out["erase_b"] = _store(_sigmoid(n((B, T, H, dk))), w.dtype)
        out["write_w"] = _store(_sigmoid(n((B, T, H, dv))), w.dtype)
    return out


def make_cotangents(w: Workload, seed: int) -> tuple:
    """Seeded adjoints for a backward pass of workload ``w``: dout
    [B,T,H,dv] (standard normal, stored in w's dtype) and dstate_out fp32
    [B,H,dv,dk] (standard normal), as float64 arrays of the stored values."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dout = _store(rng.standard_normal((w.B, w.T, w.H, w.dv)), w.dtype)
    dstate = round_f32(rng.standard_normal((w.B, w.H, w.dv, w.dk))).astype(np.float64)
    return dout, dstate


def to_device(inputs: dict, dtype: str, device="cuda"):
    """Copy host inputs to device tensors in the storage dtype (exact: the
    host values are already representable)."""
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device=device).to(tdt)
            for k, v in inputs.items()}
