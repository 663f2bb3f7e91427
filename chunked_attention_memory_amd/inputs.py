"""Seeded synthetic inputs for the SCA + AWM forward.

This module only draws and rounds numbers; it holds none of the forward's
arithmetic. Both the GPU path's tests/bench and the CPU oracle consume what it
returns.

Recipe (per (batch, head) slab, independently regenerable):

* Z': rows of iid N(0, 1) in float64, each divided by its L2 norm (the shared
  representation is normalised per token row), then rounded to the run dtype;
* V: silu(N(0, 1)) in float64, rounded to the run dtype;
* kappa_q, kappa_k, eta_q, eta_k ~ N(1, 0.1) and nu_q, nu_k, rho_q, rho_k
  ~ N(0, 0.1) (standard deviations), one vector of d values per head, float32.

Host generation uses NumPy PCG64 seeded with
SeedSequence(seed, spawn_key=(tag, tensor_id, b, h)). Rounding to bf16 is
round-to-nearest-even done on the float32 bit pattern. Values are returned as
float32 arrays whose entries are exactly representable in the run dtype.
"""

from __future__ import annotations

import numpy as np

AFFINE_NAMES = ("kappa_q", "nu_q", "kappa_k", "nu_k", "eta_q", "rho_q", "eta_k", "rho_k")
_Z, _V, _P = 0, 1, 2


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _rng(seed: int, tag: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tag, tensor, b, h))))


def _round(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(x32)
    if dtype == "f32":
        return x32
    raise ValueError(f"unknown dtype {dtype!r}")


def make_z(n: int, d: int, dtype: str, seed: int, tag: int, b: int, h: int) -> np.ndarray:
    g = _rng(seed, tag, _Z, b, h).standard_normal((n, d))
    g /= np.linalg.norm(g, axis=1, keepdims=True)
    return _round(g, dtype)


def make_v(n: int, dv: int, dtype: str, seed: int, tag: int, b: int, h: int) -> np.ndarray:
    g = _rng(seed, tag, _V, b, h).standard_normal((n, dv))
    return _round(g / (1.0 + np.exp(-g)), dtype)


def make_params(H: int, d: int, seed: int, tag: int) -> dict:
    rng = _rng(seed, tag, _P, 0, 0)
    p = {}
    for name in AFFINE_NAMES:
        mean = 1.0 if name[0] in ("k", "e") else 0.0  # kappa/eta scale, nu/rho shift
        p[name] = (mean + 0.1 * rng.standard_normal((H, d))).astype(np.float32)
    return p


def make_inputs(B: int, H: int, n: int, d: int, dv: int, dtype: str, seed: int = 0, tag: int = 0) -> dict:
    """Host inputs: z [B,H,n,d], v [B,H,n,dv] float32 (dtype-exact), params [H,d] float32."""
    z = np.empty((B, H, n, d), np.float32)
    v = np.empty((B, H, n, dv), np.float32)
    for b in range(B):
        for h in range(H):
            z[b, h] = make_z(n, d, dtype, seed, tag, b, h)
            v[b, h] = make_v(n, dv, dtype, seed, tag, b, h)
    return {"z": z, "v": v, "params": make_params(H, d, seed, tag), "dtype": dtype}


def make_inputs_device(B: int, H: int, n: int, d: int, dv: int, dtype: str, seed: int = 0,
                       tag: int = 0, device: str = "cuda") -> dict:
    """Same recipe drawn with torch's device generator (for sizes too large to draw
    on the host in a test's time). Returns torch tensors on ``device`` in the run
    dtype; params are float32 [H, d] drawn on the host as in ``make_params``.
    """
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    z = torch.empty((B, H, n, d), dtype=tdt, device=device)
    v = torch.empty((B, H, n, dv), dtype=tdt, device=device)
    step = 1 << 20
    for b in range(B):
        for h in range(H):
            gen.manual_seed((seed * 1000003 + tag * 10007 + b * 101 + h) & 0x7FFFFFFF)
            for a in range(0, n, step):
                e = min(a + step, n)
                g = torch.randn((e - a, d), generator=gen, device=device, dtype=torch.float32)
                z[b, h, a:e] = (g / g.norm(dim=1, keepdim=True)).to(tdt)
                g = torch.randn((e - a, dv), generator=gen, device=device, dtype=torch.float32)
                v[b, h, a:e] = (g * torch.sigmoid(g)).to(tdt)
    params = make_params(H, d, seed, tag)
    return {"z": z, "v": v, "params": params, "dtype": dtype}


# ---------------------------------------------------------------- backward
_DO = 3


def make_dout(B: int, H: int, n: int, dv: int, dtype: str, seed: int = 0, tag: int = 0) -> np.ndarray:
    """Upstream gradient dL/dO for the backward: iid N(0, 1), rounded to the run
    dtype, float32 [B, H, n, dv] (drawn per (batch, head) slab like Z' and V)."""
    out = np.empty((B, H, n, dv), np.float32)
    for b in range(B):
        for h in range(H):
            out[b, h] = _round(_rng(seed, tag, _DO, b, h).standard_normal((n, dv)), dtype)
    return out


def sharpen(params: dict, factor: float) -> dict:
    """The same affine vectors with the scales (kappa, eta) multiplied by
    ``factor``: larger logits, peakier attention and feature softmaxes."""
    return {k: (v * np.float32(factor) if k[0] in ("k", "e") else v).astype(np.float32) for k, v in params.items()}


# ---------------------------------------------------------------- CEMA
_CX, _CP, _CR = 10, 11, 12


def make_cema_inputs(B: int, n: int, D: int, h: int, dtype: str, seed: int = 0, tag: int = 0,
                     reset_rate: float = 0.0) -> dict:
    """Seeded inputs for CEMA: x [B, n, D] iid N(0, 1) rounded to the run dtype;
    per (dimension, hidden dimension) float32 parameters alpha ~ U(0.05, 0.5),
    delta ~ U(0.1, 1) (so the damping factor stays at most 0.995), theta ~
    U(-pi, pi), beta ~ N(0, 1), eta = N(0, 1) + i N(0, 1) as [D, h, 2]; reset
    [B, n] uint8, each token a document boundary with probability reset_rate."""
    x = np.empty((B, n, D), np.float32)
    for b in range(B):
        x[b] = _round(_rng(seed, tag, _CX, b, 0).standard_normal((n, D)), dtype)
    rng = _rng(seed, tag, _CP, 0, 0)
    params = {
        "alpha": rng.uniform(0.05, 0.5, (D, h)).astype(np.float32),
        "delta": rng.uniform(0.1, 1.0, (D, h)).astype(np.float32),
        "theta": rng.uniform(-np.pi, np.pi, (D, h)).astype(np.float32),
        "beta": rng.standard_normal((D, h)).astype(np.float32),
        "eta": rng.standard_normal((D, h, 2)).astype(np.float32),
    }
    reset = (_rng(seed, tag, _CR, 0, 0).random((B, n)) < reset_rate).astype(np.uint8)
    return {"x": x, "params": params, "reset": reset, "dtype": dtype}


def make_cema_inputs_device(B: int, n: int, D: int, h: int, dtype: str, seed: int = 0, tag: int = 0,
                            device: str = "cuda") -> dict:
    """The CEMA recipe with x drawn by torch's device generator (sizes too large
    to draw on the host quickly); parameters as in make_cema_inputs; no resets."""
    import torch

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed((seed * 1000003 + tag * 10007 + 17) & 0x7FFFFFFF)
    x = torch.empty((B, n, D), dtype=tdt, device=device)
    step = 1 << 14
    for b in range(B):
        for a in range(0, n, step):
            e = min(a + step, n)
            x[b, a:e] = torch.randn((e - a, D), generator=gen, device=device, dtype=torch.float32).to(tdt)
    host = make_cema_inputs(1, 1, D, h, dtype, seed, tag)
    params = {k: torch.from_numpy(v).to(device).contiguous() for k, v in host["params"].items()}
    return {"x": x, "params": params}


# ---------------------------------------------------------------- TDN
_TX, _TP = 20, 21


def make_tdn_inputs(B: int, n: int, D: int, dtype: str, seed: int = 0, tag: int = 0) -> dict:
    """Seeded inputs for timestep decay normalisation: x [B, n, D] =
    s_t N(0, 1) + o_t + f_d, with a per-token scale s_t and offset o_t that
    drift over the sequence (random walks, so the decayed statistics matter)
    and a fixed per-feature offset f_d, rounded to the run dtype; gamma
    ~ N(1, 0.1), shift ~ N(0, 0.1) per feature, float32."""
    x = np.empty((B, n, D), np.float32)
    for b in range(B):
        rng = _rng(seed, tag, _TX, b, 0)
        walk = np.cumsum(rng.standard_normal((n, 2)) * 0.05, axis=0)
        scale = np.exp(0.5 * np.tanh(walk[:, :1]))
        offset = 2.0 * np.tanh(walk[:, 1:])
        feat = rng.standard_normal((1, D)) * 0.5
        x[b] = _round(rng.standard_normal((n, D)) * scale + offset + feat, dtype)
    rng = _rng(seed, tag, _TP, 0, 0)
    return {"x": x, "gamma": (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32),
            "shift": (0.1 * rng.standard_normal(D)).astype(np.float32), "dtype": dtype}
