"""Shared helpers for the GPU tier: run the HIP path through the C ABI and the
oracle on the same seeded inputs, and measure the error the way the parity bar
defines it."""

from __future__ import annotations

import sys

import numpy as np

import oracle
from chunked_attention_memory_amd import inputs

BF16_TOL = 2e-2  # max |y - x| / rms(x), bf16 inputs with fp32 accumulation
F32_TOL = 1e-4   # max |y - x| / max(|x|, 1e-3 rms(x)), float32 path


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def gecko():
    from chunked_attention_memory_amd import gecko as g

    return g


def to_numpy(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_raw(host: dict, c: int, entry: str = "full", flags: int = 0, device_inputs=None, out_f32=True):
    """Run one entry point on the GPU; returns the output tensor (float32 output
    unless ``out_f32`` is False, then the input dtype)."""
    import torch

    g = gecko()
    z, v, p = device_inputs if device_inputs is not None else g.to_device_inputs(host)
    od = torch.float32 if out_f32 else z.dtype
    announce(f"{entry} B,H,n,d,dv={tuple(z.shape[:3]) + (z.shape[3], v.shape[3])} c={c} dtype={z.dtype} "
             f"out={od} flags={flags}")
    if entry == "full":
        out = g.gecko_sca_awm_forward(z, p, v, c, flags=flags, out_dtype=od)
    elif entry == "sca":
        out = g.gecko_sca_forward(z, p, v, c, out_dtype=od)
    elif entry == "awm":
        out = g.gecko_awm_forward(z, p, v, c, flags=flags, out_dtype=od)
    else:
        raise ValueError(entry)
    torch.cuda.synchronize()
    # the output starts as NaN (tests/conftest.py): every row must be written
    assert bool(torch.isfinite(out).all()), f"{entry}: output holds unwritten or non-finite entries"
    return out


def run(host: dict, c: int, entry: str = "full", flags: int = 0, device_inputs=None, out_f32=True):
    """As run_raw, as float64 numpy [B, H, n, dv]."""
    return to_numpy(run_raw(host, c, entry, flags, device_inputs, out_f32))


def oracle_parts(host: dict, c: int, heads=None, no_delta=False, sca_chunks=None) -> dict:
    """Oracle O_SCA, O_m and O per (b, h) in ``heads`` (default: all)."""
    z, v, p = host["z"], host["v"], host["params"]
    B, H = z.shape[:2]
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    res = {}
    for b, h in heads:
        res[(b, h)] = oracle.forward_head(z[b, h], v[b, h], p, h, c, no_delta=no_delta, sca_chunks=sca_chunks)
    return res


def rms_err(got: np.ndarray, want: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(got - want))) / max(rms, 1e-30)


def floor_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-3 * rms)))


def make(B, H, n, d, dv, dtype="bf16", seed=0, tag=99):
    return inputs.make_inputs(B, H, n, d, dv, dtype, seed=seed, tag=tag)
