"""GPU tier: CEMA (gecko_cema_forward) through the C ABI against the complex128
oracle on the same seeded inputs (bf16 inputs are exact in float32, so both
sides see the same values). The kernel keeps its state in float32 with a
damping factor of at most 0.995, so rounding stays near 2^-24 times the
effective length of the memory (<= 200 steps): the bar is max |y - x| /
rms(x) <= 1e-4 on float32 output, the same for the final state. The bf16
output is the round-to-nearest-even of the float32 one. Cases: every
supported h, a dimension count that is not a multiple of a wave, one token,
resets (at the first token, consecutive, across the chunk boundaries of the
chunked three-phase path), calls without a reset array (the kernels built
without reset handling), a carried state in and out, and two calls that
continue one sequence."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from chunked_attention_memory_amd import inputs
from gpu_helpers import announce, gecko

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _dev(host, dtype=None):
    import torch

    tdt = torch.bfloat16 if host["dtype"] == "bf16" else torch.float32
    x = torch.from_numpy(host["x"]).to("cuda").to(tdt).contiguous()
    p = {k: torch.from_numpy(v).to("cuda").contiguous() for k, v in host["params"].items()}
    r = torch.from_numpy(host["reset"]).to("cuda").contiguous()
    return x, p, r


def _oracle(host, b, h0=None):
    p = host["params"]
    eta = p["eta"][..., 0].astype(np.float64) + 1j * p["eta"][..., 1]
    return oracle.cema(host["x"][b], p["alpha"], p["delta"], p["theta"], p["beta"], eta,
                       reset=host["reset"][b], h0=h0)


def _err(got, want):
    """max |got - want| / rms(want); complex arrays by modulus."""
    return float(np.max(np.abs(got - want)) / max(np.sqrt(np.mean(np.abs(want) ** 2)), 1e-30))


def _run(host, use_reset=True, h0=None, want_state=True, out_dtype=None):
    import torch

    g = gecko()
    x, p, r = _dev(host)
    announce(f"cema B,n,D={tuple(x.shape)} h={p['alpha'].shape[1]} dtype={x.dtype} reset={use_reset} "
             f"h0={h0 is not None}")
    res = g.gecko_cema_forward(x, p, reset=r if use_reset else None, h0=h0, want_state=want_state,
                               out_dtype=out_dtype or torch.float32)
    torch.cuda.synchronize()
    return res


def _state64(t):
    a = t.cpu().numpy().astype(np.float64)
    return a[..., 0] + 1j * a[..., 1]


@pytest.mark.parametrize("B,n,D,h,dtype,rate", [
    (1, 300, 64, 16, "f32", 0.0),
    (2, 257, 100, 8, "bf16", 0.01),   # D not a multiple of 64
    (1, 1, 64, 4, "bf16", 0.0),       # one token
    (1, 1000, 128, 2, "f32", 0.05),
    (1, 513, 192, 1, "bf16", 0.02),
])
def test_cema_matches_oracle(B, n, D, h, dtype, rate):
    host = inputs.make_cema_inputs(B, n, D, h, dtype, tag=40 + h, reset_rate=rate)
    y, hf = _run(host)
    for b in range(B):
        want, hn = _oracle(host, b)
        assert _err(y[b].cpu().numpy().astype(np.float64), want) <= TOL
        assert _err(_state64(hf[b]), hn) <= TOL


def test_cema_chunked_path_with_resets_and_carried_state():
    """n = 16384 at D = 64 runs as many chunks (three phases); resets fall on
    the first token, on chunk boundaries and in runs; a given h0 enters."""
    import torch

    B, n, D, h = 2, 16384, 64, 16
    g = gecko()
    plan_bytes = g.gecko_cema_workspace_size(B, n, D, h)
    assert plan_bytes > 0  # the chunked path
    host = inputs.make_cema_inputs(B, n, D, h, "bf16", tag=50, reset_rate=0.001)
    host["reset"][0, [0, 512, 1024, 1025, 1026, 8191, 8192]] = 1
    rng = np.random.default_rng(5)
    h0 = (rng.standard_normal((B, D, h)) + 1j * rng.standard_normal((B, D, h))).astype(np.complex64)
    h0t = torch.from_numpy(np.stack([h0.real, h0.imag], axis=-1).astype(np.float32)).cuda().contiguous()
    y, hf = _run(host, h0=h0t)
    for b in range(B):
        want, hn = _oracle(host, b, h0=h0[b].astype(np.complex128))
        assert _err(y[b].cpu().numpy().astype(np.float64), want) <= TOL
        assert _err(_state64(hf[b]), hn) <= TOL


def test_cema_two_calls_continue_one_sequence_and_bf16_output():
    import torch

    g = gecko()
    B, n, D, h = 1, 12000, 128, 16
    host = inputs.make_cema_inputs(B, n, D, h, "bf16", tag=51, reset_rate=0.0005)
    x, p, r = _dev(host)
    y, hf = g.gecko_cema_forward(x, p, reset=r, want_state=True, out_dtype=torch.float32)
    m = 7000
    y1, h1 = g.gecko_cema_forward(x[:, :m].contiguous(), p, reset=r[:, :m].contiguous(), want_state=True,
                                  out_dtype=torch.float32)
    y2, h2 = g.gecko_cema_forward(x[:, m:].contiguous(), p, reset=r[:, m:].contiguous(), h0=h1, want_state=True,
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    want, hn = _oracle(host, 0)
    got = torch.cat([y1, y2], dim=1)[0].cpu().numpy().astype(np.float64)
    assert _err(got, want) <= TOL
    assert _err(y[0].cpu().numpy().astype(np.float64), want) <= TOL
    assert _err(_state64(h2[0]), hn) <= TOL
    # bf16 output: the nearest-even rounding of the float32 output
    y16 = g.gecko_cema_forward(x, p, reset=r, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    u = y.cpu().numpy().view(np.uint32)
    want16 = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    np.testing.assert_array_equal(y16.view(torch.int16).cpu().numpy().view(np.uint16), want16)


@pytest.mark.parametrize("B,n,D,h,dtype,with_h0", [
    (1, 300, 64, 16, "f32", False),    # one chunk: phase C only
    (2, 257, 100, 8, "bf16", True),    # D not a multiple of 64
    (1, 16384, 64, 16, "bf16", True),  # the chunked three-phase path
    (2, 9000, 128, 4, "f32", False),   # chunked, ragged last chunk
])
def test_cema_without_reset_array(B, n, D, h, dtype, with_h0):
    """No reset array: the kernels built without reset handling (no step
    scales the state) against the oracle with no resets, and against the
    kernels that take an all-zero reset array."""
    import torch

    g = gecko()
    host = inputs.make_cema_inputs(B, n, D, h, dtype, tag=70 + h, reset_rate=0.0)
    assert not host["reset"].any()
    h0 = h0t = None
    if with_h0:
        rng = np.random.default_rng(11)
        h0 = (rng.standard_normal((B, D, h)) + 1j * rng.standard_normal((B, D, h))).astype(np.complex64)
        h0t = torch.from_numpy(np.stack([h0.real, h0.imag], axis=-1).astype(np.float32)).cuda().contiguous()
    if n >= 8192:
        assert g.gecko_cema_workspace_size(B, n, D, h) > 0  # the chunked path
    y, hf = _run(host, use_reset=False, h0=h0t)
    yz, hz = _run(host, use_reset=True, h0=h0t)
    for b in range(B):
        want, hn = _oracle(host, b, h0=None if h0 is None else h0[b].astype(np.complex128))
        assert _err(y[b].cpu().numpy().astype(np.float64), want) <= TOL
        assert _err(_state64(hf[b]), hn) <= TOL
        assert _err(y[b].cpu().numpy().astype(np.float64), yz[b].cpu().numpy().astype(np.float64)) <= TOL
