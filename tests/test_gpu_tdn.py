"""GPU tier: timestep decay normalisation (gecko_tdn_forward) through the C ABI
against the float64 oracle on the same seeded inputs (bf16 inputs are exact in
float32). Statistics and sums are float32 on the GPU; the outputs are O(1)
normalised values, so the bar is max |y - x| / rms(x) <= 1e-4 on float32
output, and the carried sums match to 1e-4 relative. Cases: no decay (plain
per-token group normalisation), typical and near-one decay factors (the bias
correction at its most delicate, and a sequence long enough for the sums to
reach their steady state, where float32 sums would drift by about
2^-25 / (1 - beta)), groups of 8 to 1024 features (reduced across lanes, or
through LDS where a group is not a power-of-two run of at most 64 lanes), one
token, the chunked scan, a
sequence continued over two calls, and the bf16 output rounding."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from chunked_attention_memory_amd import inputs
from gpu_helpers import announce, gecko

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _err(got, want):
    return float(np.max(np.abs(got - want)) / max(np.sqrt(np.mean(want * want)), 1e-30))


def _dev(host):
    import torch

    tdt = torch.bfloat16 if host["dtype"] == "bf16" else torch.float32
    x = torch.from_numpy(host["x"]).to("cuda").to(tdt).contiguous()
    return x, torch.from_numpy(host["gamma"]).cuda(), torch.from_numpy(host["shift"]).cuda()


@pytest.mark.parametrize("B,n,D,G,b1,b2,dtype", [
    (1, 300, 64, 8, 0.9, 0.99, "f32"),
    (2, 1000, 512, 8, 0.95, 0.999, "bf16"),
    (1, 1, 16, 2, 0.9, 0.99, "bf16"),
    (1, 700, 256, 4, 0.0, 0.0, "f32"),          # no decay: group norm of each token
    (1, 5000, 4096, 64, 0.999, 0.9999, "bf16"),  # chunked scan, factors near one
    (1, 65536, 256, 8, 0.999, 0.9999, "bf16"),   # long enough for the sums to settle
    (1, 900, 192, 1, 0.9, 0.99, "f32"),          # 24 lanes per group: the LDS reduction
    (2, 333, 1024, 1, 0.95, 0.999, "bf16"),      # 128 lanes per group: the LDS reduction
    (1, 100, 8192, 16, 0.9, 0.99, "bf16"),       # four 8-feature runs per thread, 64 lanes per group
    (1, 200, 128, 8, 0.9, 0.99, "f32"),          # 2 lanes per group
    (1, 500, 512, 4, 0.9, 0.99, "bf16"),         # 16 lanes per group
    (1, 300, 1024, 4, 0.9, 0.99, "f32"),         # 32 lanes per group
])
def test_tdn_matches_oracle(B, n, D, G, b1, b2, dtype):
    import torch

    g = gecko()
    host = inputs.make_tdn_inputs(B, n, D, dtype, tag=70 + G)
    x, gamma, shift = _dev(host)
    announce(f"tdn B,n,D={B},{n},{D} G={G} betas={b1},{b2} dtype={dtype}")
    y, (m, v, t) = g.gecko_tdn_forward(x, gamma, shift, G, b1, b2, want_state=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert t == n
    f1, f2 = float(np.float32(b1)), float(np.float32(b2))  # the factors the kernel receives
    for b in range(B):
        want, (mw, vw, tw) = oracle.tdn(host["x"][b], G, f1, f2, host["gamma"], host["shift"])
        assert _err(y[b].cpu().numpy().astype(np.float64), want) <= TOL
        assert np.max(np.abs(m[b].cpu().numpy() - mw)) <= TOL * max(1.0, np.max(np.abs(mw)))
        assert np.max(np.abs(v[b].cpu().numpy() - vw)) <= TOL * np.max(np.abs(vw))


def test_tdn_two_calls_continue_one_sequence_and_bf16_output():
    import torch

    g = gecko()
    B, n, D, G, b1, b2 = 1, 3000, 256, 8, 0.97, 0.995
    host = inputs.make_tdn_inputs(B, n, D, "bf16", tag=80)
    x, gamma, shift = _dev(host)
    k = 1234
    y1, st = g.gecko_tdn_forward(x[:, :k].contiguous(), gamma, shift, G, b1, b2, want_state=True,
                                 out_dtype=torch.float32)
    y2 = g.gecko_tdn_forward(x[:, k:].contiguous(), gamma, shift, G, b1, b2, state=st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want, _ = oracle.tdn(host["x"][0], G, float(np.float32(b1)), float(np.float32(b2)), host["gamma"], host["shift"])
    got = torch.cat([y1, y2], dim=1)[0].cpu().numpy().astype(np.float64)
    assert _err(got, want) <= TOL
    y = g.gecko_tdn_forward(x, gamma, shift, G, b1, b2, out_dtype=torch.float32)
    y16 = g.gecko_tdn_forward(x, gamma, shift, G, b1, b2, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    u = y.cpu().numpy().view(np.uint32)
    want16 = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    np.testing.assert_array_equal(y16.view(torch.int16).cpu().numpy().view(np.uint16), want16)
