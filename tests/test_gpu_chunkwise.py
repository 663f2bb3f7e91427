"""GPU tier: the chunk-wise variant (flag GECKO_CHUNKWISE: attention inside
the chunk, memory read one chunk earlier) through the C ABI, against the fp64
oracle's variant (sca_head(sliding=False), awm_head(lag=1)) on the same seeded
inputs, with the same bars as the default form (float32 path 1e-4 with the
floor, bf16 inputs 2e-2 of the rms), plus its closed forms and its exact lag."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import pins
from chunked_attention_memory_amd import configs
from gpu_helpers import BF16_TOL, F32_TOL, floor_rel_err, gecko, make, rms_err, run, run_raw

pytestmark = pytest.mark.gpu


def _oracle(host, c, heads=None, no_delta=False):
    z, v, p = host["z"], host["v"], host["params"]
    B, H = z.shape[:2]
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    return {bh: oracle.forward_head(z[bh[0], bh[1]], v[bh[0], bh[1]], p, bh[1], c, no_delta=no_delta,
                                    chunkwise=True) for bh in heads}


def _flags(extra=0):
    return gecko().GECKO_CHUNKWISE | extra


def test_f32_tiny_workload():
    w = configs.WORKLOADS[0]
    host = make(w.B, w.H, w.n, w.d, w.dv, "f32", tag=30)
    ref = _oracle(host, w.c)[(0, 0)]
    got = run(host, w.c, "full", flags=_flags())
    assert floor_rel_err(got[0, 0], ref["o"]) <= F32_TOL
    got = run(host, w.c, "awm", flags=_flags())
    assert floor_rel_err(got[0, 0], ref["o_m"]) <= F32_TOL


@pytest.mark.parametrize("B,H,n,c,d,dv", [
    (1, 2, 700, 128, 128, 256),   # ragged tail
    (2, 1, 513, 64, 128, 256),    # chunk smaller than a query tile
    (1, 1, 300, 300, 128, 256),   # one chunk: causal attention, no memory
    (1, 1, 777, 100, 128, 128),   # c not a multiple of the tile sizes
    (1, 2, 640, 128, 64, 128),
    (1, 1, 450, 64, 64, 64),
    (1, 1, 4096, 512, 128, 256),
    (1, 1, 600, 128, 32, 64),     # 64-byte key rows
    (1, 2, 500, 64, 128, 32),     # 64-byte value rows
])
def test_bf16_shapes(B, H, n, c, d, dv):
    host = make(B, H, n, d, dv, "bf16", tag=31)
    ref = _oracle(host, c)
    got = run(host, c, "full", flags=_flags())
    for (b, h), r in ref.items():
        assert rms_err(got[b, h], r["o"]) <= BF16_TOL
    got_m = run(host, c, "awm", flags=_flags())
    for (b, h), r in ref.items():
        if np.any(r["o_m"] != 0):
            assert rms_err(got_m[b, h], r["o_m"]) <= BF16_TOL
        else:
            assert np.all(got_m[b, h] == 0)


def test_f32_shapes_and_no_delta():
    host = make(1, 2, 300, 32, 64, "f32", tag=32)
    for extra in (0, gecko().GECKO_AWM_NO_DELTA):
        ref = _oracle(host, 64, no_delta=bool(extra))
        got = run(host, 64, "full", flags=_flags(extra))
        for (b, h), r in ref.items():
            assert floor_rel_err(got[b, h], r["o"]) <= F32_TOL


def test_first_chunk_reads_nothing_and_lag_is_one_chunk():
    """Perturbing V in chunk t leaves every memory row of chunks <= t
    bit-identical (chunk 1 reads exact zeros) and changes chunk t + 1."""
    import torch

    g = gecko()
    c = 128
    host = make(1, 1, 6 * c, 128, 256, "bf16", tag=33)
    z, v, p = g.to_device_inputs(host)
    base = run_raw(host, c, "awm", flags=_flags(), device_inputs=(z, v, p))
    assert bool((base[0, 0, :c] == 0).all())
    t = 2
    v2 = v.clone()
    v2[0, 0, t * c + 5] += 1.0
    pert = run_raw(host, c, "awm", flags=_flags(), device_inputs=(z, v2, p))
    assert torch.equal(base[0, 0, :(t + 1) * c], pert[0, 0, :(t + 1) * c])
    assert not torch.equal(base[0, 0, (t + 1) * c:(t + 2) * c], pert[0, 0, (t + 1) * c:(t + 2) * c])


def test_closed_forms_every_row_128k():
    """Equal logits (query affine zero) and equal memory keys (eta_k zero):
    every row is the window mean over its own chunk plus the constant-key
    state one chunk back, at 128K tokens (B1 H2), checked on every row."""
    w = configs.WORKLOADS[2]
    n, c = w.n, w.c
    host = make(1, 2, n, w.d, w.dv, "bf16", tag=34)
    p = host["params"]
    p["kappa_q"][:] = 0.0
    p["nu_q"][:] = 0.0
    p["eta_k"][:] = 0.0
    got = run(host, c, "full", flags=_flags())
    for h in range(2):
        vh = host["v"][0, h].astype(np.float64)
        want = pins.window_mean(vh, c, prev=0) + pins.awm_const_key_closed(vh, c, lag=1)
        assert rms_err(got[0, h], want) <= BF16_TOL
