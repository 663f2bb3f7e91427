"""GPU tier: properties the method fixes exactly, checked through the C ABI.

* closed forms of the memory (without the delta term; with constant keys);
* the memory is exactly zero on the first two chunks;
* bit-exact locality: a token only influences attention rows from itself to
  the end of the next chunk, and memory rows from two chunks later on;
* heads are independent; runs are deterministic; value columns permute
  bit for bit;
* large memory keys (the chunk pass's exact-maximum path) still match.
"""

from __future__ import annotations

import numpy as np
import pytest

import pins
from gpu_helpers import BF16_TOL, gecko, make, oracle_parts, rms_err, run, run_raw

pytestmark = pytest.mark.gpu

B, H, N_TOK, C, D, DV = 1, 2, 1400, 128, 128, 256   # 11 chunks, ragged tail


def _dev(host):
    return gecko().to_device_inputs(host)


def _bits(t):
    import torch

    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def test_no_delta_matches_linear_attention_closed_form():
    host = make(B, H, N_TOK, D, DV, tag=11)
    got = run(host, C, "awm", flags=gecko().GECKO_AWM_NO_DELTA)
    for h in range(H):
        p = host["params"]
        qm = host["z"][0, h].astype(np.float64) * p["eta_q"][h] + p["rho_q"][h]
        km = host["z"][0, h].astype(np.float64) * p["eta_k"][h] + p["rho_k"][h]
        want = pins.awm_no_delta_closed(qm, km, host["v"][0, h], C)
        assert rms_err(got[0, h], want) <= BF16_TOL


def test_no_delta_constant_values_read_back_one():
    host = make(B, H, N_TOK, D, DV, tag=12)
    host["v"][:] = 1.0
    got = run(host, C, "awm", flags=gecko().GECKO_AWM_NO_DELTA)
    assert np.all(got[:, :, : 2 * C] == 0.0)
    assert np.max(np.abs(got[:, :, 2 * C:] - 1.0)) <= 1e-2


def test_constant_keys_closed_form():
    host = make(B, H, N_TOK, D, DV, tag=13)
    host["params"]["eta_k"][:] = 0.0
    got = run(host, C, "awm")
    for h in range(H):
        want = pins.awm_const_key_closed(host["v"][0, h], C)
        assert rms_err(got[0, h], want) <= BF16_TOL


def test_memory_is_exactly_zero_on_first_two_chunks():
    host = make(B, H, N_TOK, D, DV, tag=14)
    got = run(host, C, "awm")
    assert np.all(got[:, :, : 2 * C] == 0.0)
    assert np.all(np.abs(got[:, :, 2 * C:]).sum(axis=-1) > 0)
    # two chunks or fewer: the memory is never read
    got = run(make(1, 1, 2 * C, D, DV, tag=15), C, "awm")
    assert np.all(got == 0.0)


@pytest.mark.parametrize("j", [0, 77, 128, 300, 640, 1399])
def test_attention_band_is_exact(j):
    """Changing token j's Z' and V leaves every attention row outside
    [j, end of the chunk after j's chunk) bit-identical and changes the rows inside."""
    host = make(B, 1, N_TOK, D, DV, tag=16)
    base = run_raw(host, C, "sca")
    host2 = {**host, "z": host["z"].copy(), "v": host["v"].copy()}
    host2["z"][0, 0, j] = -host2["z"][0, 0, j]
    host2["v"][0, 0, j] += 0.5
    pert = run_raw(host2, C, "sca")
    same = np.all(_bits(base) == _bits(pert), axis=-1)[0, 0]
    lo, hi = j, min((j // C + 2) * C, N_TOK)
    inside = np.zeros(N_TOK, bool)
    inside[lo:hi] = True
    assert np.all(same[~inside])
    assert np.mean(~same[inside]) > 0.99


@pytest.mark.parametrize("j", [5, 200, 700, 1100])
def test_memory_lag_is_exact(j):
    """Changing V_j (token j in chunk t) leaves memory rows of chunks <= t+1
    bit-identical and changes rows of chunks >= t+2."""
    host = make(B, 1, N_TOK, D, DV, tag=17)
    base = run_raw(host, C, "awm")
    host2 = {**host, "v": host["v"].copy()}
    host2["v"][0, 0, j] += 1.0
    pert = run_raw(host2, C, "awm")
    same = np.all(_bits(base) == _bits(pert), axis=-1)[0, 0]
    cut = min((j // C + 2) * C, N_TOK)
    assert np.all(same[:cut])
    if cut < N_TOK:
        assert np.mean(~same[cut:]) > 0.99


def test_heads_are_independent_and_runs_deterministic():
    host = make(2, 2, 900, D, DV, tag=18)
    a = run_raw(host, C, "full")
    b = run_raw(host, C, "full")
    assert np.array_equal(_bits(a), _bits(b))
    host2 = {**host, "z": host["z"].copy(), "v": host["v"].copy()}
    host2["z"][1, 0] = host2["z"][1, 0][::-1]
    host2["v"][1, 0] *= 2.0
    c = run_raw(host2, C, "full")
    ba, bc = _bits(a), _bits(c)
    for bb, hh in [(0, 0), (0, 1), (1, 1)]:
        assert np.array_equal(ba[bb, hh], bc[bb, hh])
    assert not np.array_equal(ba[1, 0], bc[1, 0])


def test_value_columns_permute():
    """Permuting V's columns permutes O's columns bit for bit: every value
    column goes through the same products (P V, E^T V, the state update and
    the readout, each a dot product over keys or features in a fixed order),
    and the row statistics (attention and feature softmax sums) do not read V."""
    host = make(B, H, N_TOK, D, DV, tag=19)
    perm = np.random.default_rng(0).permutation(DV)
    host2 = {**host, "v": np.ascontiguousarray(host["v"][..., perm])}
    a = _bits(run_raw(host, C, "full"))
    b = _bits(run_raw(host2, C, "full"))
    assert np.array_equal(b, a[..., perm])


def test_feature_permutation_with_affine_vectors():
    host = make(B, H, N_TOK, D, DV, tag=20)
    perm = np.random.default_rng(1).permutation(D)
    host2 = {**host, "z": np.ascontiguousarray(host["z"][..., perm]),
             "params": {k: np.ascontiguousarray(v[:, perm]) for k, v in host["params"].items()}}
    a = run(host, C, "full")
    b = run(host2, C, "full")
    assert rms_err(b, a) <= 1e-2


@pytest.mark.parametrize("scale", [40.0, 70.0])
def test_large_memory_keys(scale):
    """|K_m| of order 100 (far outside plain fp32 exp range) with a spike late
    in the chunk, which drives the chunk pass past its first-tile offset."""
    host = make(B, H, N_TOK, D, DV, tag=21)
    host["params"]["eta_k"][:] *= scale
    host["z"][:, :, 3 * C + 100, 5] = 3.0  # one large key deep inside chunk 4
    ref = oracle_parts(host, C)
    got = run(host, C, "awm")
    want = np.stack([ref[(0, h)]["o_m"] for h in range(H)])[None]
    assert np.all(np.isfinite(got))
    assert rms_err(got, want) <= BF16_TOL

