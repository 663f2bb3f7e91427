"""CPU tier: the gradient oracle against finite differences of the independent
numpy forward and against exact invariants of the definition."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import gecko_grad_oracle as go


def rand_problem(n, d, dv, H, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((1, H, n, d)) * 0.7
    v = rng.standard_normal((1, H, n, dv))
    p = {}
    for k in go.AFFINE:
        base = 1.0 if k.startswith(("kappa", "eta")) else 0.0
        p[k] = (base + 0.4 * rng.standard_normal((H, d))) * (scale if k.startswith(("kappa", "eta")) else 1.0)
    dout = rng.standard_normal((1, H, n, dv))
    return z, v, p, dout


def numpy_loss(z, v, p, c, dout, parts, chunkwise, no_delta):
    """L = sum(dout * O) from the numpy forward oracle (gecko_oracle)."""
    tot = 0.0
    for h in range(z.shape[1]):
        r = oracle.forward_head(z[0, h], v[0, h], p, h, c, no_delta=no_delta, chunkwise=chunkwise)
        o = sum(r["o_sca" if part == "sca" else "o_m"] for part in parts)
        tot += float((o * dout[0, h]).sum())
    return tot


VARIANTS = [
    (("sca", "awm"), False, False),
    (("sca",), False, False),
    (("awm",), False, False),
    (("awm",), False, True),
    (("sca", "awm"), True, False),
]


@pytest.mark.parametrize("parts,chunkwise,no_delta", VARIANTS)
def test_torch_forward_matches_numpy_forward(parts, chunkwise, no_delta):
    z, v, p, _ = rand_problem(37, 6, 5, 2, seed=3, scale=1.5)
    for h in range(2):
        pt = {k: torch.as_tensor(p[k][h]) for k in go.AFFINE}
        got = go.forward_torch_head(torch.as_tensor(z[0, h]), torch.as_tensor(v[0, h]), pt, 8, parts=parts,
                                    chunkwise=chunkwise, no_delta=no_delta).numpy()
        r = oracle.forward_head(z[0, h], v[0, h], p, h, 8, no_delta=no_delta, chunkwise=chunkwise)
        want = sum(r["o_sca" if part == "sca" else "o_m"] for part in parts)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("parts,chunkwise,no_delta", VARIANTS)
@pytest.mark.parametrize("n,c", [(11, 4), (9, 3)])
def test_gradients_match_finite_differences(parts, chunkwise, no_delta, n, c):
    """Every partial derivative against a central difference of the numpy
    forward (step 1e-6: truncation ~1e-12, rounding ~1e-10)."""
    d, dv, H = 4, 3, 2
    z, v, p, dout = rand_problem(n, d, dv, H, seed=n * 7 + c, scale=1.5)
    g = go.grad(z, v, p, c, dout, parts=parts, chunkwise=chunkwise, no_delta=no_delta)
    eps = 1e-6

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + eps
        up = numpy_loss(z, v, p, c, dout, parts, chunkwise, no_delta)
        arr[idx] = old - eps
        dn = numpy_loss(z, v, p, c, dout, parts, chunkwise, no_delta)
        arr[idx] = old
        return (up - dn) / (2 * eps)

    checks = [(z, "dz"), (v, "dv")] + [(p[k], "d" + k) for k in go.AFFINE]
    for arr, key in checks:
        want = np.empty(arr.shape)
        for idx in np.ndindex(arr.shape):
            want[idx] = fd(arr, idx)
        got = g[key] if key in ("dz", "dv") else g[key]
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7, err_msg=key)


@pytest.mark.parametrize("chunkwise", [False, True])
def test_key_shift_does_not_reach_attention(chunkwise):
    """Adding nu_k shifts every logit of query i by q_i . delta, the same for
    all its keys, and softmax ignores a per-row shift: d nu_k = 0 exactly."""
    z, v, p, dout = rand_problem(70, 8, 5, 2, seed=11, scale=2.0)
    g = go.grad(z, v, p, 16, dout, parts=("sca",), chunkwise=chunkwise)
    scale = np.abs(g["dkappa_k"]).max()
    assert np.abs(g["dnu_k"]).max() <= 1e-12 * scale


@pytest.mark.parametrize("no_delta", [False, True])
def test_memory_is_invariant_to_uniform_shifts(no_delta):
    """psi (a feature softmax) ignores a shift shared by all features of a row,
    and phi^s = exp(k)/z^s and the ratio z^{s-1}/z^s ignore any per-feature
    shift of the keys. So sum_f d rho_q = 0 and sum_f d rho_k = 0, and without
    the delta term (no psi(K)) d rho_k = 0 per feature."""
    z, v, p, dout = rand_problem(90, 8, 6, 2, seed=12, scale=1.5)
    g = go.grad(z, v, p, 16, dout, parts=("awm",), no_delta=no_delta)
    scale = max(np.abs(g["deta_q"]).max(), np.abs(g["deta_k"]).max())
    assert np.abs(g["drho_q"].sum(axis=1)).max() <= 1e-11 * scale
    assert np.abs(g["drho_k"].sum(axis=1)).max() <= 1e-11 * scale
    if no_delta:
        assert np.abs(g["drho_k"]).max() <= 1e-11 * scale
    else:
        assert np.abs(g["drho_k"]).max() > 1e-3 * scale


@pytest.mark.parametrize("parts", [("sca",), ("awm",), ("sca", "awm")])
def test_output_is_linear_in_values(parts):
    """O is linear in V (SCA weights and the memory transition depend on Z'
    only), so <V, dL/dV> = L for L = sum(dout * O)."""
    z, v, p, dout = rand_problem(75, 8, 6, 2, seed=13, scale=1.5)
    g = go.grad(z, v, p, 16, dout, parts=parts)
    loss = numpy_loss(z, v, p, 16, dout, parts, False, False)
    assert abs(float((v * g["dv"]).sum()) - loss) <= 1e-10 * max(1.0, abs(loss))


@pytest.mark.parametrize("chunkwise", [False, True])
def test_lse_reproduces_attention(chunkwise):
    """exp(logit - lse) are the softmax weights: applied to V they give the
    numpy oracle's O_SCA."""
    z, v, p, _ = rand_problem(70, 8, 5, 1, seed=14, scale=2.0)
    lse = go.lse_head(z[0, 0], p, 0, 16, chunkwise=chunkwise)
    q = z[0, 0] * p["kappa_q"][0] + p["nu_q"][0]
    k = z[0, 0] * p["kappa_k"][0] + p["nu_k"][0]
    n = 70
    out = np.zeros((n, 5))
    for i in range(n):
        a = (i // 16) * 16
        k0 = a if chunkwise else max(0, a - 16)
        for j in range(k0, i + 1):
            out[i] += np.exp(q[i] @ k[j] - lse[i]) * v[0, 0, j]
    want = oracle.sca_head(z[0, 0], v[0, 0], p["kappa_q"][0], p["nu_q"][0], p["kappa_k"][0], p["nu_k"][0], 16,
                           sliding=not chunkwise)
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("parts,chunkwise,no_delta", VARIANTS)
def test_per_token_gradients_compose(parts, chunkwise, no_delta):
    """The per-token gradients with respect to Q, K, Q_m, K_m give back, by
    the chain rule through the affine maps, the finite-difference-pinned dZ'
    and affine gradients."""
    z, v, p, dout = rand_problem(60, 8, 5, 2, seed=21, scale=1.5)
    g = go.grad(z, v, p, 16, dout, parts=parts, chunkwise=chunkwise, no_delta=no_delta)
    dz = (p["kappa_q"][None, :, None] * g["dq"] + p["kappa_k"][None, :, None] * g["dk"]
          + p["eta_q"][None, :, None] * g["dqm"] + p["eta_k"][None, :, None] * g["dkm"])
    np.testing.assert_allclose(dz, g["dz"], rtol=1e-10, atol=1e-12)
    for scale, shift, key in (("kappa_q", "nu_q", "dq"), ("kappa_k", "nu_k", "dk"),
                              ("eta_q", "rho_q", "dqm"), ("eta_k", "rho_k", "dkm")):
        np.testing.assert_allclose((z * g[key]).sum(axis=(0, 2)), g["d" + scale], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g[key].sum(axis=(0, 2)), g["d" + shift], rtol=1e-10, atol=1e-12)
