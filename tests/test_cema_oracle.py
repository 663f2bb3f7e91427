"""CPU tier: the CEMA oracle against what fixes it independently: scipy's
IIR filter routine, closed forms (impulse response, constant input), resets
and the split of a sequence into two calls."""

from __future__ import annotations

import numpy as np
import pytest
from scipy.signal import lfilter

import oracle


def rand_params(D, h, seed):
    rng = np.random.default_rng(seed)
    alpha = rng.uniform(0.05, 0.95, (D, h))
    delta = rng.uniform(0.05, 1.0, (D, h))
    theta = rng.uniform(-np.pi, np.pi, (D, h))
    beta = rng.standard_normal((D, h))
    eta = rng.standard_normal((D, h)) + 1j * rng.standard_normal((D, h))
    return alpha, delta, theta, beta, eta


def lfilter_reference(x, alpha, delta, theta, beta, eta, reset=None):
    """Each (d, j) chain as a first-order complex IIR filter h = p / (1 - q z^-1)
    with p_t = alpha beta x_t, restarted from zero at every reset."""
    n, D = x.shape
    q = (1 - alpha * delta) * np.exp(1j * theta)
    starts = [0] + ([t for t in range(1, n) if reset[t]] if reset is not None else []) + [n]
    y = np.zeros((n, D))
    for d in range(D):
        for j in range(alpha.shape[1]):
            p = alpha[d, j] * beta[d, j] * x[:, d].astype(np.complex128)
            h = np.empty(n, np.complex128)
            for a, b in zip(starts[:-1], starts[1:]):
                h[a:b] = lfilter([1.0], [1.0, -q[d, j]], p[a:b])
            y[:, d] += np.real(eta[d, j] * h)
    return y


@pytest.mark.parametrize("n,D,h", [(1, 1, 1), (50, 3, 4), (200, 5, 16), (97, 2, 8)])
def test_cema_matches_iir_filter(n, D, h):
    rng = np.random.default_rng(n + D + h)
    x = rng.standard_normal((n, D))
    prm = rand_params(D, h, seed=n * 7 + h)
    y, _ = oracle.cema(x, *prm)
    np.testing.assert_allclose(y, lfilter_reference(x, *prm), rtol=1e-11, atol=1e-12)


def test_cema_resets_match_restarted_filter():
    rng = np.random.default_rng(3)
    n, D, h = 300, 4, 8
    x = rng.standard_normal((n, D))
    reset = np.zeros(n, np.uint8)
    reset[[0, 17, 18, 150, 299]] = 1
    prm = rand_params(D, h, seed=5)
    y, _ = oracle.cema(x, *prm, reset=reset)
    np.testing.assert_allclose(y, lfilter_reference(x, *prm, reset=reset), rtol=1e-11, atol=1e-12)
    # after a reset the outputs are those of a fresh run on the suffix
    y2, _ = oracle.cema(x[150:], *prm)
    np.testing.assert_allclose(y[150:299], y2[:149], rtol=1e-12, atol=1e-13)


def test_cema_impulse_response_closed_form():
    D, h, n, t0 = 2, 6, 40, 5
    alpha, delta, theta, beta, eta = rand_params(D, h, seed=11)
    x = np.zeros((n, D))
    x[t0, 1] = 1.0
    y, _ = oracle.cema(x, alpha, delta, theta, beta, eta)
    q = (1 - alpha[1] * delta[1]) * np.exp(1j * theta[1])
    k = np.arange(n - t0)
    want = np.real((eta[1] * alpha[1] * beta[1])[None, :] * q[None, :] ** k[:, None]).sum(axis=1)
    np.testing.assert_allclose(y[t0:, 1], want, rtol=1e-12, atol=1e-14)
    assert np.all(y[:t0] == 0.0) and np.all(y[:, 0] == 0.0)


def test_cema_constant_input_geometric_series():
    D, h, n = 3, 4, 60
    alpha, delta, theta, beta, eta = rand_params(D, h, seed=13)
    c = np.array([0.5, -1.25, 2.0])
    x = np.broadcast_to(c, (n, D))
    y, hn = oracle.cema(x, alpha, delta, theta, beta, eta)
    q = (1 - alpha * delta) * np.exp(1j * theta)
    t = np.arange(n)[:, None, None]
    hs = (alpha * beta * c[:, None])[None] * (1 - q[None] ** (t + 1)) / (1 - q[None])
    np.testing.assert_allclose(y, np.real((eta[None] * hs).sum(axis=2)), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(hn, hs[-1], rtol=1e-11, atol=1e-12)


def test_cema_two_calls_equal_one():
    rng = np.random.default_rng(17)
    n, D, h = 120, 3, 8
    x = rng.standard_normal((n, D))
    prm = rand_params(D, h, seed=19)
    y, hn = oracle.cema(x, *prm)
    y1, h1 = oracle.cema(x[:53], *prm)
    y2, h2 = oracle.cema(x[53:], *prm, h0=h1)
    np.testing.assert_allclose(np.concatenate([y1, y2]), y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h2, hn, rtol=1e-12, atol=1e-13)
