"""CPU tier: the TDN oracle against what fixes it independently: torch's group
normalisation (when the statistics reduce to the current token's), SciPy's
IIR filter for the decayed statistics, the bias correction's defining
property, and the split of a sequence into two calls."""

from __future__ import annotations

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.signal import lfilter

import oracle


def group_norm(x, G, gamma, shift, eps):
    t = torch.from_numpy(np.ascontiguousarray(x, np.float64))
    y = F.group_norm(t, G, weight=torch.from_numpy(gamma.astype(np.float64)),
                     bias=torch.from_numpy(shift.astype(np.float64)), eps=eps)
    return y.numpy()


def params(D, seed):
    rng = np.random.default_rng(seed)
    return 1.0 + 0.1 * rng.standard_normal(D), 0.1 * rng.standard_normal(D)


@pytest.mark.parametrize("n,D,G", [(1, 8, 2), (30, 12, 3), (64, 64, 8)])
def test_no_decay_is_group_norm_of_each_token(n, D, G):
    x = np.random.default_rng(n + D).standard_normal((n, D)) * 3 + 1
    gamma, shift = params(D, 1)
    y, _ = oracle.tdn(x, G, 0.0, 0.0, gamma, shift, eps=1e-5)
    np.testing.assert_allclose(y, group_norm(x, G, gamma, shift, 1e-5), rtol=1e-12, atol=1e-12)


def test_repeated_token_is_group_norm_for_any_decay():
    # bias correction makes m_hat and v_hat the current statistics when they
    # do not change over time
    D, G = 16, 4
    row = np.random.default_rng(2).standard_normal(D)
    x = np.tile(row, (50, 1))
    gamma, shift = params(D, 3)
    y, _ = oracle.tdn(x, G, 0.9, 0.99, gamma, shift)
    np.testing.assert_allclose(y, group_norm(x, G, gamma, shift, 1e-5), rtol=1e-10, atol=1e-10)


def test_statistics_are_first_order_filters():
    n, D, G, b1, b2, eps = 200, 12, 3, 0.9, 0.97, 1e-5
    x = np.random.default_rng(4).standard_normal((n, D))
    gamma, shift = params(D, 5)
    y, (m, v, t) = oracle.tdn(x, G, b1, b2, gamma, shift, eps)
    grp = x.reshape(n, G, D // G)
    mu = grp.mean(axis=2)
    var = grp.var(axis=2)
    mf = lfilter([1 - b1], [1, -b1], mu, axis=0)
    vf = lfilter([1 - b2], [1, -b2], var, axis=0)
    tt = np.arange(1, n + 1)[:, None]
    mh = mf / (1 - b1 ** tt)
    vh = vf / (1 - b2 ** tt)
    want = (grp - mh[..., None]) / np.sqrt(vh[..., None] + eps)
    np.testing.assert_allclose(y, gamma * want.reshape(n, D) + shift, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(m, mf[-1], rtol=1e-12)
    np.testing.assert_allclose(v, vf[-1], rtol=1e-12)
    assert t == n


def test_two_calls_equal_one():
    n, D, G = 90, 8, 2
    x = np.random.default_rng(6).standard_normal((n, D))
    gamma, shift = params(D, 7)
    y, st = oracle.tdn(x, G, 0.8, 0.95, gamma, shift)
    y1, s1 = oracle.tdn(x[:37], G, 0.8, 0.95, gamma, shift)
    y2, s2 = oracle.tdn(x[37:], G, 0.8, 0.95, gamma, shift, state=s1)
    np.testing.assert_allclose(np.concatenate([y1, y2]), y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s2[0], st[0], rtol=1e-12)
    assert s2[2] == st[2] == n
