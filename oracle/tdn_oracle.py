"""Plain float64 CPU oracle for timestep decay normalisation (TDN).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py`` may import or call this module. It shares no code with the HIP
library or its binding.

Sources (cited by site and section):

* [rainbus] structured summary on paper.rainbus.top, "Novelty": the current
  statistics enter the cumulative ones with a fixed weight through decay
  factors beta_1, beta_2, m_t = beta_1 m_{t-1} + (1 - beta_1) mu_t, and the
  initialisation bias is corrected as in Adam.
* [paperlayer] section-by-section summary on paperlayer.ai, 2.2 (Megalodon's
  timestep normalisation accumulates means and variances of groups of the
  input over previous timesteps) and 3.1 (the decay fixes the share of the
  current mean and variance; bias correction applies to both statistics).

Readings taken where the pages leave a step open:

* T1 the features of a token are split into G equal groups; mu_t and
  sigma^2_t are the mean and the (biased) variance of token t's values in a
  group.
* T2 m_t = beta_1 m_{t-1} + (1 - beta_1) mu_t and
  v_t = beta_2 v_{t-1} + (1 - beta_2) sigma^2_t from m_0 = v_0 = 0; bias
  correction m_hat_t = m_t / (1 - beta_1^t), v_hat_t = v_t / (1 - beta_2^t)
  with t counted from 1 at the first token.
* T3 y_t = gamma * (x_t - m_hat_t) / sqrt(v_hat_t + eps) + b, with the group's
  m_hat_t and v_hat_t and a per-feature scale gamma and shift b.
* T4 a sequence may continue an earlier part: (m, v) and the token count are
  carried over.
"""

from __future__ import annotations

import numpy as np

__all__ = ["tdn"]


def tdn(x, G: int, beta1: float, beta2: float, gamma, shift, eps: float = 1e-5, state=None):
    """TDN of one sequence: x [n, D] (real), G groups of D / G features.

    Returns (y [n, D] float64, state) where state = (m [G], v [G], t) after
    the last token, to continue the sequence in a later call (T4).
    """
    x = np.asarray(x, np.float64)
    n, D = x.shape
    if D % G:
        raise ValueError("D must be a multiple of G")
    gamma = np.asarray(gamma, np.float64)
    shift = np.asarray(shift, np.float64)
    if state is None:
        m, v, t0 = np.zeros(G), np.zeros(G), 0
    else:
        m, v, t0 = np.array(state[0], np.float64), np.array(state[1], np.float64), int(state[2])
    y = np.empty((n, D))
    for i in range(n):
        t = t0 + i + 1
        grp = x[i].reshape(G, D // G)
        mu = grp.mean(axis=1)
        var = ((grp - mu[:, None]) ** 2).mean(axis=1)
        m = beta1 * m + (1.0 - beta1) * mu
        v = beta2 * v + (1.0 - beta2) * var
        mh = m / (1.0 - beta1 ** t)
        vh = v / (1.0 - beta2 ** t)
        norm = (grp - mh[:, None]) / np.sqrt(vh[:, None] + eps)
        y[i] = gamma * norm.reshape(D) + shift
    return y, (m, v, t0 + n)
