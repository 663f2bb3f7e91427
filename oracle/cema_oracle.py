"""Plain complex128 CPU oracle for CEMA, the complex multi-dimensional damped
exponential moving average that produces X' = CEMA(X) before Z'.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py`` may import or call this module. It shares no code with the HIP
library or its binding.

Sources (cited by site and section):

* [rainbus] structured summary on paper.rainbus.top, "Prerequisites / EMA"
  (the damped complex recurrence) and "Method steps" (1) (X' = CEMA(X)).
* [paperlayer] section-by-section summary on paperlayer.ai, 2.1 "CEMA"
  (each input dimension is expanded into h dimensions, the damped EMA runs in
  a complex hidden space, and the hidden state is projected back to one
  output per input dimension) and Appendix B.1 (the recurrence as an affine
  map h_t = q_t h_{t-1} + p_t; a boundary mask M_t = 0 resets the state to
  h_t = p_t).

The recurrence, per input dimension d and hidden dimension j:

    h_t = alpha * u_t + (1 - alpha * delta) (cos theta + i sin theta) * h_{t-1}

Readings taken where the pages leave a step open (each repeated where used):

* C1 expansion: u_t[d, j] = beta[d, j] x_t[d] (a real scale per hidden
  dimension, the plainest way to expand one value into h).
* C2 projection: y_t[d] = Re(sum_j eta[d, j] h_t[d, j]) with complex eta:
  every real-linear map from C^h to R has this form.
* C3 alpha, delta, theta, beta are real per (d, j); the multiplier
  q = (1 - alpha delta) e^{i theta} does not depend on t.
* C4 document resets: reset[t] != 0 means M_t = 0, so h_t = p_t.
* C5 the state before the first token is h_0 = 0, or a given state carried
  over from an earlier part of the same sequence.
"""

from __future__ import annotations

import numpy as np

__all__ = ["cema_multiplier", "cema"]


def cema_multiplier(alpha, delta, theta) -> np.ndarray:
    """q = (1 - alpha delta)(cos theta + i sin theta) per (d, j) (C3)."""
    alpha, delta, theta = (np.asarray(a, np.float64) for a in (alpha, delta, theta))
    return (1.0 - alpha * delta) * (np.cos(theta) + 1j * np.sin(theta))


def cema(x, alpha, delta, theta, beta, eta, reset=None, h0=None):
    """CEMA of one sequence: x [n, D] (real), parameters [D, h] (eta complex).

    Returns (y [n, D] float64, h_n [D, h] complex128): the outputs and the
    hidden state after the last token. Follows [rainbus "Prerequisites /
    EMA"] step by step: u_t = beta x_t (C1), h_t = alpha u_t + q M_t h_{t-1}
    with M_t = 0 on a reset (C4) and h_0 = h0 or 0 (C5), y_t = Re(eta . h_t)
    (C2).
    """
    x = np.asarray(x, np.float64)
    n, D = x.shape
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    eta = np.asarray(eta, np.complex128)
    q = cema_multiplier(alpha, delta, theta)
    h = np.zeros(alpha.shape, np.complex128) if h0 is None else np.array(h0, np.complex128)
    y = np.empty((n, D))
    for t in range(n):
        u = beta * x[t][:, None]
        keep = 0.0 if (reset is not None and reset[t]) else 1.0
        h = alpha * u + keep * q * h
        y[t] = np.real((eta * h).sum(axis=1))
    return y, h
