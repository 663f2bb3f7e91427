"""Independent formulations that pin the oracle (CPU, float64).

Each function here computes something the pages or plain mathematics fix, in a
form that differs from the oracle's own code (full masked matrices instead of a
chunk loop, explicit transition-matrix products instead of the recurrence,
closed forms, a library attention routine), so that a dropped term, a wrong
sign, an off-by-one chunk index or a transposed operand in the oracle shows up
as a mismatch. Nothing here imports the oracle or the HIP path.
"""

from __future__ import annotations

import numpy as np
from scipy.special import softmax as sp_softmax


def band_mask(n: int, c: int, prev: int = 1) -> np.ndarray:
    """Visibility of key j to query i: causal, and key chunk >= query chunk - prev
    (prev = 1: sliding chunks; prev = 0: the chunk-wise variant)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i) & (j // c >= i // c - prev)


def brute_sca(q, k, v, c, prev: int = 1):
    """Full n x n masked softmax attention (scale 1) with the band mask."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    logits = q @ k.T
    logits[~band_mask(q.shape[0], c, prev)] = -np.inf
    return sp_softmax(logits, axis=1) @ v


def causal_attention_torch(q, k, v):
    """Textbook causal softmax attention with scale 1, via torch's routine on CPU."""
    import torch
    import torch.nn.functional as F

    t = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None] for a in (q, k, v)]
    o = F.scaled_dot_product_attention(t[0], t[1], t[2], is_causal=True, scale=1.0)
    return o[0, 0].numpy()


def window_mean(v, c, prev: int = 1):
    """Closed form of SCA when every logit is equal: the mean of v over the window.

    The window of token i is [max(0, (i//c - prev) c), i]; prefix sums give each mean.
    """
    v = np.asarray(v, np.float64)
    n = v.shape[0]
    cs = np.vstack([np.zeros((1, v.shape[1])), np.cumsum(v, axis=0)])
    i = np.arange(n)
    lo = np.maximum(0, (i // c - prev) * c)
    return (cs[i + 1] - cs[lo]) / (i + 1 - lo)[:, None]


def _chunks(n, c):
    return [(a, min(a + c, n)) for a in range(0, n, c)]


def awm_unrolled(qm, km, v, c, lag: int = 2):
    """O_m from the unrolled sum of transition-matrix products.

    With z^t the cumulative per-feature exp-sum through chunk t,
      T_t = diag(z^{t-1}/z^t) - diag(1/z^t) exp(K_t)^T psi(K_t)   (d x d)
      B_t = diag(1/z^t) exp(K_t)^T V_t                           (d x dv)
    the memory is M'_s = sum_{t=1}^{s-1} T_{s-1} ... T_{t+1} B_t (it holds chunks
    1..s-1), and chunk s reads the one holding chunks 1..s-lag: psi(Q_m,s)
    M'_{s+1-lag} (zero for s <= lag). Products are formed explicitly.
    """
    qm, km, v = (np.asarray(a, np.float64) for a in (qm, km, v))
    n, d = km.shape
    dv = v.shape[1]
    ch = _chunks(n, c)
    N = len(ch)
    z = [np.zeros(d)]
    for a, b in ch:
        z.append(z[-1] + np.exp(km[a:b]).sum(axis=0))
    T = {}
    Bm = {}
    for t in range(1, N + 1):
        a, b = ch[t - 1]
        e = np.exp(km[a:b])
        psi = sp_softmax(km[a:b], axis=1)
        inv = np.diag(1.0 / z[t])
        T[t] = np.diag(z[t - 1] / z[t]) - inv @ e.T @ psi
        Bm[t] = inv @ e.T @ v[a:b]

    def mem(s):
        total = np.zeros((d, dv))
        for t in range(1, s):
            prod = np.eye(d)
            for u in range(t + 1, s):
                prod = T[u] @ prod
            total += prod @ Bm[t]
        return total

    out = np.zeros((n, dv))
    for s in range(lag + 1, N + 1):
        a, b = ch[s - 1]
        out[a:b] = sp_softmax(qm[a:b], axis=1) @ mem(s + 1 - lag)
    return out


def awm_no_delta_closed(qm, km, v, c, lag: int = 2):
    """Closed form without the delta correction: linear attention with the
    online-softmax kernel. The state holding chunks 1..u is (sum over their
    tokens of exp(k)^T v) / z^u, row f divided by z^u_f; chunk s reads
    psi(Q_m) times the one with u = s - lag."""
    qm, km, v = (np.asarray(a, np.float64) for a in (qm, km, v))
    n, d = km.shape
    out = np.zeros((n, v.shape[1]))
    ch = _chunks(n, c)
    for s in range(lag + 1, len(ch) + 1):
        end = ch[s - lag - 1][1]  # last token of chunk s - lag
        e = np.exp(km[:end])
        mem = (e.T @ v[:end]) / e.sum(axis=0)[:, None]
        a, b = ch[s - 1]
        out[a:b] = sp_softmax(qm[a:b], axis=1) @ mem
    return out


def awm_const_key_chunk_rows(v, c, lag: int = 2):
    """Closed form when every memory key row is the same vector, one row per chunk.

    Then every row of the state is the same vector, psi(Q_m) M' is that
    vector for any query, and with vbar_t the mean of V over chunk t
    (1-based) the state holding chunks 1..u is
      f(0) = 0, f(1) = vbar_1, f(u) = sum_{t=2}^{u} (t-1) vbar_t / (u (u-1)).
    Chunk s reads f(s - lag) (sliding chunks: lag 2, so chunk 3 reads vbar_1
    and chunk s >= 4 reads sum_{t=2}^{s-2} (t-1) vbar_t / ((s-2)(s-3))).
    Returns [N, dv]: row s-1 is what every query of chunk s reads.
    """
    v = np.asarray(v, np.float64)
    ch = _chunks(v.shape[0], c)
    N = len(ch)
    vbar = np.stack([v[a:b].mean(axis=0) for a, b in ch])        # row t-1 = vbar_t
    t = np.arange(1, N + 1, dtype=np.float64)
    w = np.cumsum((t - 1.0)[:, None] * vbar, axis=0)              # row u-1 = sum_{t<=u} (t-1) vbar_t
    rows = np.zeros((N, v.shape[1]))
    for s in range(lag + 1, N + 1):
        u = s - lag
        rows[s - 1] = vbar[0] if u == 1 else w[u - 1] / (u * (u - 1))
    return rows


def awm_const_key_closed(v, c, lag: int = 2):
    """awm_const_key_chunk_rows expanded to every token row."""
    v = np.asarray(v, np.float64)
    rows = awm_const_key_chunk_rows(v, c, lag)
    out = np.zeros_like(v)
    for s, (a, b) in enumerate(_chunks(v.shape[0], c)):
        out[a:b] = rows[s]
    return out


class ConstKeyStream:
    """Both closed forms of a sequence handed over in segments of whole chunks,
    with all attention logits equal and all memory keys equal: chunk s
    (1-based) reads the window mean (pins.window_mean) plus the constant-key
    state f(s - 2) of awm_const_key_chunk_rows, carried across segments.
    push(v_segment) yields, chunk by chunk, the rows the segment must hold."""

    def __init__(self, c: int):
        self.c = c
        self.prev = None        # the last chunk of v seen (float64)
        self.u = 0              # chunks seen
        self.vbar1 = None
        self.w = {0: 0.0}       # u -> sum_{t<=u} (t-1) vbar_t

    def state(self, u):
        if u <= 0:
            return 0.0
        if u == 1:
            return self.vbar1
        return self.w[u] / (u * (u - 1))

    def push(self, v):
        c = self.c
        n = v.shape[0]
        for a in range(0, n, c):
            cur = np.asarray(v[a:a + c], np.float64)
            before = self.prev
            win = cur if before is None else np.vstack([before, cur])
            off = 0 if before is None else before.shape[0]
            mean = np.cumsum(win, axis=0)[off:] / np.arange(off + 1, off + cur.shape[0] + 1)[:, None]
            s = self.u + 1
            yield mean + self.state(s - 2)
            vbar = cur.mean(axis=0)
            if s == 1:
                self.vbar1 = vbar
            self.w[s] = self.w[s - 1] + (s - 1) * vbar
            self.w.pop(s - 3, None)
            self.prev = cur
            self.u = s
