"""Plain fp64 CPU oracle for the Gecko per-layer forward: sliding chunk attention
(SCA) plus adaptive working memory (AWM).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path (the HIP library and its Python binding) never touches it and it
never touches the product path: the two share no code, no constants and no
helpers.

Sources (the pages this follows; cited by site and section):

* [rainbus] "Gecko: An Efficient Neural Architecture Inherently Processing
  Sequences with Arbitrary Lengths", structured summary on paper.rainbus.top.
  Sections used: "Core method" (the position-aware online-softmax kernel, the
  feature-softmax query map and the normaliser identity) and "Method steps"
  (steps (2)-(5): the affine derivations, SCA, the memory update and the
  readout).
* [paperlayer] the same paper's section-by-section summary on paperlayer.ai.
  Sections used: 3.2 "Sliding Chunk Attention", 3.3 "Adaptive Working
  Memory" (chunk-by-chunk updates, normaliser fixed to one) and Appendix A
  (the initial states of the memory).
* [chatpaper] the abstract on chatpaper.ai (sequences of arbitrary length,
  processed in one pass; used by ``HeadStream``).

Readings taken where the pages are silent or garbled (each is repeated where it
is used):

* R1 memory update: the printed update lost its parentheses; the delta rule the
  appendix names, with shapes that type-check, is
  ``M'_s = (z^{s-2}/z^{s-1}) * M'_{s-1} + phi^{s-1}(K_{s-1})^T (V_{s-1} - psi(K_{s-1}) M'_{s-1})``.
* R2 causality inside a chunk: key j is visible to query i iff j <= i; the whole
  previous chunk is visible.
* R3 attention logits carry no 1/sqrt(d) scale (none is printed in step (3)).
* R4 the first chunk attends to itself only; the last chunk may be partial;
  c >= n gives one chunk.
* R5 inside AWM, K means the memory key K_m and Q the memory query Q_m; V is the
  same V as in SCA.
* R6 the ratio z^{s-2}/z^{s-1} scales row f (key feature f) of M'.
* R7 z^0 = 0 (empty sum), so the ratio is 0 on the first update; M'_0 (read by
  chunk 1) is taken as 0 like M'_1.
* R8 the output is exactly O_SCA + O_m (no gate, no projection).
* R9 chunk-wise variant (the ablation the pages set SCA and AWM against:
  Megalodon's chunk-wise attention, [paperlayer 2.3], and the memory without
  sliding chunks, [paperlayer Appendix A]): attention stays inside the
  current chunk (causal), and the memory is read one chunk earlier: with
  M_0 = 0 and the same update, chunk s reads the state holding chunks
  1..s-1 (the sliding form reads the one holding chunks 1..s-2).

Everything is evaluated in float64 on the exact (already rounded) input values
the GPU receives. Inputs may be float32 (bf16-exact values are exact in
float32); they are upcast per chunk so that long sequences stream.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "chunk_ranges",
    "affine",
    "feature_softmax",
    "sca_chunk",
    "sca_head",
    "awm_head",
    "forward_head",
    "forward",
    "HeadStream",
]


def chunk_ranges(n: int, c: int) -> list[tuple[int, int]]:
    """Token ranges [start, end) of chunks 1..N, N = ceil(n / c).

    [rainbus "Method steps" (3)]: the sequence is cut into chunks of c tokens;
    R4: the last chunk holds the remainder.
    """
    if n < 0 or c < 1:
        raise ValueError("need n >= 0 and c >= 1")
    return [(s, min(s + c, n)) for s in range(0, n, c)]


def affine(z: np.ndarray, scale: np.ndarray, shift: np.ndarray) -> np.ndarray:
    """Per-feature affine map scale * z + shift, in float64.

    [rainbus "Method steps" (2)] derives Q and K from Z' this way with
    (kappa_q, nu_q) and (kappa_k, nu_k); step (4) derives Q_m and K_m with
    (eta_q, rho_q) and (eta_k, rho_k).
    """
    z = np.asarray(z, dtype=np.float64)
    return z * np.asarray(scale, dtype=np.float64) + np.asarray(shift, dtype=np.float64)


def feature_softmax(x: np.ndarray) -> np.ndarray:
    """psi: softmax of each row over the feature axis.

    [rainbus "Core method"]: the query-side map normalises exp(q) by the sum
    of exp over the features of the same row.
    """
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def sca_chunk(q_rows: np.ndarray, k_win: np.ndarray, v_win: np.ndarray,
              query_pos: np.ndarray, key_pos: np.ndarray) -> np.ndarray:
    """Softmax attention of the queries of one chunk over its window.

    [rainbus "Method steps" (3)]: chunk s attends to the concatenated keys and
    values of chunks s-1 and s. R2: key j is visible to query i iff j <= i
    (positions are absolute token indices). R3: logits are plain dot products.
    """
    logits = np.asarray(q_rows, np.float64) @ np.asarray(k_win, np.float64).T
    visible = key_pos[None, :] <= query_pos[:, None]
    logits = np.where(visible, logits, -np.inf)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return w @ np.asarray(v_win, np.float64)


def _window(n: int, c: int, s: int, sliding: bool = True) -> tuple[int, int, int]:
    """(first key, first query, end) of chunk s (0-based) and its window.

    R4: chunk 0 has no previous chunk; [paperlayer 3.2]: the window of chunk s
    is the previous chunk plus the current one. R9: without sliding, the
    current chunk only.
    """
    q0 = s * c
    q1 = min(q0 + c, n)
    return (max(0, q0 - c) if sliding else q0), q0, q1


def sca_head(z, v, kappa_q, nu_q, kappa_k, nu_k, c: int, chunks=None, sliding: bool = True) -> np.ndarray:
    """O_SCA for one head: z [n, d], v [n, dv], affine vectors [d].

    Returns float64 [n, dv]; or, if ``chunks`` (0-based chunk indices) is
    given, a dict mapping each of those chunks to its rows. ``sliding=False``
    is the chunk-wise attention of R9.
    """
    n = z.shape[0]
    out = np.empty((n, v.shape[1])) if chunks is None else {}
    nchunks = len(chunk_ranges(n, c))
    for s in (range(nchunks) if chunks is None else chunks):
        k0, q0, q1 = _window(n, c, s, sliding)
        q = affine(z[q0:q1], kappa_q, nu_q)
        k = affine(z[k0:q1], kappa_k, nu_k)
        rows = sca_chunk(q, k, v[k0:q1], np.arange(q0, q1), np.arange(k0, q1))
        if chunks is None:
            out[q0:q1] = rows
        else:
            out[s] = rows
    return out


def awm_head(z, v, eta_q, rho_q, eta_k, rho_k, c: int, no_delta: bool = False,
             trace=None, readout_chunks=None, lag: int = 2):
    """O_m for one head: z [n, d], v [n, dv], affine vectors [d].

    Follows [rainbus "Method steps" (4)-(5)] and [rainbus "Core method"],
    chunk by chunk as [paperlayer 3.3] states:

    * K_m, Q_m come from Z' by the (eta, rho) affine map (step (4), R5).
    * z^s is the per-feature sum of exp(k) over every token of chunks 1..s
      ("Core method"); z^0 = 0 (R7).
    * phi^s(k) = exp(k) / z^s, per feature ("Core method").
    * psi is the feature softmax ("Core method").
    * M'_1 = 0 ([paperlayer Appendix A]); M'_0 = 0 (R7).
    * for s >= 2: M'_s = (z^{s-2}/z^{s-1}) * M'_{s-1}
                   + phi^{s-1}(K_{s-1})^T (V_{s-1} - psi(K_{s-1}) M'_{s-1})   (R1, R6).
      With ``no_delta`` the bracket is V_{s-1} alone (plain linear attention
      with the online-softmax kernel; a test variant, not the method).
    * readout of chunk s: O_m,s = psi(Q_m,s) M'_{s-1} (step (5)); no
      denominator, since the normaliser is identically one ("Core method",
      [paperlayer 3.3]).

    ``lag=1`` is the memory without sliding chunks (R9): chunk s reads the
    state holding chunks 1..s-1 (M_{s-1} with M_0 = 0) instead of M'_{s-1}.

    ``trace``, if a list, receives one dict per chunk s (1-based) with the
    float64 z^s, phi^s(K_s) and the state used by the readout.

    Returns float64 [n, dv]; or, if ``readout_chunks`` (0-based chunk indices)
    is given, a dict mapping each of those chunks to its rows (the memory
    still passes through every chunk; only the readout is restricted, which
    keeps long sequences within host memory).
    """
    n, d = z.shape
    dv = v.shape[1]
    wanted = None if readout_chunks is None else set(readout_chunks)
    out = np.zeros((n, dv)) if wanted is None else {}
    ranges = chunk_ranges(n, c)
    z_prev = np.zeros(d)              # z^{s-1}
    mem_prev = np.zeros((d, dv))      # M'_{s-1}
    mem_cur = np.zeros((d, dv))       # M'_s
    if lag not in (1, 2):
        raise ValueError("lag is 2 (sliding chunks) or 1 (without)")
    for s, (a, b) in enumerate(ranges, start=1):
        # readout of chunk s from M'_{s-1} (lag 2), or from the state holding
        # chunks 1..s-1 (lag 1), which is M'_s of the same update
        read = mem_prev if lag == 2 else mem_cur
        if wanted is None or s - 1 in wanted:
            rows = feature_softmax(affine(z[a:b], eta_q, rho_q)) @ read
            if wanted is None:
                out[a:b] = rows
            else:
                out[s - 1] = rows
        # chunk s enters the memory: z^s, then M'_{s+1} from M'_s
        km = affine(z[a:b], eta_k, rho_k)
        ek = np.exp(km)
        z_cur = z_prev + ek.sum(axis=0)
        phi = ek / z_cur
        if no_delta:
            resid = np.asarray(v[a:b], np.float64)
        else:
            resid = np.asarray(v[a:b], np.float64) - feature_softmax(km) @ mem_cur
        mem_next = (z_prev / z_cur)[:, None] * mem_cur + phi.T @ resid
        if trace is not None:
            trace.append({"s": s, "z": z_cur.copy(), "phi": phi, "mem_read": read.copy()})
        mem_prev, mem_cur = mem_cur, mem_next
        z_prev = z_cur
    return out


def forward_head(z, v, p: dict, h: int, c: int, no_delta: bool = False,
                 sca_chunks=None, chunkwise: bool = False) -> dict:
    """O = O_SCA + O_m for head h of one batch row ([rainbus "Method steps" (5)], R8).

    ``p`` maps the eight affine-vector names to [H, d] arrays. With
    ``sca_chunks`` (0-based) every entry is a dict of those chunks' rows.
    ``chunkwise`` selects the variant of R9.
    """
    o_sca = sca_head(z, v, p["kappa_q"][h], p["nu_q"][h], p["kappa_k"][h], p["nu_k"][h],
                     c, chunks=sca_chunks, sliding=not chunkwise)
    o_m = awm_head(z, v, p["eta_q"][h], p["rho_q"][h], p["eta_k"][h], p["rho_k"][h],
                   c, no_delta=no_delta, readout_chunks=sca_chunks, lag=1 if chunkwise else 2)
    if sca_chunks is None:
        return {"o_sca": o_sca, "o_m": o_m, "o": o_sca + o_m}
    return {"o_sca": o_sca, "o_m": o_m, "o": {s: o_sca[s] + o_m[s] for s in sca_chunks}}


def forward(z, v, p: dict, c: int, no_delta: bool = False, chunkwise: bool = False) -> dict:
    """Whole-tensor forward: z [B, H, n, d], v [B, H, n, dv]; float64 outputs [B, H, n, dv]."""
    B, H, n, _ = z.shape
    dv = v.shape[3]
    res = {key: np.empty((B, H, n, dv)) for key in ("o_sca", "o_m", "o")}
    for b in range(B):
        for h in range(H):
            r = forward_head(z[b, h], v[b, h], p, h, c, no_delta=no_delta, chunkwise=chunkwise)
            for key in res:
                res[key][b, h] = r[key]
    return res


class HeadStream:
    """Forward of one head over a sequence handed over in consecutive segments.

    Gecko is built to run on sequences of any length ([chatpaper] abstract;
    [paperlayer 3.3]: the memory is updated chunk by chunk and carries what
    the attention window no longer sees). Pushing the segments of a sequence
    one after another gives exactly the rows that one ``forward_head`` call
    on the whole sequence gives. What has to be carried from one segment to
    the next follows from the definitions in ``sca_head`` and ``awm_head``:

    * SCA: the rows of the last chunk (the previous chunk of the next one);
    * AWM: z^{s-1}, M'_{s-1} and M'_s, where s is the next chunk (1-based).

    Chunks are counted from the start of the sequence, so every segment but
    the last must hold a whole number of chunks; a push after a segment that
    ended inside a chunk raises ValueError.
    """

    def __init__(self, p: dict, h: int, c: int, no_delta: bool = False):
        if c < 1:
            raise ValueError("need c >= 1")
        self.p, self.h, self.c, self.no_delta = p, h, c, no_delta
        self.pos = 0            # tokens pushed so far
        self.prev = None        # (z rows, v rows) of the last chunk pushed
        self.z_prev = None      # z^{s-1}
        self.mem_prev = None    # M'_{s-1}
        self.mem_cur = None     # M'_s

    def push(self, z, v) -> dict:
        """Rows of this segment: dict of float64 ``o_sca``, ``o_m``, ``o`` [len(z), dv]."""
        if self.pos % self.c:
            raise ValueError("an earlier segment ended inside a chunk")
        p, h, c = self.p, self.h, self.c
        z = np.asarray(z, np.float64)
        v = np.asarray(v, np.float64)
        n, d = z.shape
        dv = v.shape[1]
        if self.mem_cur is None:
            self.z_prev = np.zeros(d)
            self.mem_prev = np.zeros((d, dv))
            self.mem_cur = np.zeros((d, dv))
        o_sca = np.empty((n, dv))
        o_m = np.empty((n, dv))
        for a, b in chunk_ranges(n, c):
            # SCA over [previous chunk; this chunk], positions absolute
            # ([rainbus "Method steps" (3)], R2-R4)
            if a > 0:
                pz, pv = z[a - c:a], v[a - c:a]
            elif self.prev is not None:
                pz, pv = self.prev
            else:
                pz, pv = z[:0], v[:0]
            g0 = self.pos + a
            kz = np.concatenate([pz, z[a:b]])
            kv = np.concatenate([pv, v[a:b]])
            o_sca[a:b] = sca_chunk(affine(z[a:b], p["kappa_q"][h], p["nu_q"][h]),
                                   affine(kz, p["kappa_k"][h], p["nu_k"][h]), kv,
                                   np.arange(g0, g0 + b - a), np.arange(g0 - len(pz), g0 + b - a))
            # readout from M'_{s-1}, then chunk s enters the memory (as in awm_head)
            o_m[a:b] = feature_softmax(affine(z[a:b], p["eta_q"][h], p["rho_q"][h])) @ self.mem_prev
            km = affine(z[a:b], p["eta_k"][h], p["rho_k"][h])
            ek = np.exp(km)
            z_cur = self.z_prev + ek.sum(axis=0)
            resid = v[a:b] if self.no_delta else v[a:b] - feature_softmax(km) @ self.mem_cur
            mem_next = (self.z_prev / z_cur)[:, None] * self.mem_cur + (ek / z_cur).T @ resid
            self.mem_prev, self.mem_cur, self.z_prev = self.mem_cur, mem_next, z_cur
        last = chunk_ranges(n, c)[-1][0] if n else 0
        self.prev = (z[last:], v[last:])
        self.pos += n
        return {"o_sca": o_sca, "o_m": o_m, "o": o_sca + o_m}
