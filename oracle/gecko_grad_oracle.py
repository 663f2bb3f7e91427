"""Plain float64 CPU oracle for the gradients of the Gecko per-layer forward
(sliding chunk attention plus adaptive working memory).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py`` may import or call this module. It shares no code with the HIP
library or its binding.

What it computes: for a loss L = sum(dO * O), where O is the layer output of
[rainbus "Method steps" (2)-(5)] and dO a given array, the derivatives of L
with respect to Z', V and the eight affine vectors. The pages define the
forward only; the gradient is the plain derivative of that definition. Here
the forward is written out again with torch float64 tensor operations, in the
pages' order and notation (the same readings R1-R9 as ``gecko_oracle``), and
torch's reverse-mode differentiation takes the derivative. Nothing is blocked,
fused or reassociated: per chunk, the window's logits, the softmax, the
feature softmaxes, z^s, phi^s and the state update M' are formed exactly as
the definition states.

Sources (cited by site and section):

* [rainbus] structured summary on paper.rainbus.top, "Method steps" (2)-(5)
  and "Core method".
* [paperlayer] section-by-section summary on paperlayer.ai, 3.2, 3.3 and
  Appendix A (initial memory states), and Appendix B.1 (training recomputes
  what the backward needs at chunk boundaries rather than storing it; the
  derivative itself is the same).

Pinned in ``tests/test_grad_oracle.py`` against central finite differences of
the independent numpy forward (``gecko_oracle.forward``) and against exact
invariants of the definition.
"""

from __future__ import annotations

import numpy as np
import torch

__all__ = ["AFFINE", "forward_torch_head", "grad_head", "grad", "lse_head"]

# the eight per-head affine vectors, in the order the gradients are returned
AFFINE = ("kappa_q", "nu_q", "kappa_k", "nu_k", "eta_q", "rho_q", "eta_k", "rho_k")


def _t(x):
    return torch.as_tensor(np.asarray(x, np.float64), dtype=torch.float64)


def forward_torch_head(z, v, p, c: int, parts=("sca", "awm"), chunkwise: bool = False,
                       no_delta: bool = False, keep=None):
    """O of one head as torch float64 tensors: z [n, d], v [n, dv], p maps the
    eight names to [d] tensors. ``parts`` selects O_SCA, O_m or their sum
    ([rainbus "Method steps" (5)], R8). If ``keep`` is a dict it receives the
    derived Q, K, Q_m, K_m tensors (keys "q", "k", "qm", "km")."""
    n, _ = z.shape
    dv = v.shape[1]
    out = torch.zeros((n, dv), dtype=torch.float64)
    starts = list(range(0, n, c))
    if "sca" in parts:
        # [rainbus "Method steps" (2)]: Q and K by the per-feature affine maps
        q = p["kappa_q"] * z + p["nu_q"]
        k = p["kappa_k"] * z + p["nu_k"]
        if keep is not None:
            keep["q"], keep["k"] = q, k
        rows = []
        for a in starts:
            b = min(a + c, n)
            k0 = max(0, a - c) if not chunkwise else a  # R4, R9
            logits = q[a:b] @ k[k0:b].T                 # R3: no 1/sqrt(d)
            qi = torch.arange(a, b)[:, None]
            kj = torch.arange(k0, b)[None, :]
            logits = logits.masked_fill(kj > qi, float("-inf"))  # R2
            rows.append(torch.softmax(logits, dim=1) @ v[k0:b])
        out = out + torch.cat(rows)
    if "awm" in parts:
        # [rainbus "Method steps" (4)-(5)], "Core method"; R1, R5-R7, R9
        qm = p["eta_q"] * z + p["rho_q"]
        km = p["eta_k"] * z + p["rho_k"]
        if keep is not None:
            keep["qm"], keep["km"] = qm, km
        d = z.shape[1]
        z_prev = torch.zeros(d, dtype=torch.float64)
        mem_prev = torch.zeros((d, dv), dtype=torch.float64)  # M'_{s-1}
        mem_cur = torch.zeros((d, dv), dtype=torch.float64)   # M'_s
        rows = []
        for a in starts:
            b = min(a + c, n)
            read = mem_cur if chunkwise else mem_prev
            rows.append(torch.softmax(qm[a:b], dim=1) @ read)
            ek = torch.exp(km[a:b])
            z_cur = z_prev + ek.sum(dim=0)
            phi = ek / z_cur
            resid = v[a:b] if no_delta else v[a:b] - torch.softmax(km[a:b], dim=1) @ mem_cur
            mem_next = (z_prev / z_cur)[:, None] * mem_cur + phi.T @ resid
            mem_prev, mem_cur, z_prev = mem_cur, mem_next, z_cur
        out = out + torch.cat(rows)
    return out


def grad_head(z, v, p: dict, h: int, c: int, dout, parts=("sca", "awm"), chunkwise: bool = False,
              no_delta: bool = False) -> dict:
    """Gradients of L = sum(dout * O) for head h of one batch row.

    Returns float64 numpy arrays: ``dz`` [n, d], ``dv`` [n, dv], one [d]
    vector per affine name ("d" + name), and the per-token gradients with
    respect to the derived Q, K, Q_m, K_m ("dq", "dk", "dqm", "dkm", [n, d];
    zero for a part not selected). The affine gradients are the sums over
    tokens of Z' times (or just) these; dz is their combination through the
    scales."""
    zt = _t(z).requires_grad_(True)
    vt = _t(v).requires_grad_(True)
    pt = {k: _t(p[k][h]).requires_grad_(True) for k in AFFINE}
    keep = {}
    o = forward_torch_head(zt, vt, pt, c, parts=parts, chunkwise=chunkwise, no_delta=no_delta, keep=keep)
    loss = (o * _t(dout)).sum()
    names = [k for k in ("q", "k", "qm", "km") if k in keep]
    leaves = [zt, vt] + [pt[k] for k in AFFINE] + [keep[k] for k in names]
    grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    # a part that never reaches the output (the memory of a sequence of at
    # most lag chunks) leaves its inputs unused: their gradient is zero
    res = {"dz": np.zeros(z.shape) if grads[0] is None else grads[0].numpy(),
           "dv": np.zeros(v.shape) if grads[1] is None else grads[1].numpy()}
    for k, gk in zip(AFFINE, grads[2:2 + len(AFFINE)]):
        res["d" + k] = np.zeros(z.shape[1]) if gk is None else gk.numpy()
    for k in ("q", "k", "qm", "km"):
        res["d" + k] = np.zeros(z.shape)
    for k, gk in zip(names, grads[2 + len(AFFINE):]):
        if gk is not None:
            res["d" + k] = gk.numpy()
    return res


def grad(z, v, p: dict, c: int, dout, parts=("sca", "awm"), chunkwise: bool = False,
         no_delta: bool = False) -> dict:
    """Whole-tensor gradients: z [B, H, n, d], v and dout [B, H, n, dv].

    ``dz`` [B, H, n, d], ``dv`` [B, H, n, dv] and the per-token ``dq``,
    ``dk``, ``dqm``, ``dkm`` [B, H, n, d]; each affine gradient [H, d] is
    summed over the batch (the vectors are shared by the rows)."""
    B, H, n, d = z.shape
    dv = v.shape[3]
    res = {"dz": np.empty((B, H, n, d)), "dv": np.empty((B, H, n, dv))}
    for k in ("q", "k", "qm", "km"):
        res["d" + k] = np.empty((B, H, n, d))
    for k in AFFINE:
        res["d" + k] = np.zeros((H, d))
    for b in range(B):
        for h in range(H):
            r = grad_head(z[b, h], v[b, h], p, h, c, dout[b, h], parts=parts, chunkwise=chunkwise,
                          no_delta=no_delta)
            for k in ("dz", "dv", "dq", "dk", "dqm", "dkm"):
                res[k][b, h] = r[k]
            for k in AFFINE:
                res["d" + k][h] += r["d" + k]
    return res


def lse_head(z, p: dict, h: int, c: int, chunkwise: bool = False) -> np.ndarray:
    """Natural-log log-sum-exp of each query row's attention logits q_i . k_j
    over its window ([rainbus "Method steps" (3)], R2-R4, R9): the softmax
    normaliser that a backward pass reuses. float64 [n]."""
    z = np.asarray(z, np.float64)
    n = z.shape[0]
    q = z * p["kappa_q"][h] + p["nu_q"][h]
    k = z * p["kappa_k"][h] + p["nu_k"][h]
    out = np.empty(n)
    for a in range(0, n, c):
        b = min(a + c, n)
        k0 = a if chunkwise else max(0, a - c)
        logits = q[a:b] @ k[k0:b].T
        logits = np.where(np.arange(k0, b)[None, :] <= np.arange(a, b)[:, None], logits, -np.inf)
        m = logits.max(axis=1)
        out[a:b] = m + np.log(np.exp(logits - m[:, None]).sum(axis=1))
    return out
