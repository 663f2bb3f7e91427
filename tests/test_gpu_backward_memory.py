"""GPU tier: the memory part of both backwards (gecko_backward, and the
training pair gecko_forward_train + gecko_backward_saved) against the float64
gradient oracle element by element over long sequences, where the reverse
state scan and the zeta recurrence run tens of steps.

The gradient of the memory reaches a chunk's Z' and V through every later
chunk's readout ([rainbus] "Method steps" (4)-(5): the state S_t enters the
update of S_{t+1} and the readout of chunk t + 2), so the rows of an early
chunk carry the reverse recurrence over the whole sequence. [paperlayer]
Appendix B.1 describes the backward recomputing that recurrence from the
chunk-boundary states; the derivative itself is the plain one.

Cases:

* 64 chunks at c = 64 and at c = 128 (62 memory steps): every row of dZ' and
  dV and all affine gradients, the memory alone and both parts, for both
  backwards;
* the bench configuration (B1 H8, 131072 tokens, c 2048, 62 steps): for two
  heads, every row of the memory's dZ' and dV and its four affine gradients;
  the training pair over both parts on the rows of sampled chunks, against
  the memory oracle over the whole sequence plus the attention oracle on the
  chunk's three-chunk stretch (the attention gradient of chunk s depends on
  chunks s - 1 .. s + 1 only; the loss is a sum, so the gradients add).

Bars as in test_gpu_backward: relative Frobenius and max-relative 1e-2 for
dZ' and dV, the summation bound for the affine gradients.
"""

from __future__ import annotations

import numpy as np
import pytest

from chunked_attention_memory_amd import inputs
from gpu_helpers import announce, gecko, to_numpy
from test_gpu_backward import GRAD_TOL, NAMES, SUM_FLOOR, SUM_TOL, SUMMAND, _check, _errors

from oracle import gecko_grad_oracle as go

pytestmark = pytest.mark.gpu


def _finite(res):
    import torch

    for k, t in res.items():
        assert bool(torch.isfinite(t).all()), k


# the training forward always computes the attention, so the training pair
# runs over both parts only
@pytest.mark.parametrize("n,c,dv", [(4096, 64, 128), (8192, 128, 256)])
@pytest.mark.parametrize("which,saved", [("awm", False), ("both", False), ("both", True)])
def test_memory_backward_64_chunks(n, c, dv, which, saved):
    import torch

    g = gecko()
    parts = g.GECKO_PART_AWM | (g.GECKO_PART_SCA if which == "both" else 0)
    host = inputs.make_inputs(1, 1, n, 128, dv, "bf16", seed=0, tag=520 + c)
    dout = inputs.make_dout(1, 1, n, dv, "bf16", seed=0, tag=520 + c)
    z, v, p = g.to_device_inputs(host)
    do = torch.from_numpy(dout).to(device="cuda", dtype=torch.bfloat16)
    announce(f"memory backward n={n} c={c} dv={dv} parts={parts} saved={saved}")
    if saved:
        _, o_sca, stats = g.gecko_forward_train(z, p, v, c, parts=parts)
        res = g.gecko_backward_saved(z, p, v, do, o_sca, stats, c, parts=parts)
    else:
        res = g.gecko_backward(z, p, v, do, c, parts=parts)
    torch.cuda.synchronize()
    _finite(res)
    got = {k: to_numpy(t) for k, t in res.items()}
    names = ("awm",) if which == "awm" else ("sca", "awm")
    want = go.grad(host["z"].astype(np.float64), host["v"].astype(np.float64), host["params"], c,
                   dout.astype(np.float64), parts=names)
    _check(got, want, names, host["z"].astype(np.float64))
    if which == "awm":
        for k in NAMES[:4]:
            assert np.all(got["d" + k] == 0.0), k


def _affine_ratio(got_h, want, z64, k, tok):
    """Largest |error| / summation bound of one head's affine gradient."""
    src, with_z = SUMMAND[k]
    term = want[src] * (z64 if with_z else 1.0)
    bound = np.abs(term).sum(axis=0)
    bound = bound + SUM_FLOOR * bound.max() + 1e-3 * tok
    return float(np.max(np.abs(got_h - want["d" + k]) / (bound + 1e-30)))


def test_memory_backward_bench_configuration_every_row():
    import torch

    g = gecko()
    B, H, n, c, d, dv = 1, 8, 131072, 2048, 128, 256
    dev = inputs.make_inputs_device(B, H, n, d, dv, "bf16", seed=6, tag=530)
    z, v = dev["z"], dev["v"]
    p = {k: torch.from_numpy(a).cuda() for k, a in dev["params"].items()}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(530)
    do = torch.randn((B, H, n, dv), generator=gen, device="cuda").to(torch.bfloat16)
    announce(f"memory backward, bench configuration n={n} c={c} H={H}")
    mem = g.gecko_backward(z, p, v, do, c, parts=g.GECKO_PART_AWM)
    _, o_sca, stats = g.gecko_forward_train(z, p, v, c)
    both = g.gecko_backward_saved(z, p, v, do, o_sca, stats, c)
    torch.cuda.synchronize()
    _finite(mem)
    _finite(both)
    del o_sca, stats
    N = n // c
    for h in (0, 5):
        zh = z[0, h].float().cpu().numpy().astype(np.float64)
        vh = v[0, h].float().cpu().numpy().astype(np.float64)
        dh = do[0, h].float().cpu().numpy().astype(np.float64)
        want = go.grad_head(zh, vh, dev["params"], h, c, dh, parts=("awm",))
        tok = float(np.abs(want["dv"]).max(axis=1).sum())
        # the memory alone: every row, and its four affine gradients
        for key in ("dz", "dv"):
            fro, mx = _errors(to_numpy(mem[key][0, h]), want[key])
            assert fro <= GRAD_TOL and mx <= GRAD_TOL, ("memory", h, key, fro, mx)
        for k in NAMES[4:]:
            r = _affine_ratio(to_numpy(mem["d" + k][h]), want, zh, k, tok)
            assert r <= SUM_TOL, ("memory", h, k, r)
        for k in NAMES[:4]:
            assert bool((mem["d" + k][h] == 0).all()), k
        # the training pair over both parts: the memory's affine gradients
        # (the attention does not use eta, rho) and the rows of sampled chunks
        for k in NAMES[4:]:
            r = _affine_ratio(to_numpy(both["d" + k][h]), want, zh, k, tok)
            assert r <= SUM_TOL, ("both", h, k, r)
        for s in (1, 2, N // 2, N - 1):
            a, b = (s - 1) * c, min((s + 2) * c, n)
            ph = {k: dev["params"][k][h:h + 1] for k in dev["params"]}
            att = go.grad(zh[a:b][None, None], vh[a:b][None, None], ph, c, dh[a:b][None, None], parts=("sca",))
            for key in ("dz", "dv"):
                w = att[key][0, 0, c:2 * c] + want[key][s * c:(s + 1) * c]
                fro, mx = _errors(to_numpy(both[key][0, h, s * c:(s + 1) * c]), w)
                assert fro <= GRAD_TOL and mx <= GRAD_TOL, ("both", h, s, key, fro, mx)
