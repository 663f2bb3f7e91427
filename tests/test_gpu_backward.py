"""GPU tier: the backward (gecko_backward through the C ABI) and the forward's
log-sum-exp output (gecko_forward_lse) against the float64 gradient oracle on
the same seeded inputs.

Bar (bf16 inputs, fp32 accumulation). For dZ' and dV: relative Frobenius
error ||y - x|| / ||x|| <= 1e-2 and max-relative error
max |y - x| / max |x| <= 1e-2 over each tensor. Gradients spread over orders
of magnitude across rows (the first rows of a sequence see few keys, a
peaked softmax concentrates on few entries), so the forward's
max-error-over-rms measure would set the error of the largest rows against
the size of the typical one. Each product rounds its operands to bf16
(2^-9 relative) and accumulates in fp32; the observed errors are 0.2-0.5% of
the largest entry. Each affine-vector gradient is a sum over (batch, token)
of a per-token term (Z' dQ, dQ, ..., Z' dK_m, dK_m); its bar is the error
bound of such a sum, |y - x| <= 2e-2 * (sum of |term| + 1e-3 * its largest
value over the vector) per entry (several of these sums nearly cancel: d nu_k
vanishes exactly and d rho_k does without the delta term, so a bar relative
to the sum itself could not be met by any rounding of the terms; the floor
covers entries whose every term vanishes, such as a feature that shifts all
logits of a row alike).
Where one of dZ', dV vanishes identically (a single token: the softmax over
one key has zero derivative), its error is measured against 1e-3 of the other
gradient's norm and largest entry (both scale as |dO| |v| for L2-normalised Z'
and O(1) affine vectors), so that float32 rounding of an exact zero passes;
likewise each affine bound has 1e-3 of the per-head sum over tokens of the
largest |dL/dV| entry added.
The saved log-sum-exp is checked against the oracle's to 2e-2 absolute (the
logits themselves are formed from bf16-rounded scaled queries), and the
forward output of gecko_forward_lse is bit-identical to gecko_sca_awm_forward.
"""

from __future__ import annotations

import numpy as np
import pytest

from chunked_attention_memory_amd import inputs
from gpu_helpers import announce, gecko, to_numpy

import oracle
from oracle import gecko_grad_oracle as go

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-2
NAMES = go.AFFINE


def _device(host, dout, out_dtype):
    import torch

    g = gecko()
    z, v, p = g.to_device_inputs(host)
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    return z, v, p, torch.from_numpy(dout).to(device="cuda", dtype=odt)


def _run(host, dout, c, parts, flags=0, out_dtype="bf16"):
    import torch

    g = gecko()
    z, v, p, do = _device(host, dout, out_dtype)
    announce(f"backward B,H,n,d,dv={tuple(z.shape)}+{v.shape[3]} c={c} parts={parts} flags={flags} out={out_dtype}")
    res = g.gecko_backward(z, p, v, do, c, parts=parts, flags=flags)
    torch.cuda.synchronize()
    return {k: to_numpy(t) for k, t in res.items()}


def _rms(x):
    return float(np.sqrt(np.mean(np.asarray(x, np.float64) ** 2)))


def _errors(got, want, floor_fro=1e-30, floor_max=1e-30):
    got = np.asarray(got, np.float64).ravel()
    want = np.asarray(want, np.float64).ravel()
    fro = float(np.linalg.norm(got - want)) / max(float(np.linalg.norm(want)), floor_fro)
    mx = float(np.max(np.abs(got - want))) / max(float(np.max(np.abs(want))), floor_max)
    return fro, mx


SUMMAND = {"kappa_q": ("dq", True), "nu_q": ("dq", False), "kappa_k": ("dk", True), "nu_k": ("dk", False),
           "eta_q": ("dqm", True), "rho_q": ("dqm", False), "eta_k": ("dkm", True), "rho_k": ("dkm", False)}
SUM_TOL = 2e-2
SUM_FLOOR = 1e-3


def _check(got, want, parts_names, z):
    for key, other in (("dz", "dv"), ("dv", "dz")):
        # a gradient that vanishes identically (one token: a softmax over a
        # single key has zero derivative) is held to 1e-3 of the other one's
        # size (both scale as |dO| |v| here)
        o = np.asarray(want[other], np.float64)
        fro, mx = _errors(got[key], want[key], 1e-3 * float(np.linalg.norm(o)), 1e-3 * float(np.max(np.abs(o))))
        assert fro <= GRAD_TOL and mx <= GRAD_TOL, (key, fro, mx)
    # per head: the sum over tokens of the largest |dL/dV| entry, the scale of
    # a per-token term where every term of a sum vanishes (one token)
    tok = np.abs(np.asarray(want["dv"], np.float64)).max(axis=3).sum(axis=(0, 2))[:, None]
    for part in parts_names:
        for k in (NAMES[:4] if part == "sca" else NAMES[4:]):
            src, with_z = SUMMAND[k]
            term = want[src] * (z if with_z else 1.0)
            bound = np.abs(term).sum(axis=(0, 2))  # [H, d]
            bound = bound + SUM_FLOOR * bound.max() + 1e-3 * tok
            ratio = float(np.max(np.abs(got["d" + k] - want["d" + k]) / (bound + 1e-30)))
            assert ratio <= SUM_TOL, ("d" + k, ratio)


def _case(B, H, n, dv, c, parts, flags=0, out_dtype="bf16", sharp=1.0, tag=300):
    g = gecko()
    host = inputs.make_inputs(B, H, n, 128, dv, "bf16", seed=0, tag=tag)
    if sharp != 1.0:
        host["params"] = inputs.sharpen(host["params"], sharp)
    dout = inputs.make_dout(B, H, n, dv, out_dtype, seed=0, tag=tag)
    got = _run(host, dout, c, parts, flags, out_dtype)
    names = (("sca",) if parts & g.GECKO_PART_SCA else ()) + (("awm",) if parts & g.GECKO_PART_AWM else ())
    want = go.grad(host["z"].astype(np.float64), host["v"].astype(np.float64), host["params"], c,
                   dout.astype(np.float64), parts=names, chunkwise=bool(flags & g.GECKO_CHUNKWISE),
                   no_delta=bool(flags & g.GECKO_AWM_NO_DELTA))
    _check(got, want, names, host["z"].astype(np.float64))
    # the vectors of a part not selected get zero gradients
    for part in ("sca", "awm"):
        if part not in names:
            for k in (NAMES[:4] if part == "sca" else NAMES[4:]):
                assert np.all(got["d" + k] == 0.0), k


@pytest.mark.parametrize("B,H,n,dv,c", [
    (1, 2, 700, 256, 128),   # 6 chunks, ragged tail
    (2, 1, 520, 128, 128),   # dv 128, batch 2
    (1, 1, 600, 256, 96),    # chunk length not a multiple of the 64-row tiles
    (1, 1, 300, 256, 1000),  # one chunk (c > n): causal attention, no memory read
    (1, 1, 65, 256, 64),     # two chunks, one-token tail
    (1, 1, 1, 256, 64),      # a single token
    (2, 2, 256, 256, 128),   # exactly two chunks: the memory never reaches the output
    (2, 3, 333, 128, 64),    # batch and heads together, ragged tail
])
def test_backward_both_parts(B, H, n, dv, c):
    g = gecko()
    _case(B, H, n, dv, c, g.GECKO_PART_SCA | g.GECKO_PART_AWM)


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_backward_attention_only(out_dtype):
    g = gecko()
    _case(1, 2, 640, 256, 128, g.GECKO_PART_SCA, out_dtype=out_dtype, sharp=3.0, tag=301)


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_backward_memory_only(out_dtype):
    g = gecko()
    _case(1, 2, 900, 256, 128, g.GECKO_PART_AWM, out_dtype=out_dtype, sharp=2.0, tag=302)


def test_backward_variants():
    g = gecko()
    _case(1, 1, 700, 256, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, flags=g.GECKO_AWM_NO_DELTA, tag=303)
    _case(1, 1, 700, 256, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, flags=g.GECKO_CHUNKWISE, tag=304)
    _case(1, 1, 500, 128, 64, g.GECKO_PART_AWM, flags=g.GECKO_CHUNKWISE | g.GECKO_AWM_NO_DELTA, tag=305)
    # chunkwise over one chunk: no memory read, attention within the chunk only
    _case(1, 2, 128, 256, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, flags=g.GECKO_CHUNKWISE, tag=310)


def test_backward_sharp_logits():
    g = gecko()
    _case(1, 1, 800, 256, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, sharp=4.0, tag=306)


def test_forward_lse_matches_forward_and_oracle():
    import torch

    g = gecko()
    host = inputs.make_inputs(1, 2, 700, 128, 256, "bf16", seed=0, tag=307)
    host["params"] = inputs.sharpen(host["params"], 3.0)
    z, v, p = g.to_device_inputs(host)
    for flags in (0, g.GECKO_CHUNKWISE):
        announce(f"forward_lse flags={flags}")
        out, lse = g.gecko_forward_lse(z, p, v, 128, flags=flags)
        ref = g.gecko_sca_awm_forward(z, p, v, 128, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        got = to_numpy(lse)
        for h in range(2):
            want = go.lse_head(host["z"][0, h].astype(np.float64), host["params"], h, 128,
                               chunkwise=bool(flags & g.GECKO_CHUNKWISE))
            assert np.max(np.abs(got[0, h] - want)) <= 2e-2
        # attention only: the same lse
        out2, lse2 = g.gecko_forward_lse(z, p, v, 128, parts=g.GECKO_PART_SCA, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(lse2, lse)
        if not flags:
            assert torch.equal(out2, g.gecko_sca_forward(z, p, v, 128))


def test_backward_is_deterministic_and_repeatable():
    import torch

    g = gecko()
    host = inputs.make_inputs(1, 2, 512, 128, 256, "bf16", seed=1, tag=308)
    dout = inputs.make_dout(1, 2, 512, 256, "bf16", seed=1, tag=308)
    z, v, p, do = _device(host, dout, "bf16")
    a = g.gecko_backward(z, p, v, do, 128)
    b = g.gecko_backward(z, p, v, do, 128)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_value_gradient_identity_at_scale():
    """O is linear in V, so <V, dL/dV> = L = <dO, O> exactly in real arithmetic;
    at 32K tokens (16 chunks of 2048) the two sides agree to the bf16 bar."""
    import torch

    g = gecko()
    n, c = 32768, 2048
    dev = inputs.make_inputs_device(1, 2, n, 128, 256, "bf16", seed=2, tag=309)
    z, v = dev["z"], dev["v"]
    p = {k: torch.from_numpy(a).cuda() for k, a in dev["params"].items()}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(309)
    do = torch.randn((1, 2, n, 256), generator=gen, device="cuda").to(torch.bfloat16)
    announce(f"value-gradient identity n={n} c={c}")
    out = g.gecko_sca_awm_forward(z, p, v, c, out_dtype=torch.float32)
    res = g.gecko_backward(z, p, v, do.float(), c)
    torch.cuda.synchronize()
    lhs = float((v.double() * res["dv"].double()).sum())
    rhs = float((do.double() * out.double()).sum())
    scale = float(v.double().abs().mul(res["dv"].double().abs()).sum())
    assert abs(lhs - rhs) <= 1e-2 * scale, (lhs, rhs, scale)
    assert torch.isfinite(res["dz"]).all() and torch.isfinite(res["dv"]).all()


def test_backward_logits_past_the_exponent_range():
    """Every logit carries a large part shared by all keys (Z' feature 0 set
    to 3 and kappa_q, kappa_k = 8 there: about 830 in log2 units), so 2^s
    overflows float32 and the attention statistics take the running-maximum
    path, while the softmax over the varying parts stays unsaturated."""
    g = gecko()
    host = inputs.make_inputs(1, 1, 300, 128, 256, "bf16", seed=0, tag=310)
    host["z"][..., 0] = 3.0
    for k in ("kappa_q", "kappa_k"):
        host["params"][k][:, 0] = 8.0
    dout = inputs.make_dout(1, 1, 300, 256, "bf16", seed=0, tag=310)
    got = _run(host, dout, 128, g.GECKO_PART_SCA)
    want = go.grad(host["z"].astype(np.float64), host["v"].astype(np.float64), host["params"], 128,
                   dout.astype(np.float64), parts=("sca",))
    _check(got, want, ("sca",), host["z"].astype(np.float64))


def test_full_size_attention_gradients_on_sampled_chunks():
    """The bench configuration (B1 H8, 131072 tokens, c 2048). The attention
    gradients of chunk s depend on chunks s-1, s, s+1 only (its queries see
    chunks s-1 and s, its keys are seen by chunks s and s+1), so the oracle
    differentiates that three-chunk stretch alone and its dZ' and dV rows of
    chunk s are compared, for chunks 1 and 40 of two heads."""
    import torch

    g = gecko()
    B, H, n, c, d, dv = 1, 8, 131072, 2048, 128, 256
    dev = inputs.make_inputs_device(B, H, n, d, dv, "bf16", seed=3, tag=311)
    z, v = dev["z"], dev["v"]
    p = {k: torch.from_numpy(a).cuda() for k, a in dev["params"].items()}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(311)
    do = torch.randn((B, H, n, dv), generator=gen, device="cuda").to(torch.bfloat16)
    announce(f"full-size attention backward n={n} c={c} H={H}")
    res = g.gecko_backward(z, p, v, do, c, parts=g.GECKO_PART_SCA)
    torch.cuda.synchronize()
    for s, h in ((1, 0), (40, 5)):
        a, b = (s - 1) * c, (s + 2) * c
        zs = z[0, h, a:b].float().cpu().numpy().astype(np.float64)[None, None]
        vs = v[0, h, a:b].float().cpu().numpy().astype(np.float64)[None, None]
        ds = do[0, h, a:b].float().cpu().numpy().astype(np.float64)[None, None]
        ph = {k: dev["params"][k][h:h + 1] for k in dev["params"]}
        want = go.grad(zs, vs, ph, c, ds, parts=("sca",))
        for key in ("dz", "dv"):
            got = to_numpy(res[key][0, h, s * c:(s + 1) * c])
            fro, mx = _errors(got, want[key][0, 0, c:2 * c])
            assert fro <= GRAD_TOL and mx <= GRAD_TOL, (s, h, key, fro, mx)


def test_full_size_value_gradient_identity():
    """Both parts at the bench configuration: <V, dL/dV> = <dO, O> (O is
    linear in V) to 1e-2 of the sum of |terms|."""
    import torch

    g = gecko()
    B, H, n, c, d, dv = 1, 8, 131072, 2048, 128, 256
    dev = inputs.make_inputs_device(B, H, n, d, dv, "bf16", seed=4, tag=312)
    z, v = dev["z"], dev["v"]
    p = {k: torch.from_numpy(a).cuda() for k, a in dev["params"].items()}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(312)
    do = torch.randn((B, H, n, dv), generator=gen, device="cuda").to(torch.bfloat16)
    announce(f"full-size value-gradient identity n={n} c={c} H={H}")
    out = g.gecko_sca_awm_forward(z, p, v, c, out_dtype=torch.float32)
    res = g.gecko_backward(z, p, v, do, c)
    torch.cuda.synchronize()
    for h in range(H):
        lhs = float((v[0, h].double() * res["dv"][0, h].double()).sum())
        rhs = float((do[0, h].double() * out[0, h].double()).sum())
        scale = float((v[0, h].double() * res["dv"][0, h].double()).abs().sum())
        assert abs(lhs - rhs) <= 1e-2 * scale, (h, lhs, rhs, scale)


def test_backward_one_million_tokens():
    """1,048,576 tokens (512 chunks of 2048, B1 H2): the reverse state scan
    runs 510 steps; one (batch, head) slab of Z' spans 256 MiB and of V 512 MiB.
    Every gradient is finite; <V, dV> = <dO, O> for the whole layer; the
    attention gradients of sampled chunks (first, middle, last) match the
    oracle on their three-chunk stretches."""
    import torch

    g = gecko()
    B, H, n, c, d, dv = 1, 2, 1 << 20, 2048, 128, 256
    dev = inputs.make_inputs_device(B, H, n, d, dv, "bf16", seed=5, tag=313)
    z, v = dev["z"], dev["v"]
    p = {k: torch.from_numpy(a).cuda() for k, a in dev["params"].items()}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(313)
    do = torch.randn((B, H, n, dv), generator=gen, device="cuda").to(torch.bfloat16)
    announce(f"backward n={n} c={c} H={H}")
    out = g.gecko_sca_awm_forward(z, p, v, c, out_dtype=torch.float32)
    res = g.gecko_backward(z, p, v, do, c)
    torch.cuda.synchronize()
    for k in ("dz", "dv"):
        assert torch.isfinite(res[k]).all(), k
    assert all(torch.isfinite(res["d" + k]).all() for k in NAMES)
    for h in range(H):
        lhs = float((v[0, h].double() * res["dv"][0, h].double()).sum())
        rhs = float((do[0, h].double() * out[0, h].double()).sum())
        scale = float((v[0, h].double() * res["dv"][0, h].double()).abs().sum())
        assert abs(lhs - rhs) <= 1e-2 * scale, (h, lhs, rhs, scale)
    del out, res
    sca = g.gecko_backward(z, p, v, do, c, parts=g.GECKO_PART_SCA)
    torch.cuda.synchronize()
    N = n // c
    for s, h in ((1, 0), (N // 2, 1), (N - 2, 0)):
        a, b = (s - 1) * c, (s + 2) * c
        zs = z[0, h, a:b].float().cpu().numpy().astype(np.float64)[None, None]
        vs = v[0, h, a:b].float().cpu().numpy().astype(np.float64)[None, None]
        ds = do[0, h, a:b].float().cpu().numpy().astype(np.float64)[None, None]
        ph = {k: dev["params"][k][h:h + 1] for k in dev["params"]}
        want = go.grad(zs, vs, ph, c, ds, parts=("sca",))
        for key in ("dz", "dv"):
            got = to_numpy(sca[key][0, h, s * c:(s + 1) * c])
            fro, mx = _errors(got, want[key][0, 0, c:2 * c])
            assert fro <= GRAD_TOL and mx <= GRAD_TOL, (s, h, key, fro, mx)
