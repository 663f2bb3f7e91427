"""GPU tier: the training forward (gecko_forward_train) and the backward with
the forward's saved attention statistics (gecko_backward_saved) through the C
ABI, against the float64 oracles on the same seeded inputs.

The saved backward takes the attention weights as the forward's own
bf16-rounded ones, P = bf16(2^(s - m)) / l, so its gradients are those of the
forward as computed; the oracle differentiates the exact forward. The
difference is of the order of the bf16 rounding of the weights, inside the
bars of test_gpu_backward (relative Frobenius and max-relative 1e-2 for dZ'
and dV, the summation bound 2e-2 for the affine gradients), which apply here
unchanged. The forward's extra outputs are checked against the oracle's
attention output and log-sum-exp, and its main output must stay
bit-identical to the plain forward's.
"""

from __future__ import annotations

import numpy as np
import pytest

from chunked_attention_memory_amd import inputs
from gpu_helpers import announce, gecko, to_numpy
from test_gpu_backward import GRAD_TOL, NAMES, _check, _errors

import oracle
from oracle import gecko_grad_oracle as go

pytestmark = pytest.mark.gpu


def _names(g, parts):
    return (("sca",) if parts & g.GECKO_PART_SCA else ()) + (("awm",) if parts & g.GECKO_PART_AWM else ())


def _saved_case(B, H, n, dv, c, parts, flags=0, out_dtype="bf16", sharp=1.0, tag=400, host=None, keep=False):
    import torch

    g = gecko()
    if host is None:
        host = inputs.make_inputs(B, H, n, 128, dv, "bf16", seed=0, tag=tag)
        if sharp != 1.0:
            host["params"] = inputs.sharpen(host["params"], sharp)
    dout = inputs.make_dout(B, H, n, dv, out_dtype, seed=0, tag=tag)
    z, v, p = g.to_device_inputs(host)
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    do = torch.from_numpy(dout).to(device="cuda", dtype=odt)
    announce(f"saved backward B,H,n,d,dv={tuple(z.shape)}+{dv} c={c} parts={parts} flags={flags} out={out_dtype} "
             f"keep={keep}")
    if keep:
        _, o_sca, stats, mem = g.gecko_forward_train(z, p, v, c, parts=parts, flags=flags, keep_memory=True)
    else:
        (_, o_sca, stats), mem = g.gecko_forward_train(z, p, v, c, parts=parts, flags=flags), None
    res = g.gecko_backward_saved(z, p, v, do, o_sca, stats, c, parts=parts, flags=flags, mem_saved=mem)
    torch.cuda.synchronize()
    got = {k: to_numpy(t) for k, t in res.items()}
    names = _names(g, parts)
    want = go.grad(host["z"].astype(np.float64), host["v"].astype(np.float64), host["params"], c,
                   dout.astype(np.float64), parts=names, chunkwise=bool(flags & g.GECKO_CHUNKWISE),
                   no_delta=bool(flags & g.GECKO_AWM_NO_DELTA))
    _check(got, want, names, host["z"].astype(np.float64))
    for part in ("sca", "awm"):
        if part not in names:
            for k in (NAMES[:4] if part == "sca" else NAMES[4:]):
                assert np.all(got["d" + k] == 0.0), k
    return got


@pytest.mark.parametrize("chunkwise", [False, True])
@pytest.mark.parametrize("both", [True, False])
def test_forward_train_outputs(chunkwise, both):
    """out equals the plain forward bit for bit; o_sca is the attention output
    (oracle); stats give the log-sum-exp ln2 (m + log2 l) + q . nu_k (oracle,
    and the gecko_forward_lse output of the same kernel arithmetic)."""
    import torch

    g = gecko()
    host = inputs.make_inputs(1, 2, 700, 128, 256, "bf16", seed=0, tag=401)
    host["params"] = inputs.sharpen(host["params"], 3.0)
    z, v, p = g.to_device_inputs(host)
    flags = g.GECKO_CHUNKWISE if chunkwise else 0
    parts = g.GECKO_PART_SCA | (g.GECKO_PART_AWM if both else 0)
    announce(f"forward_train flags={flags} parts={parts}")
    out, o_sca, stats = g.gecko_forward_train(z, p, v, 128, parts=parts, flags=flags)
    if both:
        ref = g.gecko_sca_awm_forward(z, p, v, 128, flags=flags)
        _, lse = g.gecko_forward_lse(z, p, v, 128, flags=flags)
    else:
        ref, lse = g.gecko_forward_lse(z, p, v, 128, parts=g.GECKO_PART_SCA, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    o = to_numpy(o_sca)
    st = to_numpy(stats).astype(np.float64)
    lse_dev = to_numpy(lse).astype(np.float64)
    for h in range(2):
        zh = host["z"][0, h].astype(np.float64)
        r = oracle.forward_head(zh, host["v"][0, h].astype(np.float64), host["params"], h, 128, chunkwise=chunkwise)
        fro, mx = _errors(o[0, h], r["o_sca"])
        assert fro <= GRAD_TOL and mx <= GRAD_TOL, (h, fro, mx)
        qn = (zh * host["params"]["kappa_q"][h] + host["params"]["nu_q"][h]) @ host["params"]["nu_k"][h]
        lse_st = np.log(2.0) * (st[0, h, :, 0] + np.log2(st[0, h, :, 1])) + qn
        want = go.lse_head(zh, host["params"], h, 128, chunkwise=chunkwise)
        assert np.max(np.abs(lse_st - want)) <= 2e-2
        assert np.max(np.abs(lse_st - lse_dev[0, h])) <= 1e-4 * max(1.0, np.max(np.abs(want)))
        assert np.all(st[0, h, :, 1] > 0)


@pytest.mark.parametrize("B,H,n,dv,c", [
    (1, 2, 700, 256, 128),   # 6 chunks, ragged tail
    (2, 1, 520, 128, 128),   # dv 128, batch 2
    (1, 1, 600, 256, 96),    # chunk length not a multiple of the 64-row tiles
    (1, 1, 300, 256, 1000),  # one chunk (c > n)
    (1, 1, 65, 256, 64),     # two chunks, one-token tail
    (1, 1, 1, 256, 64),      # a single token
    (2, 3, 333, 128, 64),    # batch and heads together, ragged tail
])
def test_backward_saved_both_parts(B, H, n, dv, c):
    g = gecko()
    _saved_case(B, H, n, dv, c, g.GECKO_PART_SCA | g.GECKO_PART_AWM)


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_backward_saved_attention_only(out_dtype):
    g = gecko()
    _saved_case(1, 2, 640, 256, 128, g.GECKO_PART_SCA, out_dtype=out_dtype, sharp=3.0, tag=402)


def test_backward_saved_variants():
    g = gecko()
    _saved_case(1, 1, 700, 256, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, flags=g.GECKO_AWM_NO_DELTA, tag=403)
    _saved_case(1, 1, 700, 256, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, flags=g.GECKO_CHUNKWISE, tag=404)
    _saved_case(1, 2, 128, 256, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, flags=g.GECKO_CHUNKWISE, tag=405)
    _saved_case(1, 1, 900, 256, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, out_dtype="f32", sharp=2.0, tag=406)


def test_backward_saved_sharp_logits():
    """Peaked softmax rows, where dS = P (dP - D) is a small difference of
    large terms: D' = dO' . O must agree with the weights the kernels rebuild."""
    g = gecko()
    _saved_case(1, 1, 800, 256, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, sharp=4.0, tag=407)


def test_backward_saved_logits_past_the_exponent_range():
    """A logit component shared by every key overflows 2^s: the forward takes
    its exact-maximum path and saves that offset, which the backward reuses."""
    g = gecko()
    host = inputs.make_inputs(1, 1, 300, 128, 256, "bf16", seed=0, tag=408)
    host["z"][..., 0] = 3.0
    for k in ("kappa_q", "kappa_k"):
        host["params"][k][:, 0] = 8.0
    _saved_case(1, 1, 300, 256, 128, g.GECKO_PART_SCA, tag=408, host=host)


def test_backward_saved_agrees_with_recompute_and_repeats():
    """The saved and the recomputing backward approximate the same gradient
    (to the bar); two saved calls are bit-identical."""
    import torch

    g = gecko()
    host = inputs.make_inputs(1, 2, 512, 128, 256, "bf16", seed=1, tag=409)
    dout = inputs.make_dout(1, 2, 512, 256, "bf16", seed=1, tag=409)
    z, v, p = g.to_device_inputs(host)
    do = torch.from_numpy(dout).to(device="cuda", dtype=torch.bfloat16)
    announce("saved vs recompute backward")
    _, o_sca, stats = g.gecko_forward_train(z, p, v, 128)
    a = g.gecko_backward_saved(z, p, v, do, o_sca, stats, 128)
    b = g.gecko_backward_saved(z, p, v, do, o_sca, stats, 128)
    r = g.gecko_backward(z, p, v, do, 128)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    for k in ("dz", "dv"):
        fro, mx = _errors(to_numpy(a[k]), to_numpy(r[k]))
        assert fro <= GRAD_TOL and mx <= GRAD_TOL, (k, fro, mx)


def test_kept_memory_oracle():
    """Backward with the training forward's kept memory pass, against the
    oracle: both parts, 12 chunks, sliding and chunk-wise."""
    g = gecko()
    _saved_case(1, 2, 1500, 256, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, tag=410, keep=True)
    _saved_case(1, 1, 1500, 128, 128, g.GECKO_PART_SCA | g.GECKO_PART_AWM, flags=g.GECKO_CHUNKWISE, tag=411,
                keep=True)


@pytest.mark.parametrize("B,H,n,dv,c,flags", [
    (1, 2, 2300, 256, 256, 0),          # 9 chunks, ragged tail
    (2, 1, 1100, 128, 128, 1),          # without the delta correction (GECKO_AWM_NO_DELTA)
    (1, 2, 1100, 256, 128, 2),          # chunk-wise
    (1, 1, 256, 256, 128, 0),           # two chunks: nothing reads the memory, nothing kept
    (1, 2, 16384, 256, 2048, 0),        # the bench's chunk size, 8 chunks
])
def test_kept_memory_bit_identical(B, H, n, dv, c, flags):
    """The training forward that keeps its memory pass writes the same output,
    O_SCA and statistics as the one that does not, and the backward that reads
    the kept pass returns the same bits as the one that recomputes it, twice
    in a row (the kept buffer is only read)."""
    import torch

    g = gecko()
    parts = g.GECKO_PART_SCA | g.GECKO_PART_AWM
    host = inputs.make_inputs(B, H, n, 128, dv, "bf16", seed=2, tag=412)
    dout = inputs.make_dout(B, H, n, dv, "bf16", seed=2, tag=412)
    z, v, p = g.to_device_inputs(host)
    do = torch.from_numpy(dout).to(device="cuda", dtype=torch.bfloat16)
    announce(f"kept memory B,H,n,dv,c,flags={(B, H, n, dv, c, flags)}")
    out_k, o_k, st_k, mem = g.gecko_forward_train(z, p, v, c, parts=parts, flags=flags, keep_memory=True)
    out_r, o_r, st_r = g.gecko_forward_train(z, p, v, c, parts=parts, flags=flags)
    assert mem.numel() == max(g.gecko_memory_saved_size(B, H, n, 128, dv, c, flags=flags), 256)
    a = g.gecko_backward_saved(z, p, v, do, o_k, st_k, c, parts=parts, flags=flags, mem_saved=mem)
    b = g.gecko_backward_saved(z, p, v, do, o_k, st_k, c, parts=parts, flags=flags, mem_saved=mem)
    r = g.gecko_backward_saved(z, p, v, do, o_r, st_r, c, parts=parts, flags=flags)
    torch.cuda.synchronize()
    for x, y, name in ((out_k, out_r, "out"), (o_k, o_r, "o_sca"), (st_k, st_r, "stats")):
        assert torch.equal(x, y), name
    for k in r:
        assert torch.isfinite(a[k]).all(), k
        assert torch.equal(a[k], r[k]), k
        assert torch.equal(b[k], r[k]), k


def test_backward_saved_full_size():
    """The bench configuration (B1 H8, 131072 tokens, c 2048), both parts:
    finite gradients; <V, dV> = <dO, O>; the training forward's O_SCA of
    chunks 1, 40 and 63 against the oracle on their two-chunk stretches; the
    attention gradients of chunks 1 and 40 of two heads against the oracle on
    their three-chunk stretches (attention-only call)."""
    import torch

    g = gecko()
    B, H, n, c, d, dv = 1, 8, 131072, 2048, 128, 256
    dev = inputs.make_inputs_device(B, H, n, d, dv, "bf16", seed=3, tag=412)
    z, v = dev["z"], dev["v"]
    p = {k: torch.from_numpy(a).cuda() for k, a in dev["params"].items()}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(412)
    do = torch.randn((B, H, n, dv), generator=gen, device="cuda").to(torch.bfloat16)
    announce(f"full-size saved backward n={n} c={c} H={H}")
    out, o_sca, stats = g.gecko_forward_train(z, p, v, c, out_dtype=torch.float32)
    res = g.gecko_backward_saved(z, p, v, do, o_sca, stats, c)
    torch.cuda.synchronize()
    assert torch.isfinite(res["dz"]).all() and torch.isfinite(res["dv"]).all()
    for h in range(H):
        lhs = float((v[0, h].double() * res["dv"][0, h].double()).sum())
        rhs = float((do[0, h].double() * out[0, h].double()).sum())
        scale = float((v[0, h].double() * res["dv"][0, h].double()).abs().sum())
        assert abs(lhs - rhs) <= 1e-2 * scale, (h, lhs, rhs, scale)
    # the training forward's attention output on sampled chunks: the oracle's
    # O_SCA of chunk s needs chunks s-1 and s only
    for s, h in ((1, 0), (40, 5), (63, 7)):
        a, b = (s - 1) * c, (s + 1) * c
        zs = z[0, h, a:b].float().cpu().numpy().astype(np.float64)
        vs = v[0, h, a:b].float().cpu().numpy().astype(np.float64)
        pr = dev["params"]
        want = oracle.sca_head(zs, vs, pr["kappa_q"][h], pr["nu_q"][h], pr["kappa_k"][h], pr["nu_k"][h], c)
        fro, mx = _errors(to_numpy(o_sca[0, h, s * c:(s + 1) * c]), want[c:])
        assert fro <= GRAD_TOL and mx <= GRAD_TOL, (s, h, fro, mx)
    del out, res
    _, o_sca, stats = g.gecko_forward_train(z, p, v, c, parts=g.GECKO_PART_SCA)
    sca = g.gecko_backward_saved(z, p, v, do, o_sca, stats, c, parts=g.GECKO_PART_SCA)
    torch.cuda.synchronize()
    for s, h in ((1, 0), (40, 5)):
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


def test_backward_saved_one_million_tokens():
    """1,048,576 tokens (512 chunks of 2048, B1 H2; o_sca alone is 2 GiB):
    finite gradients, <V, dV> = <dO, O>, and the saved backward within the
    bar of the recomputing one on sampled rows of every 64th chunk."""
    import torch

    g = gecko()
    B, H, n, c, d, dv = 1, 2, 1 << 20, 2048, 128, 256
    dev = inputs.make_inputs_device(B, H, n, d, dv, "bf16", seed=5, tag=413)
    z, v = dev["z"], dev["v"]
    p = {k: torch.from_numpy(a).cuda() for k, a in dev["params"].items()}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(413)
    do = torch.randn((B, H, n, dv), generator=gen, device="cuda").to(torch.bfloat16)
    announce(f"saved backward n={n} c={c} H={H}")
    out, o_sca, stats = g.gecko_forward_train(z, p, v, c, out_dtype=torch.float32)
    res = g.gecko_backward_saved(z, p, v, do, o_sca, stats, c)
    torch.cuda.synchronize()
    assert torch.isfinite(res["dz"]).all() and torch.isfinite(res["dv"]).all()
    assert all(torch.isfinite(res["d" + k]).all() for k in NAMES)
    for h in range(H):
        lhs = float((v[0, h].double() * res["dv"][0, h].double()).sum())
        rhs = float((do[0, h].double() * out[0, h].double()).sum())
        scale = float((v[0, h].double() * res["dv"][0, h].double()).abs().sum())
        assert abs(lhs - rhs) <= 1e-2 * scale, (h, lhs, rhs, scale)
    del out, o_sca, stats
    ref = g.gecko_backward(z, p, v, do, c)
    torch.cuda.synchronize()
    rows = torch.cat([torch.arange(s * c, s * c + 256) for s in range(0, n // c, 64)]).cuda()
    for key in ("dz", "dv"):
        for h in range(H):
            got = to_numpy(res[key][0, h].index_select(0, rows))
            want = to_numpy(ref[key][0, h].index_select(0, rows))
            fro, mx = _errors(got, want)
            assert fro <= GRAD_TOL and mx <= GRAD_TOL, (key, h, fro, mx)


def test_training_pair_four_million_tokens():
    """The largest configuration (B1 H4, 4,194,304 tokens, c 2048): each (batch,
    head) slab of V and its gradients holds 2^30 values and the arrays 2^32,
    so every offset past a slab is 64-bit. The training forward and the
    saved-statistics backward run to completion with finite gradients,
    <V, dV> = <dO, O> per head, and the attention gradients of the first and
    the last chunk of a head against the oracle on their three-chunk
    stretches (attention-only call)."""
    import torch

    g = gecko()
    B, H, n, c, d, dv = 1, 4, 1 << 22, 2048, 128, 256
    dev = inputs.make_inputs_device(B, H, n, d, dv, "bf16", seed=7, tag=414)
    z, v = dev["z"], dev["v"]
    p = {k: torch.from_numpy(a).cuda() for k, a in dev["params"].items()}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(414)
    do = torch.empty((B, H, n, dv), dtype=torch.bfloat16, device="cuda")
    for h in range(H):  # drawn per head to bound the float32 temporary
        do[0, h] = torch.randn((n, dv), generator=gen, device="cuda").to(torch.bfloat16)
    announce(f"training pair n={n} c={c} H={H}")
    out, o_sca, stats = g.gecko_forward_train(z, p, v, c)
    res = g.gecko_backward_saved(z, p, v, do, o_sca, stats, c)
    torch.cuda.synchronize()
    assert torch.isfinite(res["dz"]).all() and torch.isfinite(res["dv"]).all()
    assert all(torch.isfinite(res["d" + k]).all() for k in NAMES)
    for h in range(H):
        lhs = float((v[0, h].double() * res["dv"][0, h].double()).sum())
        rhs = float((do[0, h].double() * out[0, h].float().double()).sum())
        scale = float((v[0, h].double() * res["dv"][0, h].double()).abs().sum())
        assert abs(lhs - rhs) <= 1e-2 * scale, (h, lhs, rhs, scale)
    del out, o_sca, stats, res
    torch.cuda.empty_cache()
    _, o_sca, stats = g.gecko_forward_train(z, p, v, c, parts=g.GECKO_PART_SCA)
    sca = g.gecko_backward_saved(z, p, v, do, o_sca, stats, c, parts=g.GECKO_PART_SCA)
    torch.cuda.synchronize()
    N = n // c
    for s, h in ((1, 3), (N - 2, 3)):
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
