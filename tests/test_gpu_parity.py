"""GPU tier: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs. Tolerances: float32 path max |y-x| / max(|x|, 1e-3 rms(x))
<= 1e-4; bf16 inputs with fp32 accumulation max |y-x| / rms(x) <= 2e-2,
measured on the float32 output; the bf16 output is checked to be exactly the
round-to-nearest-even of that float32 output. Index and mask logic exact."""

from __future__ import annotations

import numpy as np
import pytest

from chunked_attention_memory_amd import configs
from gpu_helpers import BF16_TOL, F32_TOL, floor_rel_err, make, oracle_parts, rms_err, run, run_raw

pytestmark = pytest.mark.gpu


def _stack(parts, key, heads):
    return np.stack([parts[bh][key] for bh in heads])


def _gpu_heads(arr, heads):
    return np.stack([arr[b, h] for b, h in heads])


def test_f32_tiny_workload_all_parts():
    w = configs.WORKLOADS[0]
    host = make(w.B, w.H, w.n, w.d, w.dv, "f32", tag=0)
    heads = [(0, 0)]
    ref = oracle_parts(host, w.c)
    for entry, key in (("full", "o"), ("sca", "o_sca"), ("awm", "o_m")):
        got = _gpu_heads(run(host, w.c, entry), heads)
        err = floor_rel_err(got, _stack(ref, key, heads))
        assert err <= F32_TOL, (entry, err)


F32_SHAPES = [
    (1, 2, 300, 64, 32, 64),
    (2, 1, 129, 16, 64, 32),
    (1, 1, 50, 1, 32, 32),
    (1, 1, 100, 128, 128, 256),
]


@pytest.mark.parametrize("B,H,n,c,d,dv", F32_SHAPES)
def test_f32_shapes(B, H, n, c, d, dv):
    host = make(B, H, n, d, dv, "f32", tag=1)
    ref = oracle_parts(host, c)
    heads = list(ref)
    got = _gpu_heads(run(host, c, "full"), heads)
    assert floor_rel_err(got, _stack(ref, "o", heads)) <= F32_TOL


def test_f32_more_than_65535_heads():
    """66,000 (batch, head) pairs of 5 tokens in chunks of 2 (one memory step
    each): more workgroups than a y or z grid dimension holds. Heads are
    independent, so sampled heads (first, last, and one in between) are
    checked against the oracle."""
    H, n, c, d, dv = 66000, 5, 2, 32, 32
    host = make(1, H, n, d, dv, "f32", tag=5)
    got = run(host, c, "full")
    heads = [(0, 0), (0, 40001), (0, H - 1)]
    ref = oracle_parts(host, c, heads=heads)
    assert floor_rel_err(_gpu_heads(got, heads), _stack(ref, "o", heads)) <= F32_TOL


BF16_SHAPES = [
    (1, 2, 700, 128, 128, 256),   # ragged tail, 6 chunks
    (1, 1, 1000, 256, 128, 256),  # 4 chunks, ragged
    (2, 1, 513, 64, 128, 256),    # chunk smaller than a query tile
    (1, 1, 300, 300, 128, 256),   # one chunk: causal attention
    (1, 1, 200, 1000, 128, 256),  # c > n
    (1, 1, 1, 7, 128, 256),       # single token
    (1, 1, 40, 1, 128, 256),      # one token per chunk
    (1, 2, 640, 128, 64, 128),
    (1, 1, 777, 100, 128, 128),   # c not a multiple of the tile sizes
    (1, 1, 450, 64, 64, 64),
    (1, 1, 4096, 512, 128, 256),  # several full tiles per chunk
    # the remaining (d, dv) pairs: 64-byte rows (d or dv = 32) and tiles with
    # fewer staging pieces than waves
    (1, 2, 700, 128, 128, 64),
    (1, 1, 650, 100, 128, 32),    # c not a multiple of the tile sizes
    (2, 1, 513, 64, 64, 256),
    (1, 1, 700, 128, 64, 32),
    (1, 2, 600, 128, 32, 256),
    (1, 1, 777, 96, 32, 128),
    (1, 1, 500, 64, 32, 64),
    (2, 2, 333, 64, 32, 32),      # batch and heads, ragged tail
    (1, 1, 1, 7, 32, 32),         # single token at the smallest shape
]


@pytest.mark.parametrize("B,H,n,c,d,dv", BF16_SHAPES)
def test_bf16_shapes(B, H, n, c, d, dv):
    host = make(B, H, n, d, dv, "bf16", tag=2)
    ref = oracle_parts(host, c)
    heads = list(ref)
    got = _gpu_heads(run(host, c, "full"), heads)
    assert rms_err(got, _stack(ref, "o", heads)) <= BF16_TOL
    got = _gpu_heads(run(host, c, "sca"), heads)
    assert rms_err(got, _stack(ref, "o_sca", heads)) <= BF16_TOL
    want_m = _stack(ref, "o_m", heads)
    got_m = _gpu_heads(run(host, c, "awm"), heads)
    if np.any(want_m != 0):
        assert rms_err(got_m, want_m) <= BF16_TOL
    else:
        assert np.all(got_m == 0)


def test_bf16_batched_16k_sampled_heads():
    w = configs.WORKLOADS[1]
    host = make(w.B, w.H, w.n, w.d, w.dv, "bf16", tag=1)
    heads = [(0, 0), (1, 5), (3, 7)]
    out = run(host, w.c, "full")
    ref = oracle_parts(host, w.c, heads=heads)
    assert rms_err(_gpu_heads(out, heads), _stack(ref, "o", heads)) <= BF16_TOL


def test_bf16_headline_128k_sampled_chunks():
    w = configs.WORKLOADS[2]
    host = make(w.B, w.H, w.n, w.d, w.dv, "bf16", tag=2)
    N = w.nchunks
    chunks = [0, 1, 2, 3, N // 2, N - 2, N - 1]
    out = run(host, w.c, "full")
    heads = [(0, h) for h in range(w.H)]
    ref = oracle_parts(host, w.c, heads=heads, sca_chunks=chunks)
    got = np.concatenate([out[b, h, s * w.c:min((s + 1) * w.c, w.n)] for b, h in heads for s in chunks])
    want = np.concatenate([ref[bh]["o"][s] for bh in heads for s in chunks])
    assert rms_err(got, want) <= BF16_TOL
    # the memory part alone, over every row
    import oracle

    got_m = _gpu_heads(run(host, w.c, "awm"), heads)
    p = host["params"]
    for i, (b, h) in enumerate(heads):
        want_m = oracle.awm_head(host["z"][b, h], host["v"][b, h], p["eta_q"][h], p["rho_q"][h], p["eta_k"][h],
                                 p["rho_k"][h], w.c)
        assert rms_err(got_m[i], want_m) <= BF16_TOL


def _rne_bf16(t):
    """Round a float32 tensor to bf16 (nearest even) on the host, bit by bit."""
    import numpy as np

    u = t.detach().cpu().numpy().view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


@pytest.mark.parametrize("entry", ["full", "sca", "awm"])
def test_bf16_output_is_rounded_fp32_output(entry):
    import torch

    from chunked_attention_memory_amd import gecko as g

    host = make(1, 2, 1500, 128, 256, "bf16", tag=3)
    dev = g.to_device_inputs(host)
    f32 = run_raw(host, 256, entry, device_inputs=dev, out_f32=True)
    b16 = run_raw(host, 256, entry, device_inputs=dev, out_f32=False)
    assert b16.dtype == torch.bfloat16
    got = b16.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, _rne_bf16(f32))


@pytest.mark.parametrize("scale", [80.0, 200.0])
def test_bf16_logits_beyond_first_tile_range(scale):
    """Logits that grow past the first key tile's maximum by more than 2^63
    (in base 2) take the kernel's exact-maximum path; with a large query
    scale each query attends almost only to itself, which keeps the bf16
    comparison well conditioned."""
    host = make(1, 2, 1100, 128, 256, "bf16", tag=4)
    host["params"]["kappa_q"][:] = scale
    host["params"]["nu_q"][:] = 0.0
    host["params"]["kappa_k"][:] = 1.0
    ref = oracle_parts(host, 256)
    heads = list(ref)
    got = _gpu_heads(run(host, 256, "sca"), heads)
    want = _stack(ref, "o_sca", heads)
    assert np.all(np.isfinite(got))
    assert rms_err(got, want) <= BF16_TOL


def test_side_stream_matches_current_stream():
    """The forward and the backward launched on a stream other than the
    current one give the results of the current stream bit for bit, while
    the current stream allocates and writes fresh memory right after the
    launches (the binding's workspaces belong to the launch stream, so the
    caching allocator cannot hand their blocks to those writes)."""
    import torch

    from chunked_attention_memory_amd import gecko as g
    from chunked_attention_memory_amd import inputs

    host = make(1, 2, 1100, 128, 256, "bf16", tag=41)
    dev = g.to_device_inputs(host)
    z, v, p = dev
    do = torch.from_numpy(inputs.make_dout(1, 2, 1100, 256, "bf16", tag=41)).to(device="cuda", dtype=torch.bfloat16)
    ref = g.gecko_sca_awm_forward(z, p, v, 256)
    ref_b = g.gecko_backward(z, p, v, do, 256)
    _, o_r, st_r, mem_r = g.gecko_forward_train(z, p, v, 256, keep_memory=True)
    ref_s = g.gecko_backward_saved(z, p, v, do, o_r, st_r, 256, mem_saved=mem_r)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = g.gecko_sca_awm_forward(z, p, v, 256, stream=side)
    res = g.gecko_backward(z, p, v, do, 256, stream=side)
    # the training pair with the kept memory pass (buffer allocated by the binding on the side stream)
    _, o_s, st_s, mem_s = g.gecko_forward_train(z, p, v, 256, keep_memory=True, stream=side)
    res_s = g.gecko_backward_saved(z, p, v, do, o_s, st_s, 256, mem_saved=mem_s, stream=side)
    junk = [torch.full((1 << 22,), 7.0, device="cuda") for _ in range(16)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out, ref)
    for k in ref_b:
        assert torch.equal(res[k], ref_b[k]), k
    for k in ref_s:
        assert torch.equal(res_s[k], ref_s[k]), k
