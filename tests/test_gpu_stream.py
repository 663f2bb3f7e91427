"""GPU tier: the streaming forward (gecko_sca_awm_forward_stream) through the
C ABI. A sequence handed over in consecutive calls must give
* bit-identical rows to one gecko_sca_awm_forward call over the whole
  sequence (the kernels see the same operands in the same order: the carried
  chunk stands where the previous chunk would be, and the carried float32
  state and denominator are the values the one-call scan holds at that
  step), and
* the fp64 oracle's rows for the whole sequence, within the bf16 bar
  (max |y - x| / rms(x) <= 2e-2 on float32 output).
Splits cover one-chunk calls (the first of which enters nothing into the
memory), calls shorter than a chunk, a ragged last call, NO_DELTA, and the
128K-token workload cut into four calls."""

from __future__ import annotations

import numpy as np
import pytest

from chunked_attention_memory_amd import configs
from gpu_helpers import BF16_TOL, announce, gecko, make, oracle_parts, rms_err, to_numpy

pytestmark = pytest.mark.gpu


def _stream(z, v, p, c, splits, flags=0, out_dtype=None, st=None):
    """Run the calls of one sequence; returns the outputs concatenated along n."""
    import torch

    g = gecko()
    B, H, n, d = z.shape
    if st is None:
        st = g.Stream(B, H, d, v.shape[3], c, p, flags=flags)
    outs, at = [], 0
    for m in splits:
        announce(f"stream B,H={B},{H} d,dv={d},{v.shape[3]} c={c} pos={at} n={m} flags={flags}")
        outs.append(st.forward(z[:, :, at:at + m].contiguous(), v[:, :, at:at + m].contiguous(),
                               out_dtype=out_dtype or torch.float32))
        torch.cuda.synchronize()
        at += m
    assert at == n
    return torch.cat(outs, dim=2)


def _one_call(z, v, p, c, flags=0, out_dtype=None):
    import torch

    g = gecko()
    announce(f"one call B,H,n={tuple(z.shape[:3])} c={c} flags={flags}")
    out = g.gecko_sca_awm_forward(z, p, v, c, flags=flags, out_dtype=out_dtype or torch.float32)
    torch.cuda.synchronize()
    return out


SPLITS = [
    # (H, n, c, d, dv, splits in tokens)
    (2, 8 * 256, 256, 128, 256, [256, 768, 1024]),
    (1, 8 * 256 + 100, 256, 128, 256, [512, 1280, 356]),     # ragged last call
    (1, 5 * 128, 128, 128, 256, [128] * 5),                   # one chunk per call
    (2, 6 * 64 + 10, 64, 64, 64, [64, 192, 64, 74]),
    (1, 3 * 256 + 50, 256, 128, 128, [256, 256, 256, 50]),    # last call shorter than a chunk
    (1, 4 * 512, 512, 64, 128, [2048]),                       # one call
    (1, 1000, 2048, 128, 256, [1000]),                        # one call, c > n
    (1, 6 * 128 + 30, 128, 32, 32, [256, 384, 158]),          # the smallest shape
    (2, 5 * 64, 64, 32, 256, [128, 64, 128]),                 # 64-byte key rows, dv 256
]


@pytest.mark.parametrize("H,n,c,d,dv,splits", SPLITS)
def test_stream_matches_one_call_bit_exact_and_oracle(H, n, c, d, dv, splits):
    import torch

    g = gecko()
    host = make(1, H, n, d, dv, "bf16", tag=11)
    z, v, p = g.to_device_inputs(host)
    got = _stream(z, v, p, c, splits)
    want = _one_call(z, v, p, c)
    assert torch.equal(got, want), float((got - want).abs().max())
    ref = oracle_parts(host, c)
    for (b, h), r in ref.items():
        assert rms_err(to_numpy(got[b, h]), r["o"]) <= BF16_TOL


def test_stream_no_delta_and_bf16_output():
    import torch

    g = gecko()
    c = 128
    host = make(1, 2, 7 * c, 128, 256, "bf16", tag=12)
    z, v, p = g.to_device_inputs(host)
    flags = g.GECKO_AWM_NO_DELTA
    got = _stream(z, v, p, c, [2 * c, c, 4 * c], flags=flags)
    assert torch.equal(got, _one_call(z, v, p, c, flags=flags))
    ref = oracle_parts(host, c, no_delta=True)
    for (b, h), r in ref.items():
        assert rms_err(to_numpy(got[b, h]), r["o"]) <= BF16_TOL
    got16 = _stream(z, v, p, c, [3 * c, 4 * c], out_dtype=torch.bfloat16)
    assert torch.equal(got16, _one_call(z, v, p, c, out_dtype=torch.bfloat16))


def test_stream_state_is_reset_by_pos_zero():
    """A second sequence on the same state object starts from pos 0 and must
    not see the first one."""
    import torch

    g = gecko()
    c = 256
    a = make(1, 2, 6 * c, 128, 256, "bf16", tag=13)
    b = make(1, 2, 5 * c, 128, 256, "bf16", tag=14)
    za, va, pa = g.to_device_inputs(a)
    zb, vb, _ = g.to_device_inputs(b)
    st = g.Stream(1, 2, 128, 256, c, pa)
    _stream(za, va, pa, c, [2 * c, 4 * c], st=st)
    st.pos = 0
    got = _stream(zb, vb, pa, c, [c, 4 * c], st=st)
    assert torch.equal(got, _one_call(zb, vb, pa, c))


def test_stream_headline_128k_in_four_calls():
    import torch

    g = gecko()
    w = configs.WORKLOADS[2]
    from chunked_attention_memory_amd import inputs

    dev = inputs.make_inputs_device(w.B, w.H, w.n, w.d, w.dv, "bf16", seed=0, tag=15)
    z, v = dev["z"], dev["v"]
    p = {k: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.float32) for k, a in dev["params"].items()}
    q = w.n // 4
    got = _stream(z, v, p, w.c, [q] * 4, out_dtype=torch.bfloat16)
    want = _one_call(z, v, p, w.c, out_dtype=torch.bfloat16)
    assert torch.equal(got, want)
    assert bool(torch.isfinite(got.float()).all())


def test_stream_refuses_bad_pos_on_device_buffers():
    import torch

    g = gecko()
    host = make(1, 1, 256, 128, 256, "bf16", tag=16)
    z, v, p = g.to_device_inputs(host)
    st = torch.empty(g.gecko_stream_state_size(1, 1, 128, 256, 128, g.GECKO_BF16), dtype=torch.uint8,
                     device=z.device)
    with pytest.raises(g.GeckoError) as e:
        g.gecko_sca_awm_forward_stream(z, p, v, 128, 64, st)
    assert e.value.status == g.GECKO_EINVAL
