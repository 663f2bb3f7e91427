"""GPU tier: gecko_sca_awm_forward_noalloc, the forward for callers that
cannot allocate device memory, through the C ABI against
gecko_sca_awm_forward (which the parity tests check against the oracle).

The two run the same kernels on the same operands, so the bar is bit
identity. Calls come in a row on one GPU, each smaller than the one before, so
that every call after the first runs on scratch memory that still holds the
previous call's values; outputs start as NaN, so an unwritten entry fails."""

from __future__ import annotations

import pytest

from chunked_attention_memory_amd import inputs
from gpu_helpers import announce, gecko, make

pytestmark = pytest.mark.gpu


def _noalloc(z, p, v, c, ref, flags=0):
    import torch

    g = gecko()
    out = torch.full(ref.shape, float("nan"), dtype=ref.dtype, device=ref.device)
    g.gecko_sca_awm_forward_noalloc(z, p, v, c, out, flags=flags)
    torch.cuda.synchronize()
    return out


def test_noalloc_equals_forward_on_calls_of_decreasing_size():
    import torch

    g = gecko()
    # 1: the bench configuration (B1 H8, 131072 tokens, c 2048): 109.5 MiB of scratch
    B, H, n, c, d, dv = 1, 8, 131072, 2048, 128, 256
    dev = inputs.make_inputs_device(B, H, n, d, dv, "bf16", seed=7, tag=600)
    p = {k: torch.from_numpy(a).cuda() for k, a in dev["params"].items()}
    need = g.gecko_workspace_size(B, H, n, d, dv, c, g.GECKO_BF16)
    assert 0 < need <= g.NOALLOC_SCRATCH_BYTES
    announce(f"noalloc n={n} c={c} H={H}")
    ref = g.gecko_sca_awm_forward(dev["z"], p, dev["v"], c)
    torch.cuda.synchronize()
    out = _noalloc(dev["z"], p, dev["v"], c, ref)
    assert torch.equal(out, ref)
    del dev, ref, out
    # 2: a smaller input (5 chunks, ragged tail, two heads, float32 output)
    host = make(1, 2, 1100, 128, 256, "bf16", tag=601)
    z, v, p = g.to_device_inputs(host)
    announce("noalloc n=1100 c=256 H=2")
    ref = g.gecko_sca_awm_forward(z, p, v, 256, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(_noalloc(z, p, v, 256, ref), ref)
    # 3: smaller still, the variants: no delta term, chunk-wise attention
    host = make(2, 1, 600, 64, 128, "bf16", tag=602)
    z, v, p = g.to_device_inputs(host)
    for flags in (g.GECKO_AWM_NO_DELTA, g.GECKO_CHUNKWISE):
        announce(f"noalloc n=600 c=128 B=2 flags={flags}")
        ref = g.gecko_sca_awm_forward(z, p, v, 128, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(_noalloc(z, p, v, 128, ref, flags=flags), ref)
    # 4: the float32 path (its own workspace layout), tiny
    host = make(1, 1, 256, 32, 32, "f32", tag=603)
    z, v, p = g.to_device_inputs(host)
    announce("noalloc f32 n=256 c=64")
    ref = g.gecko_sca_awm_forward(z, p, v, 64)
    torch.cuda.synchronize()
    assert torch.equal(_noalloc(z, p, v, 64, ref), ref)


def test_noalloc_on_a_side_stream_and_at_most_two_chunks():
    """On a non-default stream; and with at most two chunks, where the memory
    is never entered and the scratch array is not touched."""
    import torch

    g = gecko()
    host = make(1, 2, 700, 128, 256, "bf16", tag=604)
    z, v, p = g.to_device_inputs(host)
    ref = g.gecko_sca_awm_forward(z, p, v, 128)
    torch.cuda.synchronize()
    out = torch.full(ref.shape, float("nan"), dtype=ref.dtype, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())  # the inputs and the NaN fill of out are done
    announce("noalloc side stream n=700 c=128")
    g.gecko_sca_awm_forward_noalloc(z, p, v, 128, out, stream=side)
    side.synchronize()
    assert torch.equal(out, ref)
    ref2 = g.gecko_sca_awm_forward(z, p, v, 512)
    torch.cuda.synchronize()
    assert torch.equal(_noalloc(z, p, v, 512, ref2), ref2)
