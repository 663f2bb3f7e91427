"""The measurement helper on the GPU: a forward that records the stage events
(gecko_sca_awm_forward_timed) writes the same output, bit for bit, as one that
does not; the per-stage times are non-negative, count every recorded call,
stop counting at the timer's capacity, and add up to no more than the wall
time of the calls (the events carry timing only and add no work of their
own)."""

from __future__ import annotations

import numpy as np
import pytest

from chunked_attention_memory_amd import inputs
from gpu_helpers import announce, gecko

pytestmark = pytest.mark.gpu


def test_timed_forward_matches_untimed_and_stage_times_add_up():
    import torch

    g = gecko()
    B, H, n, c, d, dv = 1, 2, 8192, 2048, 128, 256
    announce(f"timer B,H,n,d,dv={(B, H, n, d, dv)} c={c}")
    host = inputs.make_inputs(B, H, n, d, dv, "bf16", seed=3, tag=31)
    z, v, p = g.to_device_inputs(host)
    plain = g.gecko_sca_awm_forward(z, p, v, c)
    calls, cap = 6, 4
    timer = g.Timer(cap)
    outs = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        outs.append(g.gecko_sca_awm_forward(z, p, v, c, timer=timer))
    e1.record()
    torch.cuda.synchronize()
    wall = e0.elapsed_time(e1)
    stages, recorded = timer.read()
    timer.close()
    for o in outs:
        assert torch.equal(o.view(torch.int16), plain.view(torch.int16))
    assert recorded == cap  # calls beyond the capacity are not recorded
    assert set(stages) == set(g.Timer.STAGES)
    assert all(t >= 0.0 for t in stages.values())
    assert stages["sca_readout"] > 0.0 and stages["awm_chunk"] > 0.0 and stages["awm_scan"] > 0.0
    # the recorded calls are a subset of the timed region
    assert sum(stages.values()) <= wall * 1.02 + 0.05
    assert np.isfinite(sum(stages.values()))
