#!/usr/bin/env python3
"""Throughput of the Gecko SCA + AWM forward on one MI355X.

One step = one gecko_sca_awm_forward call over the whole 128K-token workload
(B=1, H=8, n=131072, c=2048, d=128, dv=256, bf16 inputs, fp32 accumulation,
bf16 output): memory chunk pass, memory scan (with its running denominator),
then the attention kernel with the fused readout. Inputs are synthetic
(seeded), and resident in HBM before the timed region starts.

Prints one JSON line. ``value`` is tokens/s (B * n / step time).
``roofline`` describes the attention kernel (the dominant one): algorithmic
FLOPs per launch over its mean duration, measured with HIP events recorded on
the library's stream between its kernels during the timed steps.
``awm_scan`` gives the memory scan's mean duration and its HBM rate, from the
algorithmic bytes and from the committed counter summary's measured bytes.
``cpu_baseline`` is the fp64 oracle timed on a bounded sample of the same
workload on this host (not a target).

``--workload`` picks the workload of the JSON line (default: the 128K-token
headline); ``variants.workloads`` times the other bf16 workloads (B4 H8 16K,
B1 H8 1M, B1 H4 4M tokens) with the same flop count and stage split.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (published)
PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector (published; counts packed FMA)
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E (published)
METRIC = "SCA+AWM fwd tokens/s at 128K tokens, c=2048; % of bf16 MFMA peak"
# committed counter summaries: (file, kernel sources it was measured on)
PMC_SCA = (os.path.join(ROOT, "profiles", "sca_bf16_128k_pmc.txt"), ("sca_bf16.hip", "gecko_device.hpp"))
PMC_SCAN = (os.path.join(ROOT, "profiles", "awm_scan_128k_pmc.txt"), ("awm_bf16.hip", "gecko_device.hpp"))
PMC_CEMA = (os.path.join(ROOT, "profiles", "cema_128k_pmc.txt"), ("cema.hip", "gecko_device.hpp"))
PMC_TDN = (os.path.join(ROOT, "profiles", "tdn_128k_pmc.txt"), ("tdn.hip", "gecko_device.hpp"))


def kernel_source_hash(sources) -> str:
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "chunked_attention_memory_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(summary, launch_key: str):
    """HBM bytes per launch of a kernel from its committed counter summary, or
    None if there is none or the kernel sources changed since it was taken."""
    path, sources = summary
    try:
        fields = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip().split()[0]
        if fields.get("source_hash") != kernel_source_hash(sources) or fields.get("workload") != launch_key:
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError, IndexError):
        return None


def cpu_baseline(host, w, budget_s: float):
    """Time the fp64 oracle on a bounded sample of the workload: the first m
    chunks of head 0 (of those ``host`` holds), m grown until one call takes
    most of the budget; if a whole head takes less, further whole heads until
    the budget is spent. Scaled to the workload's tokens/s (every token passes
    all H heads)."""
    import numpy as np

    import oracle

    p = host["params"]
    cores = len(os.sched_getaffinity(0))
    z, v = host["z"][0, 0], host["v"][0, 0]
    m_max = -(-z.shape[0] // w.c)  # chunks held on the host (all, or a leading sample)
    m = 1
    while True:
        ntok = min(m * w.c, z.shape[0])
        t0 = time.perf_counter()
        oracle.forward_head(z[:ntok], v[:ntok], p, 0, w.c)
        dt = time.perf_counter() - t0
        if ntok >= w.n or m >= m_max or dt >= 0.6 * budget_s:
            break
        m = min(m_max, max(2 * m, int(m * budget_s / max(dt, 1e-9))))
    t_total, head_tokens, heads = dt, ntok, 1
    while ntok >= w.n and heads < w.H and t_total < budget_s:
        t0 = time.perf_counter()
        oracle.forward_head(host["z"][0, heads], host["v"][0, heads], p, heads, w.c)
        t_total += time.perf_counter() - t0
        heads += 1
    value = head_tokens * heads / t_total / w.H
    what = (f"heads 0..{heads - 1} of {w.H}, all {w.nchunks} chunks" if ntok >= w.n
            else f"head 0 of {w.H}, first {m} of {w.nchunks} chunks")
    cpu, blas = host_cpu_and_blas()
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu, "blas": blas,
            "sample": f"fp64 oracle on {what} ({head_tokens * heads} head-tokens) in {t_total:.2f} s; "
                      f"head-tokens/s divided by {w.H} heads; numpy {np.__version__}, "
                      f"BLAS threads up to {cores} host cores"}


def host_cpu_and_blas():
    """The host CPU model (/proc/cpuinfo) and the BLAS library numpy calls."""
    import numpy as np

    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        info = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{info.get('name')} {info.get('version')}".strip()
        conf = info.get("openblas configuration")
        if conf:
            blas += f" ({conf})"
    except Exception:
        pass
    return cpu, blas


def time_variants(gecko, w, z, v, params, out, stream, args) -> dict:
    """After the headline's timed region, on the same resident inputs: the
    chunk-wise form (flag GECKO_CHUNKWISE) and the streaming forward with the
    sequence handed over in four calls of n/4 tokens (inputs pre-split into
    contiguous per-call tensors before timing). HIP events on the launch stream."""
    import torch

    steps = max(1, min(args.steps, 20))

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    tokens = w.B * w.n
    res = {}
    flags = gecko.GECKO_CHUNKWISE
    ws_cw = gecko.alloc_workspace(z, v, w.c, flags)
    ms = timed(lambda: gecko.gecko_sca_awm_forward(z, params, v, w.c, out=out, flags=flags, workspace=ws_cw,
                                                   stream=stream))
    res["chunkwise"] = {"ms_per_step": ms, "tokens_per_s": tokens / (ms / 1e3), "steps": steps}
    del ws_cw
    q = w.n // 4
    parts = [(z[:, :, i * q:(i + 1) * q].contiguous(), v[:, :, i * q:(i + 1) * q].contiguous()) for i in range(4)]
    outs = [torch.empty((w.B, w.H, q, w.dv), dtype=out.dtype, device=out.device) for _ in range(4)]
    st = gecko.Stream(w.B, w.H, w.d, w.dv, w.c, params)
    nbytes = gecko.gecko_stream_workspace_size(w.B, w.H, q, w.d, w.dv, w.c, gecko.GECKO_BF16)
    ws_st = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=out.device)

    def stream_step():
        st.pos = 0
        for (zp, vp), o in zip(parts, outs):
            st.forward(zp, vp, out=o, workspace=ws_st, stream=stream)

    ms = timed(stream_step)
    res["stream_4_calls"] = {"ms_per_step": ms, "tokens_per_s": tokens / (ms / 1e3), "steps": steps,
                             "calls_per_step": 4, "tokens_per_call": q}
    del parts, outs, ws_st
    res["backward"] = time_backward(gecko, w, z, v, params, stream, timed)
    res.update(time_backward_saved(gecko, w, z, v, params, stream, timed))
    res["cema"] = time_cema(gecko, stream, timed)
    res["tdn"] = time_tdn(gecko, stream, timed)
    return res


def time_backward(gecko, w, z, v, params, stream, timed) -> dict:
    """The backward of the headline layer (both parts) on its resident inputs
    and a resident N(0, 1) bf16 dL/dO: one gecko_backward call per step (it
    recomputes the memory scan and the attention row statistics itself). The
    roofline counts each product of the backward once
    (configs.backward_flop_count) against the bf16 MFMA peak."""
    import torch

    from chunked_attention_memory_amd import configs

    gen = torch.Generator(device="cuda")
    gen.manual_seed(91)
    do = torch.randn((w.B, w.H, w.n, w.dv), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    dz = torch.empty((w.B, w.H, w.n, w.d), dtype=torch.float32, device="cuda")
    dvt = torch.empty((w.B, w.H, w.n, w.dv), dtype=torch.float32, device="cuda")
    daff = torch.empty((8, w.H, w.d), dtype=torch.float32, device="cuda")
    nbytes = gecko.gecko_backward_workspace_size(w.B, w.H, w.n, w.d, w.dv, w.c, gecko.GECKO_BF16, gecko.GECKO_BF16)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    ms = timed(lambda: gecko.gecko_backward(z, params, v, do, w.c, dz=dz, dv=dvt, daff=daff, workspace=ws,
                                            stream=stream))
    flops = configs.backward_flop_count(w.n, w.c, w.d, w.dv)["total"] * w.B * w.H
    achieved = flops / (ms / 1e3) / 1e12
    del do, dz, dvt, daff, ws
    return {"workload": "bwd_" + w.name, "ms_per_step": ms, "tokens_per_s": w.B * w.n / (ms / 1e3),
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / PEAK_BF16_TFLOPS, "flops_per_call": flops},
            "workspace_bytes": nbytes}


def time_backward_saved(gecko, w, z, v, params, stream, timed) -> dict:
    """The training path of the headline layer (both parts): gecko_forward_train
    (the forward output plus the float32 attention output, per-query weight
    statistics and the kept memory pass) and gecko_backward_saved, which
    reuses them in place of the attention statistics pass and the memory
    pass and scan. Timed alone ("backward_saved", the statistics made once
    before timing) and as a forward + backward pair ("train_step_saved").
    Same resident dL/dO and flop accounting as the recomputing backward (the
    forward's algorithmic flops added for the pair)."""
    import torch

    from chunked_attention_memory_amd import configs

    gen = torch.Generator(device="cuda")
    gen.manual_seed(91)
    do = torch.randn((w.B, w.H, w.n, w.dv), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    dz = torch.empty((w.B, w.H, w.n, w.d), dtype=torch.float32, device="cuda")
    dvt = torch.empty((w.B, w.H, w.n, w.dv), dtype=torch.float32, device="cuda")
    daff = torch.empty((8, w.H, w.d), dtype=torch.float32, device="cuda")
    out = torch.empty((w.B, w.H, w.n, w.dv), dtype=torch.bfloat16, device="cuda")
    o_sca = torch.empty((w.B, w.H, w.n, w.dv), dtype=torch.float32, device="cuda")
    stats = torch.empty((w.B, w.H, w.n, 2), dtype=torch.float32, device="cuda")
    mbytes = gecko.gecko_memory_saved_size(w.B, w.H, w.n, w.d, w.dv, w.c)
    mem = torch.empty(max(mbytes, 256), dtype=torch.uint8, device="cuda")
    nbytes = gecko.gecko_backward_saved_workspace_size(w.B, w.H, w.n, w.d, w.dv, w.c, gecko.GECKO_BF16,
                                                       gecko.GECKO_BF16)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")

    def fwd():
        gecko.gecko_forward_train(z, params, v, w.c, out=out, o_sca=o_sca, stats=stats, mem_saved=mem,
                                  stream=stream)

    def bwd():
        gecko.gecko_backward_saved(z, params, v, do, o_sca, stats, w.c, dz=dz, dv=dvt, daff=daff, workspace=ws,
                                   mem_saved=mem, stream=stream)

    fwd()
    ms_b = timed(bwd)
    ms_t = timed(lambda: (fwd(), bwd()))
    fl_b = configs.backward_flop_count(w.n, w.c, w.d, w.dv)["total"] * w.B * w.H
    fl_f = configs.workload_flops(w)["total"]
    del do, dz, dvt, daff, out, o_sca, stats, mem, ws
    res = {}
    for key, ms, fl in (("backward_saved", ms_b, fl_b), ("train_step_saved", ms_t, fl_b + fl_f)):
        achieved = fl / (ms / 1e3) / 1e12
        res[key] = {"workload": ("bwd_" if key == "backward_saved" else "fwd_bwd_") + w.name, "ms_per_step": ms,
                    "tokens_per_s": w.B * w.n / (ms / 1e3),
                    "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                                 "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "flops_per_call": fl}}
    res["backward_saved"]["workspace_bytes"] = nbytes
    res["backward_saved"]["mem_saved_bytes"] = mbytes
    return res


def time_tdn(gecko, stream, timed) -> dict:
    """Timestep decay normalisation at a 7B-scale layer: B1, 131072 tokens,
    D 4096 in 64 groups, bf16 in and out. HBM-bound: the algorithmic traffic
    is x read once and y written once (the kernels read x twice: statistics,
    then the normalisation)."""
    import torch

    B, n, D, G = 1, 131072, 4096, 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(71)
    x = torch.randn((B, n, D), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    gamma = torch.ones(D, dtype=torch.float32, device="cuda")
    shift = torch.zeros(D, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    ws = torch.empty(gecko.gecko_tdn_workspace_size(B, n, D, G), dtype=torch.uint8, device="cuda")
    ms = timed(lambda: gecko.gecko_tdn_forward(x, gamma, shift, G, 0.99, 0.999, out=y, workspace=ws,
                                               stream=stream))
    alg = 4.0 * B * n * D
    achieved = alg / (ms / 1e3) / 1e9
    return {"workload": "tdn_bf16_B1_n128k_D4096_G64", "ms_per_step": ms, "tokens_per_s": B * n / (ms / 1e3),
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": achieved / PEAK_HBM_GBPS,
                         "traffic": read_traffic(PMC_TDN, "tdn_bf16_B1_n128k_D4096_G64:bf16"),
                         "algorithmic_bytes": alg}}


def time_cema(gecko, stream, timed) -> dict:
    """CEMA at a 7B-scale layer: B1, 131072 tokens, D 4096, h 16, bf16 in and
    out. The kernels are plain FMA arithmetic: 12 h flops per (token, input
    dimension) for the method's one pass (input scale, complex multiply-add,
    projection), against the fp32 vector peak."""
    import torch

    from chunked_attention_memory_amd import inputs

    B, n, D, h = 1, 131072, 4096, 16
    dev = inputs.make_cema_inputs_device(B, n, D, h, "bf16", seed=0, tag=60)
    x, p = dev["x"], dev["params"]
    y = torch.empty_like(x)
    ws = torch.empty(max(gecko.gecko_cema_workspace_size(B, n, D, h), 256), dtype=torch.uint8, device=x.device)
    ms = timed(lambda: gecko.gecko_cema_forward(x, p, out=y, workspace=ws, stream=stream))
    flops = 12.0 * h * B * n * D
    achieved = flops / (ms / 1e3) / 1e12
    return {"workload": "cema_bf16_B1_n128k_D4096_h16", "ms_per_step": ms, "tokens_per_s": B * n / (ms / 1e3),
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VECTOR_TFLOPS, "unit": "TFLOP/s",
                         "frac": achieved / PEAK_FP32_VECTOR_TFLOPS,
                         "traffic": read_traffic(PMC_CEMA, "cema_bf16_B1_n128k_D4096_h16:bf16"),
                         "flops_per_launch": flops, "algorithmic_bytes": 4.0 * B * n * D}}


def time_other_workloads(gecko, skip: int, stream, out_dtype) -> dict:
    """The other bf16 workloads (B4 H8 16K; B1 H8 1M; B1 H4 4M tokens, all
    c 2048, d 128, dv 256), one after the other on inputs drawn on the device
    (same recipe), each freed before the next: ms per forward, tokens/s, the
    fraction of the bf16 peak by the same flop count, and the per-stage split
    from the library's stage events (the memory scan runs N - 2 dependent
    steps: 6, 510 and 2046)."""
    import torch

    from chunked_attention_memory_amd import configs, inputs

    res = {}
    for key in (1, 3, 4):
        if key == skip:
            continue
        w = configs.WORKLOADS[key]
        dev = inputs.make_inputs_device(w.B, w.H, w.n, w.d, w.dv, w.dtype, seed=0, tag=key)
        z, v = dev["z"], dev["v"]
        params = {k: torch.from_numpy(a).cuda() for k, a in dev["params"].items()}
        steps, warmup = (10, 3) if key == 1 else (3, 1)
        r = measure_forward(gecko, w, z, v, params, out_dtype, steps, warmup, stream)
        flops = configs.workload_flops(w)["total"]
        res[w.name] = {"B": w.B, "H": w.H, "n": w.n, "c": w.c, "ms_per_step": r["ms"],
                       "tokens_per_s": w.B * w.n / (r["ms"] / 1e3),
                       "pct_of_bf16_peak": flops / (r["ms"] / 1e3) / (PEAK_BF16_TFLOPS * 1e12) * 100.0,
                       "flops_per_step": flops, "stage_ms": r["stage_ms"], "steps": steps, "warmup": warmup,
                       "finite": r["finite"]}
        del dev, z, v, params, r
        torch.cuda.empty_cache()
    return res


def measure_forward(gecko, w, z, v, params, out_dtype, steps, warmup, stream, per_call=False) -> dict:
    """Time ``steps`` forwards (after ``warmup`` untimed ones) on resident
    inputs: wall clock around the whole timed region (synchronised on both
    sides), HIP events on the launch stream, the library's stage events, and
    optionally each call again on its own (median and minimum)."""
    import torch

    out = torch.empty((w.B, w.H, w.n, w.dv), dtype=out_dtype, device=z.device)
    ws = gecko.alloc_workspace(z, v, w.c, stream=stream)
    timer = gecko.Timer(max(steps, 1))

    def step(tm=None):
        gecko.gecko_sca_awm_forward(z, params, v, w.c, out=out, workspace=ws, stream=stream, timer=tm)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step(timer)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    stages, calls = timer.read()
    timer.close()
    res = {"ms": wall * 1e3 / steps, "ms_events": ev0.elapsed_time(ev1) / steps,
           "stage_ms": {k: v_ / calls for k, v_ in stages.items()} if calls else {},
           "finite": bool(torch.isfinite(out).all())}
    if per_call:
        evs = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        call_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        res["per_call_ms"] = {"median": call_ms[len(call_ms) // 2], "min": call_ms[0], "calls": len(call_ms)}
    res["out"] = out
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, choices=(1, 2, 3, 4), default=2,
                    help="workload of the JSON line: 2 is the 128K-token headline (default); 1 B4 H8 16K, "
                         "3 B1 H8 1M, 4 B1 H4 4M tokens")
    ap.add_argument("--out-dtype", choices=("bf16", "f32"), default="bf16")
    ap.add_argument("--cpu-budget", type=float, default=30.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the variant timings (other workloads, chunk-wise form, streaming, backward, "
                         "CEMA, TDN), e.g. under a profiler")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB "
                         "(a known-size kernel for scaling HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every (batch, head) is independent; see the sharding notes). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch

    from chunked_attention_memory_amd import configs, gecko, inputs

    w = configs.WORKLOADS[args.workload]
    flops = configs.workload_flops(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.perf_counter()
    if args.workload <= 2:
        host = inputs.make_inputs(w.B, w.H, w.n, w.d, w.dv, w.dtype, seed=0, tag=args.workload)
        z, v, params = gecko.to_device_inputs(host, device=dev)
    else:
        # too large to draw on the host quickly: the same recipe on the device
        d_in = inputs.make_inputs_device(w.B, w.H, w.n, w.d, w.dv, w.dtype, seed=0, tag=args.workload)
        z, v = d_in["z"], d_in["v"]
        params = {k: torch.from_numpy(a).to(dev) for k, a in d_in["params"].items()}
        host = None
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    out_dt = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32
    stream = torch.cuda.current_stream()

    r = measure_forward(gecko, w, z, v, params, out_dt, args.steps, args.warmup, stream, per_call=True)
    out = r.pop("out")

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    variants = None
    if not args.no_variants:
        variants = {"workloads": time_other_workloads(gecko, args.workload, stream, out_dt)}
        if args.workload == 2:
            variants.update(time_variants(gecko, w, z, v, params, out, stream, args))

    ms_per_step = r["ms"]
    tokens = w.B * w.n
    value = tokens / (ms_per_step / 1e3)
    pct_peak = flops["total"] / (ms_per_step / 1e3) / (PEAK_BF16_TFLOPS * 1e12) * 100.0
    stage_ms = r["stage_ms"]
    sca_ms = stage_ms.get("sca_readout")
    sca_flops = flops["sca"] + flops["awm_read"]
    achieved = sca_flops / (sca_ms / 1e3) / 1e12 if sca_ms else None
    launch_key = f"{w.name}:{args.out_dtype}"
    traffic = read_traffic(PMC_SCA, launch_key)
    scan_ms = stage_ms.get("awm_scan")
    rows = w.B * w.H * max(w.nchunks - 2, 0)
    # per (batch*head, chunk): G^T fp32 and H bf16 read, chunk max/sum read, bf16 state written
    scan_alg = rows * (w.d * w.dv * 4 + w.d * w.d * 2 + 2 * w.d * 4 + w.d * w.dv * 2)
    scan_meas = read_traffic(PMC_SCAN, launch_key)

    res = {
        "metric": METRIC if args.workload == 2 else "SCA+AWM fwd tokens/s; % of bf16 MFMA peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: L2-normalised Gaussian Z', silu(N(0,1)) V, N(1,.1)/N(0,.1) affine vectors)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "n": w.n, "c": w.c, "d": w.d, "dv": w.dv,
                   "in_dtype": "bf16", "out_dtype": args.out_dtype, "accumulate": "fp32"},
        "pct_of_bf16_peak": pct_peak,
        "flops_per_step": flops["total"],
        "peak_tflops_used": PEAK_BF16_TFLOPS,
        "ms_per_step_events": r["ms_events"],
        "per_call_ms": r["per_call_ms"],
        "stage_ms": stage_ms,
        "output_finite": r["finite"],
        "roofline": {"kernel": "sca_bf16_kernel (attention + readout)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": (achieved / PEAK_BF16_TFLOPS) if achieved else None,
                     "traffic": traffic, "flops_per_launch": sca_flops},
        "awm_scan": {"kernel": "awm_scan_bf16_kernel", "ms": scan_ms,
                     "algorithmic_bytes": scan_alg,
                     "algorithmic_GBps": scan_alg / (scan_ms / 1e3) / 1e9 if scan_ms else None,
                     "hbm_bytes": scan_meas,
                     "hbm_GBps": scan_meas / (scan_ms / 1e3) / 1e9 if (scan_meas and scan_ms) else None},
        "input_gen_s": gen_s,
    }
    if variants is not None:
        res["variants"] = variants
    if not args.no_cpu_baseline:
        if host is None:
            # the oracle's sample comes from head 0's first chunks on the device
            m = max(1, min(w.nchunks, 16))
            host = {"z": z[:, :1, :m * w.c].float().cpu().numpy(), "v": v[:, :1, :m * w.c].float().cpu().numpy(),
                    "params": d_in["params"]}
        res["cpu_baseline"] = cpu_baseline(host, w, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
