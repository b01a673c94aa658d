#!/usr/bin/env python3
"""Benchmark of the libwkv hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one wkv_forward over the workload (B=1, T=65536, C=5120 bfloat16 by
default: 64K tokens at the 14B model's width, the largest workload that fits one
GPU).  The timed region holds K steps with inputs resident in HBM, bracketed by
torch.cuda.synchronize().  Prints one JSON line: elements/s (B*T*C per second), the
HBM roofline of the forward kernel (algorithmic bytes: read k, v, write y) measured
with HIP events on the launch stream, and the float64 CPU oracle timed on the host
as a reported baseline.  The other workloads (the 8K-context float32 forward with its
own roofline, the 169M width, the backward and the fused time-mixing parts at the
8K-context and 64K-token shapes, causal linear attention at the linear-transformer
page's shapes, batched decode step) are timed the same way and reported under
"other_workloads".  Every case first runs its kernel back-to-back for SETTLE_S seconds
(untimed; the GPU's power management needs about 10 ms under this load to leave its
start-up transient), then its warmup steps, then its timed steps.  Every forward workload is timed on its seeded NumPy inputs
(workloads.forward_inputs), the inputs the parity tests check.
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}  # MI355X dense matrix-core peaks, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# sources of the forward kernel and its launch path (the committed counter runs are valid
# for the kernel built from exactly these)
KERNEL_SOURCES = ("wkv_forward.hip", "wkv_rows.h", "wkv_chain.h", "wkv_device.h", "wkv_kernels.h",
                  "libwkv_api.cpp")
BACKWARD_SOURCES = KERNEL_SOURCES + ("wkv_backward.hip",)
LA_SOURCES = ("la_forward.hip", "wkv_rows.h", "wkv_chain.h", "wkv_device.h", "wkv_kernels.h", "libwkv_api.cpp")
STEP_SOURCES = ("wkv_step.hip", "wkv_device.h", "wkv_kernels.h", "libwkv_api.cpp")


def strip_comments(text: str) -> str:
    """C++ source without its comments and blank lines, each line right-trimmed, so that
    editing a comment leaves the hash of the code unchanged."""
    out = []
    i, n = 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":  # string or character literal, copied with its escapes
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = ("".join(out)).split("\n")
    return "\n".join(l.rstrip() for l in lines if l.strip())


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "rwkv_linear_attention_libwkv_amd", "csrc", name)) as f:
            h.update(strip_comments(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(workload: str, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("source_hash") != kernel_source_hash(sources):
        return None
    return entry.get("bytes_per_launch")


SETTLE_S = 0.1  # untimed back-to-back work before every case's warmup steps
TIMED_LOG = []  # (settle calls, warmup calls, timed calls) of every time_launches, in order


def settle(fn, seconds=SETTLE_S, batch=8):
    """Run fn back-to-back (batches of `batch` launches, synchronized per batch) until `seconds`
    of wall time have passed; returns the number of launches.  Under a heavy sustained load the
    MI355X's power management takes about 10 ms to settle: a 64K-token bf16 forward measured
    4000 launches in a row ran 428 -> 525 -> 458 us over its first 20 launches and 401-403 us
    (median of every later block of 250) after them.  Timing starts in the settled state."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            fn()
        n += batch
        torch.cuda.synchronize()
    return n


def time_launches(fn, steps, warmup):
    """Settle, run fn warmup times, then time `steps` calls with HIP events; returns
    (total_s, per_call_s)."""
    import torch

    TIMED_LOG.append((settle(fn), warmup, steps))
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = start.elapsed_time(end) / 1e3
    return wall, ev / steps


def per_launch_stats(fn, n=20, flush=None):
    """Median and min of n single launches, each timed with its own HIP events on the launch
    stream, from an idle GPU.  flush: a callable run before every launch, e.g. a write of a
    buffer larger than the 256 MB last-level cache so that the launch reads its inputs from HBM;
    the start event then follows the flush on the stream with no host wait between, so the
    events bracket the launch itself rather than the idle queue's start-up."""
    import numpy as np
    import torch

    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(n):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / 1e3)
    return {"median_s": float(np.median(ts)), "min_s": float(np.min(ts)), "n": n}


CACHE_FLUSH_BYTES = 512 << 20  # twice the MI355X last-level (MALL) cache


def cache_flusher():
    import torch

    buf = torch.empty(CACHE_FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    state = {"i": 0}

    def flush():
        state["i"] += 1
        buf.fill_(float(state["i"]))

    return flush, buf


_INPUTS = {}  # seeded inputs drawn once per workload (the CPU baseline and the GPU run share them)


def inputs_of(spec):
    from rwkv_linear_attention_libwkv_amd import workloads

    if spec.name not in _INPUTS:
        _INPUTS[spec.name] = workloads.forward_inputs(spec)
    return _INPUTS[spec.name]


def roofline_of(achieved_gbps, traffic):
    return {"bound": "hbm", "achieved": achieved_gbps, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved_gbps / HBM_PEAK_GBS, "traffic": traffic}


def forward_case(spec, steps, warmup, gen="numpy"):
    import numpy as np
    import torch

    from rwkv_linear_attention_libwkv_amd import libwkv, workloads

    dt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
    if gen == "numpy":
        inp = inputs_of(spec)
        w = torch.from_numpy(inp["w"]).cuda()
        u = torch.from_numpy(inp["u"]).cuda()
        k = torch.from_numpy(inp["k"]).cuda().to(dt)
        v = torch.from_numpy(inp["v"]).cuda().to(dt)
    else:  # same distributions drawn on the device (faster for the largest tensors)
        rng = np.random.default_rng(spec.seed)
        w_np, u_np = workloads.channel_params(rng, (spec.C,), spec.w_raw_lo, spec.w_raw_hi, spec.u_std)
        w, u = torch.from_numpy(w_np).cuda(), torch.from_numpy(u_np).cuda()
        g = torch.Generator(device="cuda")
        g.manual_seed(spec.seed)
        shape = (spec.B, spec.T, spec.C)
        k = (torch.randn(shape, generator=g, device="cuda") * spec.k_std).to(dt)
        v = (torch.randn(shape, generator=g, device="cuda") * spec.v_std).to(dt)
    y = torch.empty_like(k)
    ws = libwkv.new_workspace(spec.B, spec.T, spec.C, dt)
    need = ws is not None

    def fn():
        libwkv.wkv_forward(w, u, k, v, y=y, workspace=ws)

    wall, per_call = time_launches(fn, steps, warmup)
    elt = 4 if spec.dtype == "f32" else 2
    bytes_per_launch = 3 * elt * spec.elements  # read k, v; write y
    single = per_launch_stats(fn)
    cold = None
    if bytes_per_launch < CACHE_FLUSH_BYTES:  # fits in the last-level cache: also time it cold
        flush, buf = cache_flusher()
        cold = per_launch_stats(fn, flush=flush)
        cold["achieved_GBps_median"] = bytes_per_launch / cold["median_s"] / 1e9
        del buf
    if need:
        assert libwkv.lookback_error(ws) == 0, "look-back gave up"
    out = {
        "workload": spec.name,
        "elements": spec.elements,
        "seconds": wall,
        "per_launch_s": per_call,
        "per_launch_single": single,
        "elements_per_s": spec.elements / per_call,
        "algorithmic_bytes_per_launch": bytes_per_launch,
        "achieved_GBps": bytes_per_launch / per_call / 1e9,
        "algo": "chunked" if need else "seq",
        "inputs": "seeded NumPy draws (workloads.forward_inputs)" if gen == "numpy" else "seeded torch draws on the GPU",
    }
    if spec.elements >= 1e8:  # the long-sequence workloads carry their own roofline
        out["roofline"] = roofline_of(out["achieved_GBps"], measured_traffic(spec.name))
    if cold is not None:
        out["cold_cache"] = cold
    del k, v, y, ws
    torch.cuda.empty_cache()
    return out


def backward_case(spec, steps, warmup):
    """wkv_backward over a forward workload's shape with gy ~ N(0, 1) drawn on the device."""
    import numpy as np
    import torch

    from rwkv_linear_attention_libwkv_amd import libwkv, workloads

    dt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
    rng = np.random.default_rng(spec.seed)
    w_np, u_np = workloads.channel_params(rng, (spec.C,), spec.w_raw_lo, spec.w_raw_hi, spec.u_std)
    w, u = torch.from_numpy(w_np).cuda(), torch.from_numpy(u_np).cuda()
    g = torch.Generator(device="cuda")
    g.manual_seed(spec.seed)
    shape = (spec.B, spec.T, spec.C)
    k = (torch.randn(shape, generator=g, device="cuda") * spec.k_std).to(dt)
    v = (torch.randn(shape, generator=g, device="cuda") * spec.v_std).to(dt)
    gy = torch.randn(shape, generator=g, device="cuda").to(dt)
    gk, gv = torch.empty_like(k), torch.empty_like(k)
    gw = torch.empty((spec.B, spec.C), device="cuda")
    gu = torch.empty_like(gw)
    ws = libwkv.new_backward_workspace(spec.B, spec.T, spec.C, dt)

    def fn():
        libwkv.wkv_backward(w, u, k, v, gy, gk=gk, gv=gv, gw=gw, gu=gu, workspace=ws)

    wall, per_call = time_launches(fn, steps, warmup)
    assert libwkv.lookback_error(ws) == 0, "look-back gave up"
    # the training pair: forward that saves the scan's states, backward that starts from them
    y = torch.empty_like(k)
    fws = libwkv.new_workspace(spec.B, spec.T, spec.C, dt, "chunked", 0)
    _, saved = libwkv.wkv_forward_save(w, u, k, v, y=y, workspace=fws)

    def train():
        libwkv.wkv_forward_save(w, u, k, v, y=y, saved=saved, workspace=fws)
        libwkv.wkv_backward(w, u, k, v, gy, saved=saved, gk=gk, gv=gv, gw=gw, gu=gu, workspace=ws)

    _, per_train = time_launches(train, steps, warmup)

    def saved_backward():  # the backward scan (and its small per-lane reduction) alone
        libwkv.wkv_backward(w, u, k, v, gy, saved=saved, gk=gk, gv=gv, gw=gw, gu=gu, workspace=ws)

    _, per_saved = time_launches(saved_backward, steps, warmup)
    assert libwkv.lookback_error(ws) == 0 and libwkv.lookback_error(fws) == 0, "look-back gave up"
    elt = 4 if spec.dtype == "f32" else 2
    bytes_per_launch = 5 * elt * spec.elements + 8 * spec.B * spec.C  # read k, v, gy; write gk, gv, gw, gu
    out = {
        "workload": spec.name.replace("wkv_fwd", "wkv_bwd"),
        "elements": spec.elements,
        "per_launch_s": per_call,
        "elements_per_s": spec.elements / per_call,
        "algorithmic_bytes_per_launch": bytes_per_launch,
        "achieved_GBps": bytes_per_launch / per_call / 1e9,
        "scan_kernel_traffic_bytes": measured_traffic(spec.name.replace("wkv_fwd", "wkv_bwd"), BACKWARD_SOURCES),
        "train_pair_s": per_train,
        "train_pair_note": "wkv_forward_save + wkv_backward_saved (y, then all four gradients)",
        "train_pair_algorithmic_GBps": (bytes_per_launch + 3 * elt * spec.elements) / per_train / 1e9,
        "backward_saved_s": per_saved,
        "backward_saved_note": "wkv_backward_saved: the backward scan kernel and its per-lane reduction",
        "roofline": roofline_of(bytes_per_launch / per_saved / 1e9,
                                measured_traffic(spec.name.replace("wkv_fwd", "wkv_bwd"), BACKWARD_SOURCES)),
    }
    del k, v, gy, gk, gv, ws, y, fws, saved
    torch.cuda.empty_cache()
    return out


def mix_case(spec, steps, warmup):
    """The time-mixing block's fused parts at a forward workload's shape: the token shift
    (three mixes) and the gated forward z = sigmoid(r) * WKV, against the plain forward."""
    import numpy as np
    import torch

    from rwkv_linear_attention_libwkv_amd import libwkv, workloads

    dt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
    elt = 4 if spec.dtype == "f32" else 2
    rng = np.random.default_rng(spec.seed)
    w_np, u_np = workloads.channel_params(rng, (spec.C,), spec.w_raw_lo, spec.w_raw_hi, spec.u_std)
    w, u = torch.from_numpy(w_np).cuda(), torch.from_numpy(u_np).cuda()
    g = torch.Generator(device="cuda")
    g.manual_seed(spec.seed)
    shape = (spec.B, spec.T, spec.C)
    k = (torch.randn(shape, generator=g, device="cuda") * spec.k_std).to(dt)
    v = (torch.randn(shape, generator=g, device="cuda") * spec.v_std).to(dt)
    r = torch.randn(shape, generator=g, device="cuda").to(dt)
    z = torch.empty_like(k)
    ws = libwkv.new_workspace(spec.B, spec.T, spec.C, dt)
    _, per_gated = time_launches(lambda: libwkv.wkv_forward_gated(w, u, k, v, r, z=z, workspace=ws), steps, warmup)
    mu = torch.rand((3, spec.C), generator=g, device="cuda")
    out = torch.empty((3,) + shape, dtype=dt, device="cuda")
    _, per_shift = time_launches(lambda: libwkv.wkv_token_shift(k, mu, out=out), steps, warmup)
    # the token shift's backward (out reused as dL/dout)
    gx = torch.empty_like(k)
    gmu = torch.empty((3, spec.B, spec.C), device="cuda")
    gprev = torch.empty((spec.B, spec.C), dtype=dt, device="cuda")
    sws = torch.empty(libwkv.lib.wkv_token_shift_backward_workspace_bytes(spec.B, spec.T, spec.C, 3),
                      dtype=torch.uint8, device="cuda")
    _, per_shift_bwd = time_launches(lambda: libwkv.wkv_token_shift_backward(k, mu, out, gx=gx, gmu=gmu, gprev=gprev,
                                                                             workspace=sws), steps, warmup)
    n = spec.elements
    res = {
        "workload": spec.name.replace("wkv_fwd", "wkv_mix"),
        "gated_forward_s": per_gated,
        "gated_forward_algorithmic_GBps": 4 * elt * n / per_gated / 1e9,  # read k, v, r; write z
        "token_shift3_s": per_shift,
        "token_shift3_algorithmic_GBps": 4 * elt * n / per_shift / 1e9,  # read x; write three mixes
        "token_shift3_backward_s": per_shift_bwd,
        "token_shift3_backward_algorithmic_GBps": 5 * elt * n / per_shift_bwd / 1e9,  # read x, 3 g; write gx
    }
    # each call against the HBM peak (algorithmic bytes; no counter run is kept for these)
    res["rooflines"] = {op: roofline_of(res[op + "_algorithmic_GBps"], None)
                        for op in ("gated_forward", "token_shift3", "token_shift3_backward")}
    del k, v, r, z, ws, out, gx, gmu, gprev, sws
    torch.cuda.empty_cache()
    return res


def la_case(spec, steps, warmup):
    """wkv_linear_attention on one of the linear-transformer page's shapes."""
    import torch

    from rwkv_linear_attention_libwkv_amd import libwkv

    from rwkv_linear_attention_libwkv_amd import workloads

    dt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
    inp = workloads.linear_attention_inputs(spec)  # the seeded draws the parity tests use
    q, k, v = (torch.from_numpy(inp[n]).cuda().to(dt) for n in ("q", "k", "v"))
    del inp
    out = torch.empty_like(v)
    ws = libwkv.new_la_workspace(spec.BH, spec.N, spec.D, spec.M, dt)
    fn = lambda: libwkv.linear_attention(q, k, v, out=out, workspace=ws)  # noqa: E731
    _, per = time_launches(fn, steps, warmup)
    elt = 4 if spec.dtype == "f32" else 2
    nbytes = spec.tokens * (2 * spec.D + 2 * spec.M) * elt  # read q, k, v; write out
    cold = None
    if nbytes < CACHE_FLUSH_BYTES:
        flush, buf = cache_flusher()
        cold = per_launch_stats(fn, flush=flush)
        cold["achieved_GBps_median"] = nbytes / cold["median_s"] / 1e9
        del buf
    # similarities (causal half of each 32 x 32 block), their product with v, the carried state
    # product, and the sub-chunk aggregate (counted twice: aggregate pass and output pass)
    flops = 2 * spec.tokens * (16 * spec.D + 16 * spec.M + 3 * spec.D * spec.M)
    res = {
        "workload": spec.name,
        "per_call_s": per,
        "tokens_per_s": spec.tokens / per,
        "algorithmic_bytes_per_call": nbytes,
        "achieved_GBps": nbytes / per / 1e9,
        "useful_TFLOPs": flops / per / 1e12,
        "traffic_bytes_per_call": measured_traffic(spec.name, LA_SOURCES),
        "inputs": "seeded NumPy draws (workloads.linear_attention_inputs)",
    }
    res["roofline"] = roofline_of(res["achieved_GBps"], res["traffic_bytes_per_call"])
    # the contractions against the dense MFMA peak of their operand type
    mfma_peak = MFMA_PEAK_TFLOPS["f32" if spec.dtype == "f32" else "bf16"]
    res["mfma"] = {"achieved": res["useful_TFLOPs"], "peak": mfma_peak, "unit": "TFLOP/s",
                   "frac": res["useful_TFLOPs"] / mfma_peak}
    if cold is not None:
        res["cold_cache"] = cold
    assert libwkv.lookback_error(ws) == 0, "look-back gave up"
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return res


def step_case(spec, steps, warmup):
    import torch

    from rwkv_linear_attention_libwkv_amd import libwkv, workloads

    w_np, u_np = workloads.step_params(spec)
    w, u = torch.from_numpy(w_np).cuda(), torch.from_numpy(u_np).cuda()
    a, b, p = libwkv.empty_state((spec.N, spec.G, spec.C))
    for s in range(spec.prefix):  # the seeded prefix builds the starting state (not timed)
        k, v = workloads.step_kv(spec, s, device="cuda")
        libwkv.wkv_step(w, u, k, v, a, b, p)
    kv = [workloads.step_kv(spec, spec.prefix + s, device="cuda") for s in range(spec.steps)]
    y = torch.empty_like(kv[0][0])
    torch.cuda.synchronize()

    def one_decode():  # the 16 successive steps of the workload
        for k, v in kv:
            libwkv.wkv_step(w, u, k, v, a, b, p, y=y)

    wall, per_call = time_launches(one_decode, max(1, steps // 4), 1)
    lane_steps = spec.lanes * spec.steps
    bytes_per_step = 30 * spec.lanes  # k, v 2+2, a b p 12 read + 12 written, y 2
    out = {
        "workload": spec.name,
        "lane_steps": lane_steps,
        "per_decode_s": per_call,
        "per_step_launch_s": per_call / spec.steps,
        "lane_steps_per_s": lane_steps / per_call,
        "algorithmic_bytes_per_launch": bytes_per_step,
        "achieved_GBps": bytes_per_step / (per_call / spec.steps) / 1e9,
    }
    out["roofline"] = roofline_of(out["achieved_GBps"], measured_traffic(spec.name, STEP_SOURCES))
    del kv, a, b, p, y
    torch.cuda.empty_cache()
    return out


def decode_graph_case(spec, reps):
    """Decoding at a small batch, where launches rather than bytes set the pace: the workload's
    successive steps called one by one from Python, and the same steps captured once in a HIP
    graph (torch.cuda.CUDAGraph) and replayed, on the same buffers."""
    import torch

    from rwkv_linear_attention_libwkv_amd import libwkv, workloads

    w_np, u_np = workloads.step_params(spec)
    w, u = torch.from_numpy(w_np).cuda(), torch.from_numpy(u_np).cuda()
    a, b, p = libwkv.empty_state((spec.N, spec.G, spec.C))
    for s in range(spec.prefix):
        k, v = workloads.step_kv(spec, s, device="cuda")
        libwkv.wkv_step(w, u, k, v, a, b, p)
    kv = [workloads.step_kv(spec, spec.prefix + s, device="cuda") for s in range(spec.steps)]
    ys = [torch.empty_like(kv[0][0]) for _ in range(spec.steps)]

    def decode():
        for (k, v), y in zip(kv, ys):
            libwkv.wkv_step(w, u, k, v, a, b, p, y=y)

    _, per_eager = time_launches(decode, reps, 3)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode()
    _, per_graph = time_launches(graph.replay, reps, 3)
    bytes_per_step = 30 * spec.lanes
    out = {
        "workload": spec.name,
        "steps_per_decode": spec.steps,
        "eager_per_step_s": per_eager / spec.steps,
        "graph_per_step_s": per_graph / spec.steps,
        "graph_lane_steps_per_s": spec.lanes * spec.steps / per_graph,
        "graph_achieved_GBps": bytes_per_step / (per_graph / spec.steps) / 1e9,
        "note": "16 wkv_step calls per decode; eager: one Python call each; graph: one replay of all 16",
    }
    del graph, kv, ys, a, b, p
    torch.cuda.empty_cache()
    return out


_CPU_INPUTS = None  # the oracle sample, inherited by the forked workers of cpu_baseline


def _oracle_slice(sl):
    """Worker of cpu_baseline: wkv_recurrent on channels [c0, c1) of the first n_tok tokens."""
    from oracle import wkv_recurrent

    c0, c1, n_tok = sl
    w, u, k, v = _CPU_INPUTS
    t0 = time.perf_counter()
    wkv_recurrent(w[c0:c1], u[c0:c1], k[:, :n_tok, c0:c1], v[:, :n_tok, c0:c1])
    return time.perf_counter() - t0


def _cpu_model():
    """lscpu's model name (falls back to /proc/cpuinfo)."""
    import subprocess

    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, budget_s=20.0, max_workers=16):
    """The float64 oracle (wkv_recurrent) on a bounded sample of the workload, on the host:
    one process, then the same sample split by channels over the cores this process may use,
    at most max_workers forked processes (16: the host share of one GPU on the boxes this
    runs on, whatever the affinity mask shows).  Must run before anything touches the GPU (the
    workers are forked)."""
    import multiprocessing

    import numpy as np

    from oracle import wkv_recurrent
    from rwkv_linear_attention_libwkv_amd import workloads

    global _CPU_INPUTS
    inp = inputs_of(spec)
    # probe the cost per token, then size the sample (all lanes, leading tokens) to the budget
    t0 = time.perf_counter()
    wkv_recurrent(inp["w"], inp["u"], inp["k"][:, :64], inp["v"][:, :64])
    per_token = (time.perf_counter() - t0) / 64
    n_tok = int(min(spec.T, max(64, budget_s / max(per_token, 1e-9))))
    t0 = time.perf_counter()
    wkv_recurrent(inp["w"], inp["u"], inp["k"][:, :n_tok], inp["v"][:, :n_tok])
    dt = time.perf_counter() - t0
    elements = spec.B * n_tok * spec.C
    single = {"value": elements / dt, "unit": "elements/s", "cores": 1, "seconds": dt}

    affinity = len(os.sched_getaffinity(0))
    n = max(1, min(max_workers, affinity, spec.C))
    bounds = np.linspace(0, spec.C, n + 1).astype(int)
    slices = [(int(bounds[i]), int(bounds[i + 1]), n_tok) for i in range(n)]
    _CPU_INPUTS = (inp["w"], inp["u"], inp["k"], inp["v"])
    with multiprocessing.get_context("fork").Pool(n) as pool:
        pool.map(_oracle_slice, [(0, 1, 1)] * n)  # start every worker before the clock
        t0 = time.perf_counter()
        pool.map(_oracle_slice, slices, chunksize=1)
        wall = time.perf_counter() - t0
    _CPU_INPUTS = None
    # the O(T^2) definition, on the smallest workload only
    from oracle import wkv_direct

    small = workloads.forward_inputs(workloads.FWD_SMALL)
    t0 = time.perf_counter()
    wkv_direct(small["w"], small["u"], small["k"], small["v"])
    dt_direct = time.perf_counter() - t0
    direct = {"value": workloads.FWD_SMALL.elements / dt_direct, "unit": "elements/s", "cores": 1,
              "sample": f"wkv_direct (float64 NumPy, the O(T^2) definition) on {workloads.FWD_SMALL.name}"}
    return {
        "value": elements / wall,
        "unit": "elements/s",
        "cores": n,
        "kind": "oracle",
        "sample": f"wkv_recurrent (float64 NumPy) over all {spec.B * spec.C} lanes of {spec.name}, tokens "
                  f"0..{n_tok - 1} ({elements} elements): channels split over {n} forked processes, "
                  f"{wall:.2f} s wall; one process alone {dt:.1f} s",
        "single_process": single,
        "direct_definition": direct,
        "cpu_model": _cpu_model(),
        "affinity_cores": affinity,
        "worker_cap": max_workers,
        "numpy": np.__version__,
    }


COPY_BYTES = 512 << 20


def profile_run(name, launches):
    """Launches to profile: the workload's forward (or decode step) and a plain copy."""
    import torch

    from rwkv_linear_attention_libwkv_amd import workloads

    block = 0
    if name in workloads.FORWARD_SPECS:
        spec = workloads.FORWARD_SPECS[name]
        r = forward_case(spec, launches, 1)
        print(f"# {name}: {r['per_launch_s'] * 1e6:.1f} us/launch", flush=True)
        per_call, before = 1, 0
    elif name in workloads.LA_SPECS:
        r = la_case(workloads.LA_SPECS[name], launches, 1)
        print(f"# {name}: {r['per_call_s'] * 1e6:.1f} us/call", flush=True)
        per_call, before = 1, 0
    elif name.replace("wkv_bwd", "wkv_fwd") in workloads.FORWARD_SPECS:
        spec = workloads.FORWARD_SPECS[name.replace("wkv_bwd", "wkv_fwd")]
        r = backward_case(spec, launches, 1)
        print(f"# {name}: {r['backward_saved_s'] * 1e6:.1f} us/call (wkv_backward_saved)", flush=True)
        per_call, before = 1, 0
        block = 2  # the saved-states backward: one scan per call, after two blocks of one scan per call
    else:
        r = step_case(workloads.STEP_DECODE, 4, 1)
        print(f"# {r['workload']}: {r['per_step_launch_s'] * 1e6:.1f} us/step", flush=True)
        per_call, before = workloads.STEP_DECODE.steps, workloads.STEP_DECODE.prefix
    # the timed block reported (the case's first, the saved-states backward for a backward
    # workload), in launches of its main kernel (one per call; the decode step: `steps` per call,
    # after the untimed prefix)
    for n_settle, n_warm, n_timed in TIMED_LOG[:block]:
        before += per_call * (n_settle + n_warm + n_timed)
    n_settle, n_warm, n_timed = TIMED_LOG[block]
    print(f"# timed block: skip {before + per_call * (n_settle + n_warm)} take {per_call * n_timed}", flush=True)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)  # reads and writes COPY_BYTES each
    torch.cuda.synchronize()
    print(f"# copy calibration: {COPY_BYTES} bytes read and written per launch", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wkv_fwd_bf16_B1_T65536_C5120")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="time only the main workload")
    ap.add_argument("--profile-run", action="store_true",
                    help="a few launches of the workload's kernel and of a plain 512 MiB copy "
                         "(the byte-counter calibration), for rocprofv3")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the WKV lanes (batch x channel) are independent, "
              "so each GPU of a data-parallel job runs this same kernel on its own share and the "
              "figure to measure is one GPU's rate; pass --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from rwkv_linear_attention_libwkv_amd import workloads

    spec = workloads.FORWARD_SPECS.get(args.workload)
    # the oracle's baseline runs first: its workers are forked, which must happen before the
    # GPU is initialised
    cpu = None
    if not (args.profile_run or args.no_cpu_baseline):
        cpu = cpu_baseline(spec)
        print(f"# cpu baseline: {cpu['value']:.3g} elements/s on {cpu['cores']} cores", file=sys.stderr, flush=True)

    import torch

    from rwkv_linear_attention_libwkv_amd import libwkv  # noqa: F401  (fails loudly if unbuilt)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.profile_run:
        profile_run(args.workload, max(1, min(args.steps, 20)))
        return
    main_res = forward_case(spec, args.steps, args.warmup)
    _INPUTS.pop(spec.name, None)
    print(f"# {spec.name}: {main_res['per_launch_s'] * 1e6:.1f} us/launch, "
          f"{main_res['achieved_GBps']:.0f} GB/s", file=sys.stderr, flush=True)

    others = []
    if not args.no_others:
        for name, s in workloads.FORWARD_SPECS.items():
            if name == spec.name or s.elements < 1e6:
                continue
            # a launch of under 50 us: 200 timed launches, so that the first one's enqueue after the
            # start event (about 16 us of Python and HIP launch work) weighs under 1% of the region
            small = 3 * (4 if s.dtype == "f32" else 2) * s.elements < CACHE_FLUSH_BYTES
            r = forward_case(s, max(200 if small else 5, args.steps // 2), 2)
            _INPUTS.pop(s.name, None)
            others.append(r)
            print(f"# {name}: {r['per_launch_s'] * 1e6:.1f} us/launch, {r['achieved_GBps']:.0f} GB/s",
                  file=sys.stderr, flush=True)
        for s in (workloads.FWD_CTX8K, workloads.FWD_LONG_BF16):
            r = backward_case(s, max(5, args.steps // 2), 2)
            others.append(r)
            print(f"# {r['workload']}: {r['per_launch_s'] * 1e6:.1f} us/call, {r['achieved_GBps']:.0f} GB/s "
                  f"(algorithmic bytes); forward_save + backward_saved {r['train_pair_s'] * 1e6:.1f} us, "
                  f"{r['train_pair_algorithmic_GBps']:.0f} GB/s; backward_saved {r['backward_saved_s'] * 1e6:.1f} us, "
                  f"{r['roofline']['achieved']:.0f} GB/s", file=sys.stderr, flush=True)
        for s in (workloads.FWD_CTX8K, workloads.FWD_LONG_BF16):
            r = mix_case(s, max(5, args.steps // 2), 2)
            others.append(r)
            print(f"# {r['workload']}: gated forward {r['gated_forward_s'] * 1e6:.1f} us "
                  f"({r['gated_forward_algorithmic_GBps']:.0f} GB/s), token shift x3 {r['token_shift3_s'] * 1e6:.1f} us "
                  f"({r['token_shift3_algorithmic_GBps']:.0f} GB/s), its backward "
                  f"{r['token_shift3_backward_s'] * 1e6:.1f} us ({r['token_shift3_backward_algorithmic_GBps']:.0f} GB/s)",
                  file=sys.stderr, flush=True)
        for s in workloads.LA_SPECS.values():
            if s.tokens < 100000:
                continue
            r = la_case(s, max(5, args.steps // 2), 2)
            others.append(r)
            print(f"# {r['workload']}: {r['per_call_s'] * 1e6:.1f} us, {r['achieved_GBps']:.0f} GB/s, "
                  f"{r['useful_TFLOPs']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        r = step_case(workloads.STEP_DECODE, args.steps, 1)
        others.append(r)
        print(f"# {r['workload']}: {r['per_step_launch_s'] * 1e6:.1f} us/step, "
              f"{r['achieved_GBps']:.0f} GB/s", file=sys.stderr, flush=True)
        r = decode_graph_case(workloads.STEP_DECODE_SMALL, max(10, args.steps))
        others.append(r)
        print(f"# {r['workload']}: {r['eager_per_step_s'] * 1e6:.2f} us/step called one by one, "
              f"{r['graph_per_step_s'] * 1e6:.2f} us/step replayed as one graph", file=sys.stderr, flush=True)

    bytes_per_launch = main_res["algorithmic_bytes_per_launch"]
    achieved = main_res["achieved_GBps"]
    traffic = measured_traffic(spec.name)
    line = {
        "metric": "WKV fwd elements/sec (B\u00b7T\u00b7C) and achieved HBM GB/s vs MI355X peak",
        "value": main_res["elements_per_s"],
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": main_res["per_launch_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if spec.dtype == "f32" else "bf16",
        "data": "synthetic (seeded NumPy draws; no dataset or weights involved)",
        "config": {"workload": spec.name, "B": spec.B, "T": spec.T, "C": spec.C,
                   "algo": main_res["algo"], "inputs": main_res["inputs"], "parallelism": "single GPU"},
        "roofline": roofline_of(achieved, traffic),
        "cpu_baseline": cpu,
        "other_workloads": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
