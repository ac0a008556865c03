"""Benchmark: decode-stage SwiGLU MLP on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--batch B]
                    [--no-cpu-baseline] [--no-sweep] [--sections a,b,...]

A step is one call of the whole hot path, dfk_swiglu_mlp (the fused gate-up
kernel, then the down-projection kernel), on a Llama-3-8B-shaped layer
(d_model 4096, d_ff 14336) at decode batch B (default 1), with every input
already resident in HBM.  Weights rotate over 5 seeded sets (5 x 352 MB, far
beyond the 256 MB Infinity Cache) so every call streams its weights from HBM.

Printed: one JSON line with the metric (us per MLP call, the mean over K
back-to-back calls; lower is better) and its per-call p10 / p50 / p90, the
dominant kernel's roofline (algorithmic bytes / measured launch duration vs
the 8 TB/s HBM peak), the practical ceiling (a plain streaming read of the
same weight bytes on this machine, dfk_stream_read) and the call's fraction of
it, and context sections: per-batch figures for B = 1..64, the scheduler's
shape sweep, FP8 weights, packed gate/up weights, the persistent kernel, the
RMS-normalized MLP, the Llama-3-70B layer shape, and the 32-layer Llama-3-8B
MLP stack with its between-layer RMS rescale (timed separately and
excluded), eager and as one captured HIP graph; then the fp64 CPU oracle
timed on the host cores over a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/MLP call + achieved HBM GB/s (% of peak), Llama-3-8B shape, batch 1–64"
HBM_PEAK_GBPS = 8000.0
D_MODEL, D_FF = 4096, 14336
ROTATE = 5
KERNEL_SOURCE = os.path.join(ROOT, "swiglu_mlp_amd", "csrc", "dfk_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_llama8b_B1_traffic.txt")


def gate_up_bytes(B, d_model=D_MODEL, d_ff=D_FF):
    """Algorithmic HBM bytes of one fused gate-up launch: both weight matrices
    once, x once, h (fp32) written once."""
    return 2 * (2 * d_ff * d_model) + 2 * B * d_model + 4 * B * d_ff


def down_bytes(B, d_model=D_MODEL, d_ff=D_FF):
    """W_down once, h (fp32) read once, y (bf16) written once."""
    return 2 * d_model * d_ff + 4 * B * d_ff + 2 * B * d_model


def mlp_bytes(B, d_model=D_MODEL, d_ff=D_FF):
    return gate_up_bytes(B, d_model, d_ff) + down_bytes(B, d_model, d_ff)


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(B):
    """HBM bytes per gate-up launch from the committed rocprofv3 PMC summary,
    if it was taken on the current kernel source and batch; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if int(fields.get("batch", -1)) != B:
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def make_weights(R, device):
    from swiglu_mlp_amd import inputs
    sets = []
    for r in range(R):
        base = 6000 + 10 * r
        sets.append((inputs.randn_bf16_device((D_FF, D_MODEL), 0.02, base + 1, device),
                     inputs.randn_bf16_device((D_FF, D_MODEL), 0.02, base + 2, device),
                     inputs.randn_bf16_device((D_MODEL, D_FF), 0.02, base + 3, device)))
    return sets


def _timed(fn, steps, warmup):
    """Average ms per call of fn(i) over `steps` back-to-back calls, bracketed
    by one pair of HIP events on the current stream (the launch stream)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def _per_call_us(fn, steps, warmup):
    """(p10, p50, p90) us of single calls of fn(i): a pair of HIP events
    around each call, on the current stream, calls back to back."""
    import torch
    for i in range(warmup):
        fn(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)

    def q(f):
        return t[min(len(t) - 1, max(0, int(round(f * (len(t) - 1)))))]
    return q(0.10), q(0.50), q(0.90)


def time_batch(B, sets, steps, warmup, device):
    """Per batch B: ms per whole-MLP call (dfk_swiglu_mlp, the step), and ms
    per launch of each kernel timed back to back on its own.  Weights rotate
    every call."""
    import torch
    import swiglu_mlp_amd as dfk
    from swiglu_mlp_amd import inputs

    x = inputs.randn_bf16_device((B, D_MODEL), 1.0, 6100 + B, device)
    h = torch.empty((B, D_FF), dtype=torch.float32, device=device)
    out = torch.empty((B, D_MODEL), dtype=torch.bfloat16, device=device)
    gl, dl = dfk.dfk_schedule_select(B, D_MODEL, D_FF)
    R = len(sets)

    def mlp(i):
        dfk.dfk_swiglu_mlp(x, *sets[i % R], out)

    def gate_up(i):
        wg, wu, _ = sets[i % R]
        dfk.dfk_gate_up_silu_mul(x, wg, wu, h, layout=gl)

    def down(i):
        dfk.dfk_down_proj(h, sets[i % R][2], out, layout=dl)

    ms_call = _timed(mlp, steps, warmup)
    ms_gu = _timed(gate_up, steps, warmup)
    ms_dn = _timed(down, steps, warmup)
    return ms_call, ms_gu, ms_dn, (dfk.layout_name(gl), dfk.layout_name(dl))


def time_stack(device, B=1, layers=32, steps=20, warmup=3):
    """The 32-layer Llama-3-8B MLP stack (11.3 GB of distinct weights, cold by
    construction), chained y_l -> RMS rescale -> x_{l+1}.  The rescale is
    dfk_rmsnorm with a unit gain and eps 1e-6: bf16_RNE(y / sqrt(mean(y^2) +
    eps)) per batch row, bit for bit the oracle's between-layer rescale.  It is
    timed separately and excluded from the per-layer MLP figure.  Eager (with
    HIP events around every MLP call) and as one captured HIP graph; and the
    same chain with each rescale fused into the next layer's gate-up
    (dfk_rmsnorm_swiglu_mlp), as context."""
    import torch
    import swiglu_mlp_amd as dfk
    from swiglu_mlp_amd import inputs

    W = [inputs.stack_layer_weights_device(l, device) for l in range(layers)]
    x0 = inputs.randn_bf16_device((B, D_MODEL), 1.0, 3000, device)
    ones = torch.ones(D_MODEL, dtype=torch.bfloat16, device=device)
    ys = [torch.empty((B, D_MODEL), dtype=torch.bfloat16, device=device) for _ in range(layers)]
    xs = [x0] + [torch.empty((B, D_MODEL), dtype=torch.bfloat16, device=device) for _ in range(layers - 1)]
    s = torch.cuda.Stream()
    EPS = 1e-6

    def chain(ev=None):
        for l in range(layers):
            if ev is not None:
                ev[l][0].record(s)
            dfk.dfk_swiglu_mlp(xs[l], *W[l], out=ys[l])
            if ev is not None:
                ev[l][1].record(s)
            if l + 1 < layers:
                dfk.dfk_rmsnorm(ys[l], ones, EPS, xs[l + 1])

    def rescales():
        for l in range(layers - 1):
            dfk.dfk_rmsnorm(ys[l], ones, EPS, xs[l + 1])

    def fused_chain():
        dfk.dfk_swiglu_mlp(xs[0], *W[0], out=ys[0])
        for l in range(1, layers):
            dfk.dfk_rmsnorm_swiglu_mlp(ys[l - 1], ones, EPS, *W[l], out=ys[l])

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(n):
            fn()
        e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n  # us per chain

    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for _ in range(warmup):
            chain()
            fused_chain()
        s.synchronize()
        eager_chain_us = timed(chain, steps)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(layers)]
        mlp_us = 0.0
        for _ in range(steps):
            chain(ev)
            s.synchronize()
            mlp_us += sum(a.elapsed_time(b) * 1e3 for a, b in ev)
        mlp_us /= steps * layers
        rescale_us = timed(rescales, steps) / (layers - 1)
        eager_fused_us = timed(fused_chain, steps)
    graphs = {}
    for name, fn in (("chain", chain), ("rescales", rescales), ("fused", fused_chain)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
        graphs[name] = g
    with torch.cuda.stream(s):
        for g in graphs.values():
            for _ in range(warmup):
                g.replay()
        s.synchronize()
        gt = {name: timed(g.replay, steps) for name, g in graphs.items()}
    graph_mlp_us = (gt["chain"] - gt["rescales"]) / layers
    bytes_layer = mlp_bytes(B)
    del graphs, W
    torch.cuda.empty_cache()
    return {"layers": layers, "batch": B, "weights_GB": round(layers * 3 * D_MODEL * D_FF * 2 / 1e9, 2),
            "rescale": "dfk_rmsnorm, unit gain, eps 1e-6, between layers",
            "eager_us_per_layer_with_rescale": round(eager_chain_us / layers, 2),
            "eager_mlp_us_per_layer": round(mlp_us, 2),
            "rescale_us": round(rescale_us, 2),
            "graph_us_per_layer_with_rescale": round(gt["chain"] / layers, 2),
            "graph_mlp_us_per_layer": round(graph_mlp_us, 2),
            "graph_mlp_GBps": round(bytes_layer / (graph_mlp_us * 1e-6) / 1e9, 1),
            "fused_rescale_eager_us_per_layer": round(eager_fused_us / layers, 2),
            "fused_rescale_graph_us_per_layer": round(gt["fused"] / layers, 2)}


def time_stream_ceiling(device, steps=100, warmup=10, rotate=5, d_model=D_MODEL, d_ff=D_FF, only_two=False):
    """The practical HBM read ceiling on this machine: dfk_stream_read (plain
    16-byte streaming loads, no arithmetic) over `rotate` buffers of a layer's
    weight bytes (the 8B layer's by default), read as the MLP call reads them
    (gate-up's bytes in one launch, then down's) and in one launch; us and
    GB/s.  only_two: the two-launch figure alone."""
    import torch
    import swiglu_mlp_amd as dfk

    gu, dn = 2 * 2 * d_ff * d_model, 2 * d_model * d_ff
    bufs = [torch.ones(gu + dn, dtype=torch.uint8, device=device) for _ in range(rotate)]
    sink = torch.zeros(64, dtype=torch.int32, device=device)

    def two(i):
        b = bufs[i % rotate]
        dfk.dfk_stream_read(b[:gu], sink)
        dfk.dfk_stream_read(b[gu:], sink)

    res = {}
    legs = (("gate_up_bytes", lambda i: dfk.dfk_stream_read(bufs[i % rotate][:gu], sink), gu),
            ("down_bytes", lambda i: dfk.dfk_stream_read(bufs[i % rotate][gu:], sink), dn),
            ("both_two_launches", two, gu + dn),
            ("both_one_launch", lambda i: dfk.dfk_stream_read(bufs[i % rotate], sink), gu + dn))
    for name, fn, nbytes in (legs[2:3] if only_two else legs):
        us = _timed(fn, steps, warmup) * 1e3
        res[name] = {"bytes": nbytes, "us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
    del bufs
    torch.cuda.empty_cache()
    return res


def time_70b(device, batches=(1, 4, 16, 64), steps=100, warmup=10, persistent=True):
    """Context: whole-MLP us per call at the Llama-3-70B layer shape
    (d_model 8192, d_ff 28672), two weight sets rotated (2.8 GB); with
    `persistent`, also the persistent kernel at B = 1 (a cooperative launch)."""
    import torch
    import swiglu_mlp_amd as dfk
    from swiglu_mlp_amd import inputs

    dm, dff = 8192, 28672
    sets = [(inputs.randn_bf16_device((dff, dm), 0.02, 7000 + 10 * r + 1, device),
             inputs.randn_bf16_device((dff, dm), 0.02, 7000 + 10 * r + 2, device),
             inputs.randn_bf16_device((dm, dff), 0.02, 7000 + 10 * r + 3, device)) for r in range(2)]
    res = {}
    for B in batches:
        x = inputs.randn_bf16_device((B, dm), 1.0, 7100 + B, device)
        out = torch.empty((B, dm), dtype=torch.bfloat16, device=device)
        ms = _timed(lambda i: dfk.dfk_swiglu_mlp(x, *sets[i % 2], out), steps, warmup)
        gbps = mlp_bytes(B, dm, dff) / (ms * 1e-3) / 1e9
        res[str(B)] = {"us_per_call": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                       "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        if B == 1 and persistent:
            from swiglu_mlp_amd import Layout
            ms_p = _timed(lambda i: dfk.dfk_swiglu_mlp(x, *sets[i % 2], out, layout=Layout.ROW_PERSISTENT),
                          steps, warmup)
            res[str(B)]["persistent_us"] = round(ms_p * 1e3, 2)
    del sets
    torch.cuda.empty_cache()
    return res


def time_shape_sweep(device, steps=100, warmup=10, min_rotated_bytes=600e6):
    """The scheduler's shape sweep: whole-MLP us per call for every
    (d_model, d_ff) x batch of the sweep, under AUTO and with both kernels
    forced to ROW or to COL (the scheduler picks per kernel among four
    variants, so AUTO should be at least as fast as either).  Enough weight
    sets are rotated that they do not fit in the 256 MB last-level cache.
    Per shape also the practical ceiling (two streaming-read launches over
    the same bytes, as many buffers rotated) and each call's fraction of it."""
    import math
    import torch
    import swiglu_mlp_amd as dfk
    from swiglu_mlp_amd import Layout, inputs

    res = {}
    for s, (dm, dff) in enumerate(inputs.SWEEP_SHAPES):
        set_bytes = 3 * dm * dff * 2
        R = max(2, math.ceil(min_rotated_bytes / set_bytes))
        sets = [(inputs.randn_bf16_device((dff, dm), 0.02, 8000 + 100 * s + 10 * r + 1, device),
                 inputs.randn_bf16_device((dff, dm), 0.02, 8000 + 100 * s + 10 * r + 2, device),
                 inputs.randn_bf16_device((dm, dff), 0.02, 8000 + 100 * s + 10 * r + 3, device)) for r in range(R)]
        ceiling = time_stream_ceiling(device, steps, warmup, rotate=R, d_model=dm, d_ff=dff,
                                      only_two=True)["both_two_launches"]
        shape = {"practical_two_launch_us": ceiling["us"]}
        for B in inputs.SWEEP_BATCHES:
            x = inputs.randn_bf16_device((B, dm), 1.0, 8900 + B, device)
            out = torch.empty((B, dm), dtype=torch.bfloat16, device=device)
            # burn-in: the first timed variant of a fresh batch otherwise runs
            # a few per cent slow
            _timed(lambda i: dfk.dfk_swiglu_mlp(x, *sets[i % R], out), steps, warmup)
            t = {}
            for name, layout in (("auto", Layout.AUTO), ("row", Layout.ROW), ("col", Layout.COL)):
                t[name] = _timed(lambda i: dfk.dfk_swiglu_mlp(x, *sets[i % R], out, layout=layout), steps, warmup) * 1e3
            gbps = mlp_bytes(B, dm, dff) / (t["auto"] * 1e-6) / 1e9
            shape[str(B)] = {"us_per_call": round(t["auto"], 2), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                             "frac_of_practical": round(gbps / ceiling["GBps"], 4),
                             "row_us": round(t["row"], 2), "col_us": round(t["col"], 2)}
        res[f"{dm}x{dff}"] = shape
        del sets
        torch.cuda.empty_cache()
    return res


def time_persistent(sets, device, batches=(1, 2), steps=300, warmup=30):
    """Context: the persistent MLP kernel (both row walks in one cooperative
    launch, DFK_LAYOUT_ROW_PERSISTENT) against the scheduler's two-kernel
    call, us per call at the 8B shape."""
    import torch
    import swiglu_mlp_amd as dfk
    from swiglu_mlp_amd import Layout, inputs

    R = len(sets)
    res = {}
    for B in batches:
        x = inputs.randn_bf16_device((B, D_MODEL), 1.0, 6100 + B, device)
        out = torch.empty((B, D_MODEL), dtype=torch.bfloat16, device=device)
        us = {}
        for name, layout in (("persistent_us", Layout.ROW_PERSISTENT), ("two_kernel_us", Layout.AUTO),
                             ("two_kernel_row_valu_us", Layout.ROW_VALU)):
            us[name] = round(_timed(lambda i: dfk.dfk_swiglu_mlp(x, *sets[i % R], out, layout=layout),
                                    steps, warmup) * 1e3, 2)
        us["persistent_GBps"] = round(mlp_bytes(B) / (us["persistent_us"] * 1e-6) / 1e9, 1)
        res[str(B)] = us
    return res


def time_packed(sets, device, batches=(1, 4, 8), steps=200, warmup=20):
    """Context: the MLP with W_gate and W_up packed in one tensor (blocked and
    row-interleaved) against separate tensors, us per call at the 8B shape
    (scheduler's variants)."""
    import torch
    import swiglu_mlp_amd as dfk
    from swiglu_mlp_amd import Packing, inputs

    R = len(sets)
    packed = {p: [dfk.pack_gate_up(s[0], s[1], p) for s in sets] for p in Packing}
    res = {}
    for B in batches:
        x = inputs.randn_bf16_device((B, D_MODEL), 1.0, 6100 + B, device)
        out = torch.empty((B, D_MODEL), dtype=torch.bfloat16, device=device)
        r = {"separate_us": round(_timed(lambda i: dfk.dfk_swiglu_mlp(x, *sets[i % R], out), steps, warmup) * 1e3, 2)}
        for p in Packing:
            r[p.name.lower() + "_us"] = round(_timed(
                lambda i: dfk.dfk_swiglu_mlp_packed(x, packed[p][i % R], sets[i % R][2], p, out), steps,
                warmup) * 1e3, 2)
        res[str(B)] = r
    del packed
    torch.cuda.empty_cache()
    return res


def fp8_mlp_bytes(B, d_model=D_MODEL, d_ff=D_FF):
    """Algorithmic bytes of one FP8-weight MLP call: the E4M3 codes and row
    scales of the three matrices, x, h written and read (fp32), y."""
    return 3 * d_model * d_ff + 4 * (2 * d_ff + d_model) + 2 * B * d_model + 2 * 4 * B * d_ff + 2 * B * d_model


def time_fp8(device, batches=(1, 2, 4, 8, 16, 64), steps=300, warmup=30, rotate=8):
    """Context: the MLP over weight-only FP8 weights (E4M3 codes + per-row
    fp32 scales) at the 8B shape, `rotate` weight sets (2.8 GB) so every call
    streams from HBM: us per call and HBM roofline fraction of the codes."""
    import torch
    import swiglu_mlp_amd as dfk
    from swiglu_mlp_amd import inputs

    def codes(rows, cols, seed):
        w = inputs.randn_bf16_device((rows, cols), 0.02, seed, device).float()
        s = (w.abs().amax(dim=1) / 448.0).clamp_min(1e-30)
        return (w / s[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), s.contiguous()

    sets = []
    for r in range(rotate):
        base = 6500 + 10 * r
        qg, sg = codes(D_FF, D_MODEL, base + 1)
        qu, su = codes(D_FF, D_MODEL, base + 2)
        qd, sd = codes(D_MODEL, D_FF, base + 3)
        sets.append((qg, sg, qu, su, qd, sd))
    torch.cuda.synchronize()
    res = {}
    for B in batches:
        x = inputs.randn_bf16_device((B, D_MODEL), 1.0, 6100 + B, device)
        out = torch.empty((B, D_MODEL), dtype=torch.bfloat16, device=device)
        ms = _timed(lambda i: dfk.dfk_swiglu_mlp_fp8(x, *sets[i % rotate], out), steps, warmup)
        gbps = fp8_mlp_bytes(B) / (ms * 1e-3) / 1e9
        res[str(B)] = {"us_per_call": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                       "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    del sets
    torch.cuda.empty_cache()
    return res


def time_rmsnorm(sets, device, batches=(1, 4, 8, 16), steps=200, warmup=20):
    """Context: the MLP on RMS-normalized input at the 8B layer shape, us per
    call: the fused entry point (norm inside gate-up where the kernel stages
    x in LDS), the norm kernel then the plain MLP, and the plain MLP alone."""
    import torch
    import swiglu_mlp_amd as dfk
    from swiglu_mlp_amd import inputs

    gain = inputs.randn_bf16_device((D_MODEL,), 0.1, 6200, device).add_(1.0)
    R = len(sets)
    res = {}
    for B in batches:
        x = inputs.randn_bf16_device((B, D_MODEL), 1.0, 6100 + B, device)
        xn = torch.empty_like(x)
        out = torch.empty((B, D_MODEL), dtype=torch.bfloat16, device=device)

        def fused(i):
            dfk.dfk_rmsnorm_swiglu_mlp(x, gain, 1e-5, *sets[i % R], out)

        def separate(i):
            dfk.dfk_rmsnorm(x, gain, 1e-5, xn)
            dfk.dfk_swiglu_mlp(xn, *sets[i % R], out)

        def plain(i):
            dfk.dfk_swiglu_mlp(x, *sets[i % R], out)

        res[str(B)] = {k: round(_timed(f, steps, warmup) * 1e3, 2)
                       for k, f in (("fused_us", fused), ("separate_us", separate), ("no_norm_us", plain))}
    return res


def cpu_baseline(sets, budget_s=12.0, max_calls=400):
    """The fp64 oracle on the host cores: whole-MLP calls at B=1 on weight set 0."""
    import numpy as np
    import torch
    import oracle
    from swiglu_mlp_amd import inputs

    wg, wu, wd = (t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16) for t in sets[0])
    x = inputs.randn_bf16((1, D_MODEL), 1.0, 6101)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = min(cores, 16)  # the host CPU share that goes with one GPU
    orc = oracle.get()
    orc.mlp(x, wg, wu, wd, nthreads=cores)  # warm
    n = 0
    t0 = time.perf_counter()
    while n < max_calls and (time.perf_counter() - t0) < budget_s:
        orc.mlp(x, wg, wu, wd, nthreads=cores)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(dt / n * 1e6, 1), "unit": "µs/MLP call", "cores": cores, "kind": "oracle",
            "sample": f"{n} whole-MLP calls (all outputs, fp64) at B=1 on one Llama-3-8B-shaped "
                      f"weight set, {dt:.1f} s wall"}


SECTIONS = ("ceiling", "per_batch", "sweep", "fp8", "packed", "persistent", "norm", "70b", "stack")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="only the headline batch and the streaming-read ceiling (no context sections)")
    ap.add_argument("--sections", default=None,
                    help="comma-separated context sections to run (default: all): " + ",".join(SECTIONS))
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy 10 times (the reference kernel "
                         "that scales rocprofv3 FETCH_SIZE / WRITE_SIZE into bytes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode MLP here runs on a single MI355X "
              "(no sharding or collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.sections is not None:
        sections = {x for x in args.sections.split(",") if x}
        unknown = sections - set(SECTIONS)
        if unknown:
            print(f"unknown sections: {sorted(unknown)}; known: {', '.join(SECTIONS)}", file=sys.stderr)
            sys.exit(2)
    else:
        sections = {"ceiling"} if args.no_sweep else set(SECTIONS)

    import torch
    import swiglu_mlp_amd as dfk

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    if args.calibrate_copy:
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "launches": 10}))
        return
    dfk.lib()
    sets = make_weights(ROTATE, device)
    torch.cuda.synchronize()

    B = args.batch
    ms_per_step, ms_gu, ms_dn, variants = time_batch(B, sets, args.steps, args.warmup, device)
    us_per_call = ms_per_step * 1e3
    gu_us, dn_us = ms_gu * 1e3, ms_dn * 1e3
    bytes_call = mlp_bytes(B)
    achieved_call = bytes_call / (us_per_call * 1e-6) / 1e9
    gu_achieved = gate_up_bytes(B) / (gu_us * 1e-6) / 1e9
    from swiglu_mlp_amd import inputs as _inputs
    x = _inputs.randn_bf16_device((B, D_MODEL), 1.0, 6100 + B, device)
    out = torch.empty((B, D_MODEL), dtype=torch.bfloat16, device=device)
    p10, p50, p90 = _per_call_us(lambda i: dfk.dfk_swiglu_mlp(x, *sets[i % ROTATE], out),
                                 max(args.steps, 20), args.warmup)

    ceiling = time_stream_ceiling(device) if "ceiling" in sections else None
    per_batch = {}
    if "per_batch" in sections:
        for b in (1, 2, 4, 8, 16, 32, 64):
            t, g, d, v = time_batch(b, sets, 200, 20, device)
            us = t * 1e3
            gbps = mlp_bytes(b) / (us * 1e-6) / 1e9
            per_batch[str(b)] = {"us_per_call": round(us, 2), "GBps": round(gbps, 1),
                                 "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                                 "gate_up_us": round(g * 1e3, 2), "down_us": round(d * 1e3, 2),
                                 "variants": list(v)}
            if ceiling:
                per_batch[str(b)]["frac_of_practical"] = round(
                    gbps / ceiling["both_two_launches"]["GBps"], 4)

    sweep = time_shape_sweep(device) if "sweep" in sections else None
    fp8 = time_fp8(device) if "fp8" in sections else None
    packed = time_packed(sets, device) if "packed" in sections else None
    persistent = time_persistent(sets, device) if "persistent" in sections else None
    norm = time_rmsnorm(sets, device) if "norm" in sections else None
    shape70b = time_70b(device, persistent="persistent" in sections) if "70b" in sections else None
    stack = time_stack(device) if "stack" in sections else None

    result = {
        "metric": METRIC,
        "value": round(us_per_call, 3),
        "unit": "µs/MLP call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"Llama-3-8B-shaped SwiGLU MLP layer, decode batch {B}",
            "batch": B, "d_model": D_MODEL, "d_ff": D_FF,
            "weight_sets_rotated": ROTATE,
            "variants": {"gate_up": variants[0], "down": variants[1]},
            "parallelism": "single GPU",
        },
        "achieved_GBps": round(achieved_call, 1),
        "frac_of_hbm_peak": round(achieved_call / HBM_PEAK_GBPS, 4),
        "us_per_call_p10_p50_p90": [round(p10, 2), round(p50, 2), round(p90, 2)],
        "algorithmic_bytes_per_call": bytes_call,
        "kernel_us": {"gate_up": round(gu_us, 2), "down": round(dn_us, 2)},
        "roofline": {
            "kernel": "gate_up (fused gate+up+SiLU*mul)",
            "bound": "hbm",
            "achieved": round(gu_achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gu_achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(B),
            "algorithmic_bytes_per_launch": gate_up_bytes(B),
        },
        "stream_read_ceiling": ceiling,
        "frac_of_practical": (round(achieved_call / ceiling["both_two_launches"]["GBps"], 4)
                              if ceiling else None),
        "per_batch": per_batch,
        "per_batch_llama70b_shape": shape70b,
        "stack32_llama8b": stack,
        "rmsnorm_mlp_llama8b": norm,
        "persistent_mlp_llama8b": persistent,
        "packed_gate_up_llama8b": packed,
        "fp8_weights_mlp_llama8b": fp8,
        "shape_sweep": sweep,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(sets)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
