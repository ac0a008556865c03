"""Profiler-driven tuning of the row / column kernel variants.

    python -m swiglu_mlp_amd.tune [--shapes 4096x14336,...] [--batches 1,2,4,...]
                                  [--timer rocprof|events] [--out PATH]

For every (d_model, d_ff) shape, batch B and op (gate_up, down), each variant
that can run the shape (row_valu, col_valu, row_mfma, col_mfma) is launched
back to back with rotating weight copies (at least 1.5 GB of distinct weights,
so every launch streams from HBM rather than the 256 MB Infinity Cache).  The
winner is the variant with the lowest median per-call cost; variants within
2 % of the best count as a tie, which goes to a row variant (VALU first).  The result is the
JSON table that dfk_schedule_select reads.

Timers:
  rocprof  (default) the worker runs under `rocprofv3 --kernel-trace`; a call's
           cost is the spacing between its last kernel's end and the previous
           call's (a block's calls run back to back, so this is the kernel
           time plus the launch gap before it: what a stream of decode calls
           pays per call).  The profile ranks every variant; those within
           2x of its best are then re-timed untraced (HIP events around
           back-to-back calls) and the confirmation picks among them;
  events   HIP events around groups of back-to-back launches only.

This is the runtime scheduling across row-major and column-major variants of
"Deep Kernel Fusion for Transformer Decoding" (podcast episode page, episode
summary), with the profiler as the measuring instrument.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import math
import os
import shutil
import statistics
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_SHAPES = [(2048, 5632), (3072, 8192), (4096, 14336), (5120, 13824), (8192, 28672)]
DEFAULT_BATCHES = [1, 2, 4, 8, 16, 32, 64]
VARIANTS = ["row_valu", "col_valu", "row_mfma", "col_mfma"]
# Variants within this fraction of the best count as a tie (a row variant,
# VALU first, wins a tie).
TIE = 0.02
# Variants within this fraction of the profile's best are re-timed back to
# back with HIP events and no profiler attached, and that decides among them:
# measured on MI355X, the traced run reads the LDS-transposed MFMA kernels up
# to ~5 % faster, relative to the VALU kernels, than the same calls run
# untraced, and calls of two kernels (a K-split kernel plus the reduce
# kernel) up to ~60 % slower (Llama-3-8B down at B = 16: 36.0 us traced,
# 27.9 us untraced; d_model 3072, d_ff 8192, down at B = 16: the K-split
# column variant read 1.57x the row variant traced and is the faster one
# untraced).  The profile still rules out the variants far behind.
CONFIRM_BAND = 1.00
ROTATE_BYTES = 1.5e9


def layer_bytes(d_model, d_ff):
    return 3 * d_model * d_ff * 2


def runnable(variant, op, B, d_model):
    if variant.endswith("valu"):
        if B > 8:
            return False
        if op == "gate_up" and B * d_model * 2 > 160 * 1024:
            return False
    return True


def plan_blocks(shapes, batches, reps):
    """The launch sequence: (shape, B, op, variant, reps) blocks in order."""
    blocks = []
    for (dm, dff) in shapes:
        for B in batches:
            for op in ("gate_up", "down"):
                for v in VARIANTS:
                    if runnable(v, op, B, dm):
                        blocks.append({"d_model": dm, "d_ff": dff, "B": B, "op": op, "variant": v, "reps": reps})
    return blocks


def run_worker(blocks, warmup, use_events):
    """Launch every block; returns per-block event timings (ms per launch) if asked."""
    import torch
    import swiglu_mlp_amd as dfk
    from swiglu_mlp_amd import Layout, inputs

    dev = torch.device("cuda:0")
    dfk.lib()
    layout_of = {"row_valu": Layout.ROW_VALU, "col_valu": Layout.COL_VALU,
                 "row_mfma": Layout.ROW_MFMA, "col_mfma": Layout.COL_MFMA}
    results = []
    cur_shape, sets = None, None
    for blk in blocks:
        shape = (blk["d_model"], blk["d_ff"])
        if shape != cur_shape:
            sets = None
            torch.cuda.empty_cache()
            dm, dff = shape
            R = max(2, math.ceil(ROTATE_BYTES / layer_bytes(dm, dff)))
            sets = [(inputs.randn_bf16_device((dff, dm), 0.02, 9000 + 10 * r + 1, dev),
                     inputs.randn_bf16_device((dff, dm), 0.02, 9000 + 10 * r + 2, dev),
                     inputs.randn_bf16_device((dm, dff), 0.02, 9000 + 10 * r + 3, dev)) for r in range(R)]
            cur_shape = shape
        dm, dff = shape
        B = blk["B"]
        x = inputs.randn_bf16_device((B, dm), 1.0, 9500 + B, dev)
        h = torch.randn((B, dff), device=dev, dtype=torch.float32)
        y = torch.empty((B, dm), device=dev, dtype=torch.bfloat16)
        lay = layout_of[blk["variant"]]
        R = len(sets)
        if blk["op"] == "gate_up":
            def call(i):
                wg, wu, _ = sets[i % R]
                dfk.dfk_gate_up_silu_mul(x, wg, wu, h, layout=lay)
        else:
            def call(i):
                dfk.dfk_down_proj(h, sets[i % R][2], y, layout=lay)
        for i in range(warmup):
            call(i)
        torch.cuda.synchronize()
        times = []
        if use_events:
            group = 10
            for g in range(max(1, blk["reps"] // group)):
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                for i in range(group):
                    call(g * group + i)
                e.record()
                e.synchronize()
                times.append(s.elapsed_time(e) / group)
        else:
            # marker launches are not needed: the parent maps dispatches to
            # blocks by order (warmup + reps per block)
            for i in range(blk["reps"]):
                call(warmup + i)
            torch.cuda.synchronize()
        results.append(times)
    return results


def parse_rocprof(outdir):
    """One record per library call, in dispatch order: list of (name, start_ns, end_ns).

    A call is one kernel, except the down projection's K-split variants, whose
    kernel is followed by a reduce kernel: that call runs from the first
    kernel's start to the reduce kernel's end."""
    files = glob.glob(os.path.join(outdir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise RuntimeError(f"no kernel_trace.csv under {outdir}")
    rows = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name", "")
                if "dfk::" not in name:
                    continue
                rows.append((int(r.get("Dispatch_Id", 0)), int(r["Start_Timestamp"]),
                             int(r["End_Timestamp"]), name))
    rows.sort()
    calls = []
    for _, start, end, name in rows:
        if "panel_reduce_kernel" in name and calls:
            first_name, first_start, _ = calls[-1]
            calls[-1] = (first_name, first_start, end)
        else:
            calls.append((name, start, end))
    return calls


def block_costs(calls, blocks, warmup):
    """Median per-call cost (us) of each block from the trace's calls, in
    dispatch order: the spacing between consecutive call ends, taken over a
    block's timed calls (the first of them measured from the last warm-up)."""
    if warmup < 1:
        raise RuntimeError("the rocprof timer needs at least one warm-up call per block")
    expect = sum(warmup + b["reps"] for b in blocks)
    if len(calls) != expect:
        raise RuntimeError(f"expected {expect} library calls in the trace, found {len(calls)}")
    out, i = [], 0
    for b in blocks:
        ends = [e for _, _, e in calls[i + warmup - 1:i + warmup + b["reps"]]]
        out.append(statistics.median(ends[k] - ends[k - 1] for k in range(1, len(ends))) / 1e3)
        i += warmup + b["reps"]
    return out


def choose(timings_us):
    """Winner by median; within TIE of the best, prefer a row variant."""
    best = min(timings_us.values())
    close = [v for v, t in timings_us.items() if t <= best * (1 + TIE)]
    for v in ("row_valu", "row_mfma"):
        if v in close:
            return v
    return min(timings_us, key=timings_us.get)


def _key(blk):
    return (blk["op"], blk["B"], blk["d_model"], blk["d_ff"])


def near_ties(blocks, per_block_us, band=CONFIRM_BAND):
    """Blocks whose variant is within `band` of the best for its (op, B,
    shape), for keys with more than one such variant."""
    best = {}
    for blk, us in zip(blocks, per_block_us):
        best[_key(blk)] = min(us, best.get(_key(blk), float("inf")))
    cand = [blk for blk, us in zip(blocks, per_block_us) if us <= best[_key(blk)] * (1 + band)]
    count = {}
    for blk in cand:
        count[_key(blk)] = count.get(_key(blk), 0) + 1
    return [blk for blk in cand if count[_key(blk)] > 1]


def build_table(blocks, per_block_us, confirm=None):
    """Table entries; `confirm` maps (op, B, d_model, d_ff) -> {variant: us}
    from the untraced re-timing, which then decides among its variants."""
    table = {}
    for blk, us in zip(blocks, per_block_us):
        table.setdefault(_key(blk), {})[blk["variant"]] = round(us, 3)
    entries = []
    for key, t in sorted(table.items(), key=lambda kv: (kv[0][2], kv[0][3], kv[0][1], kv[0][0])):
        op, B, dm, dff = key
        e = {"op": op, "B": B, "d_model": dm, "d_ff": dff, "us": t}
        if confirm and key in confirm:
            e["confirm_us"] = {v: round(u, 3) for v, u in confirm[key].items()}
            e["winner"] = choose(confirm[key])
        else:
            e["winner"] = choose(t)
        entries.append(e)
    return entries


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--shapes", default=",".join(f"{a}x{b}" for a, b in DEFAULT_SHAPES))
    ap.add_argument("--batches", default=",".join(map(str, DEFAULT_BATCHES)))
    ap.add_argument("--reps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--timer", choices=["rocprof", "events"], default="rocprof")
    ap.add_argument("--out", default=os.path.join(PKG, "tuning", "gfx950.json"))
    ap.add_argument("--worker", help=argparse.SUPPRESS)
    args = ap.parse_args()

    shapes = [tuple(int(v) for v in s.split("x")) for s in args.shapes.split(",") if s]
    batches = [int(b) for b in args.batches.split(",") if b]
    blocks = plan_blocks(shapes, batches, args.reps)

    if args.worker:  # child under rocprofv3: launch only
        run_worker(blocks, args.warmup, use_events=False)
        return

    if args.timer == "events":
        res = run_worker(blocks, args.warmup, use_events=True)
        per_block = [statistics.median(t) * 1e3 for t in res]
    else:
        rocprof = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
        outdir = tempfile.mkdtemp(prefix="dfk_tune_", dir=os.environ.get("TMPDIR", "/tmp"))
        cmd = [rocprof, "--kernel-trace", "--output-format", "csv", "-d", outdir, "-o", "tune", "--",
               sys.executable, "-m", "swiglu_mlp_amd.tune", "--worker", "1", "--shapes", args.shapes,
               "--batches", args.batches, "--reps", str(args.reps), "--warmup", str(args.warmup)]
        print("running:", " ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, cwd=ROOT)
        per_block = block_costs(parse_rocprof(outdir), blocks, args.warmup)
        shutil.rmtree(outdir, ignore_errors=True)

    confirm = None
    if args.timer == "rocprof":
        cand = near_ties(blocks, per_block)
        if cand:
            cblocks = [dict(b, reps=max(b["reps"], 100)) for b in cand]
            print(f"confirming {len(cblocks)} near-tie variants untraced", flush=True)
            res = run_worker(cblocks, args.warmup, use_events=True)
            confirm = {}
            for b, t in zip(cblocks, res):
                confirm.setdefault(_key(b), {})[b["variant"]] = statistics.median(t) * 1e3

    entries = build_table(blocks, per_block, confirm)
    out = {"format": "dfk-tuning-v1", "arch": "gfx950", "timer": args.timer,
           "tie_rule": f"within {int(TIE * 100)}% of the best median -> row variant (VALU first)",
           "confirm_band": CONFIRM_BAND if args.timer == "rocprof" else None,
           "entries": entries}
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    for e in entries:
        ts = " ".join(f"{k}={v:8.2f}" for k, v in e["us"].items())
        cs = " | confirm " + " ".join(f"{k}={v:8.2f}" for k, v in e["confirm_us"].items()) if "confirm_us" in e else ""
        print(f"{e['op']:8s} B={e['B']:3d} {e['d_model']}x{e['d_ff']}: {e['winner']:9s} | {ts}{cs}", flush=True)
    print(f"wrote {args.out} ({len(entries)} entries)")


if __name__ == "__main__":
    main()
