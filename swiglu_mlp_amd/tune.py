"""Profiler-driven tuning of the row / column kernel variants.

    python -m swiglu_mlp_amd.tune [--shapes 4096x14336,...] [--batches 1,2,4,...]
                                  [--ops gate_up,down,gate_up_fp8,down_fp8]
                                  [--timer rocprof|events] [--out PATH]

For every (d_model, d_ff) shape, batch B and op (gate_up, down and their FP8
weight-only forms gate_up_fp8, down_fp8), each variant that can run the shape
(row_valu, col_valu, row_mfma, col_mfma; FP8 gate-up has no col_valu, FP8 down
has it up to B = 4) is launched back
to back with rotating weight copies (at least 1.5 GB of distinct weights, so
every launch streams from HBM rather than the 256 MB Infinity Cache).  The
winner is the variant with the lowest median per-call cost; variants within
2 % of the best count as a tie, which goes to a row variant (VALU first).  The
result is the JSON table that dfk_schedule_select (and the FP8 entry points'
AUTO layout) read.

A preflight pass (untraced) calls every variant once; one that fails to launch
is ineligible: it is recorded in its entry and never wins.

Timers:
  rocprof  (default) the worker runs under `rocprofv3 --kernel-trace`; a call's
           cost is the sum of its kernels' durations in the trace (the kernel,
           plus the split-sum reduce kernel of the K-split down variants).
           Variants within CONFIRM_BAND of the profile's best are then re-timed
           untraced (HIP events around back-to-back calls) and that decides
           among them; each entry records which timer decided it.
  events   HIP events around groups of back-to-back launches only.

This is the variant scheduling of "Deep Kernel Fusion for Transformer
Decoding" (podcast episode page, episode summary: profiling picks the row- or
column-walking variant while serving), with the profiler as the measuring
instrument.
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
OPS = ["gate_up", "down", "gate_up_fp8", "down_fp8"]
VARIANTS = ["row_valu", "col_valu", "row_mfma", "col_mfma"]
FP8_MAX_BATCH = 128  # the FP8 entry points' limit (matrix cores)
# Variants within this fraction of the best count as a tie (a row variant,
# VALU first, wins a tie).
TIE = 0.02
# Variants within this fraction of the profile's best (summed kernel
# durations) are re-timed back to back with HIP events and no profiler
# attached, and that decides among them.  Kernel durations leave out what a
# stream of calls also pays between kernels (the launch gap and the
# kernel's ramp differ between variants: measured on MI355X, the
# LDS-transposed matrix-core kernels end ~1-4 us further apart than their
# durations, the vector-ALU kernels ~1 us), so close calls are settled by
# the untraced stream; the profile rules out the variants far behind.
CONFIRM_BAND = 0.15
ROTATE_BYTES = 1.5e9


def layer_bytes(d_model, d_ff, fp8=False):
    return 3 * d_model * d_ff * (1 if fp8 else 2)


def runnable(variant, op, B, d_model):
    fp8 = op.endswith("_fp8")
    if fp8 and B > FP8_MAX_BATCH:
        return False
    # FP8 codes: the vector-ALU column walk exists for down only (h in
    # registers, B <= 4)
    if fp8 and variant == "col_valu" and (op != "down_fp8" or B > 4):
        return False
    if variant.endswith("valu"):
        if B > 8:
            return False
        if op.startswith("gate_up") and B * d_model * 2 > 160 * 1024:
            return False
    return True


def plan_blocks(shapes, batches, reps, ops=("gate_up", "down")):
    """The launch sequence: (shape, B, op, variant, reps) blocks in order,
    shapes outermost (one weight set per shape and weight type)."""
    blocks = []
    for (dm, dff) in shapes:
        for fp8 in (False, True):
            for B in batches:
                for op in ops:
                    if op.endswith("_fp8") != fp8:
                        continue
                    if fp8 and (dm % 16 or dff % 16):
                        continue
                    for v in VARIANTS:
                        if runnable(v, op, B, dm):
                            blocks.append({"d_model": dm, "d_ff": dff, "B": B, "op": op, "variant": v,
                                           "reps": reps})
    return blocks


def _fp8_codes(rows, cols, seed, dev):
    """E4M3 codes and per-row scales of a seeded N(0, 0.02^2) weight (the
    benchmark's recipe)."""
    import torch
    from swiglu_mlp_amd import inputs
    w = inputs.randn_bf16_device((rows, cols), 0.02, seed, dev).float()
    s = (w.abs().amax(dim=1) / 448.0).clamp_min(1e-30)
    return (w / s[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), s.contiguous()


def run_worker(blocks, warmup, use_events, preflight=False):
    """Launch every block.  Returns per-block event timings (ms per launch) if
    asked; with preflight, one call per block and the error text of each
    block that fails (None where it runs)."""
    import torch
    import swiglu_mlp_amd as dfk
    from swiglu_mlp_amd import Layout, inputs

    dev = torch.device("cuda:0")
    dfk.lib()
    layout_of = {"row_valu": Layout.ROW_VALU, "col_valu": Layout.COL_VALU,
                 "row_mfma": Layout.ROW_MFMA, "col_mfma": Layout.COL_MFMA}
    results = []
    cur, sets = None, None
    for blk in blocks:
        dm, dff = blk["d_model"], blk["d_ff"]
        fp8 = blk["op"].endswith("_fp8")
        if (dm, dff, fp8) != cur:
            sets = None
            torch.cuda.empty_cache()
            R = max(2, math.ceil(ROTATE_BYTES / layer_bytes(dm, dff, fp8)))
            if fp8:
                sets = [(*_fp8_codes(dff, dm, 9600 + 10 * r + 1, dev), *_fp8_codes(dff, dm, 9600 + 10 * r + 2, dev),
                         *_fp8_codes(dm, dff, 9600 + 10 * r + 3, dev)) for r in range(R)]
            else:
                sets = [(inputs.randn_bf16_device((dff, dm), 0.02, 9000 + 10 * r + 1, dev),
                         inputs.randn_bf16_device((dff, dm), 0.02, 9000 + 10 * r + 2, dev),
                         inputs.randn_bf16_device((dm, dff), 0.02, 9000 + 10 * r + 3, dev)) for r in range(R)]
            cur = (dm, dff, fp8)
            print(f"tune worker: {dm}x{dff} {'fp8' if fp8 else 'bf16'} weights", flush=True)
        B = blk["B"]
        x = inputs.randn_bf16_device((B, dm), 1.0, 9500 + B, dev)
        h = torch.randn((B, dff), device=dev, dtype=torch.float32)
        y = torch.empty((B, dm), device=dev, dtype=torch.bfloat16)
        lay = layout_of[blk["variant"]]
        R = len(sets)
        op = blk["op"]
        if op == "gate_up":
            def call(i):
                wg, wu, _ = sets[i % R]
                dfk.dfk_gate_up_silu_mul(x, wg, wu, h, layout=lay)
        elif op == "down":
            def call(i):
                dfk.dfk_down_proj(h, sets[i % R][2], y, layout=lay)
        elif op == "gate_up_fp8":
            def call(i):
                qg, sg, qu, su, _, _ = sets[i % R]
                dfk.dfk_gate_up_silu_mul_fp8(x, qg, sg, qu, su, h, layout=lay)
        else:
            def call(i):
                s = sets[i % R]
                dfk.dfk_down_proj_fp8(h, s[4], s[5], y, layout=lay)
        if preflight:
            try:
                call(0)
                torch.cuda.synchronize()
                results.append(None)
            except dfk.DfkError as e:
                results.append(str(e))
            continue
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
    """One record per library call, in dispatch order: (name, start_ns,
    end_ns, busy_ns).  A call is one kernel, except the K-split down
    variants, whose kernel is followed by a reduce kernel: that call runs from
    the first kernel's start to the reduce kernel's end, and busy_ns adds the
    two kernels' durations."""
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
            first_name, first_start, _, busy = calls[-1]
            calls[-1] = (first_name, first_start, end, busy + (end - start))
        else:
            calls.append((name, start, end, end - start))
    return calls


def block_costs(calls, blocks, warmup):
    """Median per-call cost (us) of each block's timed calls, in dispatch
    order: the summed kernel durations of each call."""
    expect = sum(warmup + b["reps"] for b in blocks)
    if len(calls) != expect:
        raise RuntimeError(f"expected {expect} library calls in the trace, found {len(calls)}")
    out, i = [], 0
    for b in blocks:
        busy = [c[3] for c in calls[i + warmup:i + warmup + b["reps"]]]
        out.append(statistics.median(busy) / 1e3)
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


def build_table(blocks, per_block_us, confirm=None, ineligible=None, timer="rocprof"):
    """Table entries.  `confirm` maps (op, B, d_model, d_ff) -> {variant: us}
    from the untraced re-timing, which then decides among its variants;
    `ineligible` maps the same key -> {variant: error} (never a winner)."""
    table = {}
    for blk, us in zip(blocks, per_block_us):
        table.setdefault(_key(blk), {})[blk["variant"]] = round(us, 3)
    for key in (ineligible or {}):
        table.setdefault(key, {})
    entries = []
    for key, t in sorted(table.items(), key=lambda kv: (kv[0][2], kv[0][3], kv[0][1], kv[0][0])):
        op, B, dm, dff = key
        bad = (ineligible or {}).get(key, {})
        ok = {v: u for v, u in t.items() if v not in bad}
        if not ok:
            continue  # nothing runs this shape: the library's fallback decides
        e = {"op": op, "B": B, "d_model": dm, "d_ff": dff, "us": t}
        if confirm and key in confirm:
            e["confirm_us"] = {v: round(u, 3) for v, u in confirm[key].items()}
            e["winner"] = choose({v: u for v, u in confirm[key].items() if v not in bad})
            e["decided_by"] = "events"
        else:
            e["winner"] = choose(ok)
            e["decided_by"] = timer
        if bad:
            e["ineligible"] = dict(bad)
        entries.append(e)
    return entries


def library_versions():
    """(lib_version, rocm_version) of the loaded library, from dfk_version()
    ("dfk X gfx950 (HIP Y)")."""
    import swiglu_mlp_amd as dfk
    v = dfk.version()
    lib = v.split()[1]
    rocm = v.split("(HIP ", 1)[1].rstrip(")")
    return lib, rocm


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--shapes", default=",".join(f"{a}x{b}" for a, b in DEFAULT_SHAPES))
    ap.add_argument("--batches", default=",".join(map(str, DEFAULT_BATCHES)))
    ap.add_argument("--ops", default=",".join(OPS))
    ap.add_argument("--reps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--timer", choices=["rocprof", "events"], default="rocprof")
    ap.add_argument("--out", default=os.path.join(PKG, "tuning", "gfx950.json"))
    ap.add_argument("--worker", help=argparse.SUPPRESS)
    ap.add_argument("--preflight", help=argparse.SUPPRESS)
    ap.add_argument("--skip", default="", help=argparse.SUPPRESS)
    args = ap.parse_args()

    shapes = [tuple(int(v) for v in s.split("x")) for s in args.shapes.split(",") if s]
    batches = [int(b) for b in args.batches.split(",") if b]
    ops = [o for o in args.ops.split(",") if o]
    unknown = set(ops) - set(OPS)
    if unknown:
        ap.error(f"unknown ops {sorted(unknown)}")
    blocks = plan_blocks(shapes, batches, args.reps, ops)

    if args.preflight:  # child: one call per block, errors to a JSON file
        errs = run_worker(blocks, 0, use_events=False, preflight=True)
        with open(args.preflight, "w") as f:
            json.dump(errs, f)
        return
    skip = {int(i) for i in args.skip.split(",") if i}
    if args.worker:  # child under rocprofv3: launch only
        run_worker([b for i, b in enumerate(blocks) if i not in skip], args.warmup, use_events=False)
        return

    # preflight in a child process: a variant that fails to launch is
    # ineligible and left out of the timed runs
    with tempfile.TemporaryDirectory(prefix="dfk_tune_", dir=os.environ.get("TMPDIR", "/tmp")) as tmp:
        pf = os.path.join(tmp, "preflight.json")
        subprocess.run([sys.executable, "-m", "swiglu_mlp_amd.tune", "--preflight", pf, "--shapes", args.shapes,
                        "--batches", args.batches, "--ops", args.ops], check=True, cwd=ROOT)
        errs = json.load(open(pf))
    ineligible, skip = {}, []
    for i, (b, e) in enumerate(zip(blocks, errs)):
        if e is not None:
            ineligible.setdefault(_key(b), {})[b["variant"]] = e
            skip.append(i)
    timed_blocks = [b for i, b in enumerate(blocks) if i not in set(skip)]
    if skip:
        print(f"{len(skip)} variants failed to launch and are ineligible", flush=True)

    if args.timer == "events":
        res = run_worker(timed_blocks, args.warmup, use_events=True)
        per_block = [statistics.median(t) * 1e3 for t in res]
    else:
        rocprof = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
        outdir = tempfile.mkdtemp(prefix="dfk_tune_", dir=os.environ.get("TMPDIR", "/tmp"))
        cmd = [rocprof, "--kernel-trace", "--output-format", "csv", "-d", outdir, "-o", "tune", "--",
               sys.executable, "-m", "swiglu_mlp_amd.tune", "--worker", "1", "--shapes", args.shapes,
               "--batches", args.batches, "--ops", args.ops, "--reps", str(args.reps),
               "--warmup", str(args.warmup), "--skip", ",".join(map(str, skip))]
        print("running:", " ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, cwd=ROOT)
        per_block = block_costs(parse_rocprof(outdir), timed_blocks, args.warmup)
        shutil.rmtree(outdir, ignore_errors=True)

    confirm = None
    if args.timer == "rocprof":
        cand = near_ties(timed_blocks, per_block)
        if cand:
            cblocks = [dict(b, reps=max(b["reps"], 100)) for b in cand]
            print(f"confirming {len(cblocks)} near-tie variants untraced", flush=True)
            res = run_worker(cblocks, args.warmup, use_events=True)
            confirm = {}
            for b, t in zip(cblocks, res):
                confirm.setdefault(_key(b), {})[b["variant"]] = statistics.median(t) * 1e3

    import swiglu_mlp_amd as dfk
    dfk.lib()
    lib_version, rocm_version = library_versions()
    entries = build_table(timed_blocks, per_block, confirm, ineligible, timer=args.timer)
    out = {"format": "dfk-tuning-v2", "arch": "gfx950", "lib_version": lib_version, "rocm_version": rocm_version,
           "timer": args.timer,
           "cost": ("summed kernel durations per call (rocprofv3 kernel trace)" if args.timer == "rocprof"
                    else "HIP events around back-to-back calls"),
           "tie_rule": f"within {int(TIE * 100)}% of the best median -> row variant (VALU first)",
           "confirm_band": CONFIRM_BAND if args.timer == "rocprof" else None,
           "entries": entries}
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    for e in entries:
        ts = " ".join(f"{k}={v:8.2f}" for k, v in e["us"].items())
        cs = " | confirm " + " ".join(f"{k}={v:8.2f}" for k, v in e["confirm_us"].items()) if "confirm_us" in e else ""
        print(f"{e['op']:11s} B={e['B']:3d} {e['d_model']}x{e['d_ff']}: {e['winner']:9s} ({e['decided_by']}) | {ts}{cs}",
              flush=True)
    print(f"wrote {args.out} ({len(entries)} entries)")


if __name__ == "__main__":
    main()
