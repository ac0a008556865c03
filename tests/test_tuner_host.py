"""Host logic of the profiler-driven tuner (no GPU): trace parsing, the
per-call cost taken from summed kernel durations, the winner rule, FP8 ops,
ineligible variants and the table's version fields."""
import csv
import os

import pytest

from swiglu_mlp_amd import tune


def write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_parse_merges_reduce_kernels_and_skips_foreign(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    write_trace(d / "x_kernel_trace.csv", [
        {"Dispatch_Id": 3, "Kernel_Name": "void dfk::panel_reduce_kernel(float const*)", "Start_Timestamp": 250, "End_Timestamp": 260},
        {"Dispatch_Id": 1, "Kernel_Name": "void dfk::down_valu_row_kernel<1>(dfk::DownArgs)", "Start_Timestamp": 0, "End_Timestamp": 100},
        {"Dispatch_Id": 2, "Kernel_Name": "void dfk::down_mfma_panel_kernel<1>(dfk::DownArgs)", "Start_Timestamp": 120, "End_Timestamp": 240},
        {"Dispatch_Id": 4, "Kernel_Name": "__amd_rocclr_fillBufferAligned", "Start_Timestamp": 300, "End_Timestamp": 310},
    ])
    calls = tune.parse_rocprof(str(d))
    assert [(s, e) for _, s, e, _ in calls] == [(0, 100), (120, 260)]
    assert "panel_kernel" in calls[1][0]
    # the K-split call's cost is its two kernels' durations, not the gap between them
    assert [b for _, _, _, b in calls] == [100, 120 + 10]


def test_block_costs_use_summed_durations():
    blocks = [{"reps": 3}, {"reps": 2}]
    # warm-up 1 per block (not counted); busy times 5 | 10, 11, 12 | 40 | 50, 55
    busy = [5, 10, 11, 12, 40, 50, 55]
    calls = [("k", 1000 * i, 1000 * i + b, b) for i, b in enumerate(busy)]
    out = tune.block_costs(calls, blocks, warmup=1)
    assert out == pytest.approx([11e-3, 52.5e-3])


def test_block_costs_check_counts():
    with pytest.raises(RuntimeError):
        tune.block_costs([("k", 0, 1, 1)] * 3, [{"reps": 3}], warmup=1)


def test_choose_tie_goes_to_row():
    assert tune.choose({"row_valu": 10.15, "col_valu": 10.0}) == "row_valu"     # within 2 %
    assert tune.choose({"row_valu": 10.3, "col_valu": 10.0}) == "col_valu"      # beyond 2 %
    assert tune.choose({"row_valu": 10.15, "row_mfma": 10.0}) == "row_valu"     # VALU first in a tie
    assert tune.choose({"col_mfma": 9.0, "row_mfma": 9.1, "row_valu": 12.0}) == "row_mfma"
    assert tune.choose({"col_mfma": 9.0, "row_mfma": 9.5}) == "col_mfma"


def test_table_entries_are_sorted_and_complete():
    blocks = tune.plan_blocks([(256, 688)], [1, 16], reps=5)
    ops = {(b["op"], b["B"]) for b in blocks}
    assert ops == {("gate_up", 1), ("down", 1), ("gate_up", 16), ("down", 16)}
    # VALU variants only up to B = 8
    assert not any(b["variant"].endswith("valu") and b["B"] > 8 for b in blocks)
    entries = tune.build_table(blocks, [float(i + 1) for i in range(len(blocks))])
    assert all(e["winner"] in e["us"] for e in entries)
    assert [e["B"] for e in entries] == sorted(e["B"] for e in entries)


def test_near_ties_and_confirmed_winner():
    blocks = tune.plan_blocks([(4096, 14336)], [4], reps=5)
    # profile: gate_up row_mfma best, row_valu 3 % behind, the rest far behind
    prof = {("gate_up", "row_mfma"): 39.0, ("gate_up", "row_valu"): 40.2, ("gate_up", "col_valu"): 45.0,
            ("gate_up", "col_mfma"): 42.8, ("down", "row_valu"): 41.0, ("down", "col_valu"): 35.0,
            ("down", "row_mfma"): 26.0, ("down", "col_mfma"): 26.1}
    per = [prof[(b["op"], b["variant"])] for b in blocks]
    cand = tune.near_ties(blocks, per, band=0.10)
    got = {(b["op"], b["variant"]) for b in cand}
    assert got == {("gate_up", "row_mfma"), ("gate_up", "row_valu"), ("gate_up", "col_mfma"),
                   ("down", "row_mfma"), ("down", "col_mfma")}
    # untraced re-timing reverses the gate-up order: it decides
    confirm = {("gate_up", 4, 4096, 14336): {"row_mfma": 41.5, "row_valu": 39.6, "col_mfma": 43.0},
               ("down", 4, 4096, 14336): {"row_mfma": 26.0, "col_mfma": 26.2}}
    entries = {(e["op"]): e for e in tune.build_table(blocks, per, confirm)}
    assert entries["gate_up"]["winner"] == "row_valu"
    assert entries["down"]["winner"] == "row_mfma"
    assert "confirm_us" in entries["gate_up"]
    assert entries["gate_up"]["decided_by"] == "events"
    # without a confirmation the profile decides, and the entry says so
    assert all(e["decided_by"] == "rocprof" for e in tune.build_table(blocks, per))


def test_fp8_ops_plan_and_limits():
    blocks = tune.plan_blocks([(4096, 14336), (4104, 14336)], [1, 16], reps=5,
                              ops=("gate_up", "gate_up_fp8", "down_fp8"))
    fp8 = [b for b in blocks if b["op"].endswith("_fp8")]
    # no vector-ALU column walk for gate-up over FP8 codes (down: B <= 4);
    # d_model 4104 is not a multiple of 16
    assert fp8 and all(b["d_model"] == 4096 for b in fp8)
    assert all(b["variant"] != "col_valu" for b in fp8 if b["op"] == "gate_up_fp8")
    assert {b["variant"] for b in fp8 if b["B"] == 1 and b["op"] == "gate_up_fp8"} == {"row_valu", "row_mfma",
                                                                                       "col_mfma"}
    assert {b["variant"] for b in fp8 if b["B"] == 1 and b["op"] == "down_fp8"} == {"row_valu", "col_valu",
                                                                                    "row_mfma", "col_mfma"}
    assert {b["variant"] for b in fp8 if b["B"] == 16} == {"row_mfma", "col_mfma"}
    # per shape, the bf16 blocks come before the FP8 ones (one weight set at a time)
    for dm in (4096, 4104):
        kinds = [b["op"].endswith("_fp8") for b in blocks if b["d_model"] == dm]
        assert kinds == sorted(kinds)


def test_ineligible_variant_never_wins():
    blocks = tune.plan_blocks([(256, 688)], [1], reps=5)
    per = [1.0 if b["variant"] == "col_mfma" else 5.0 for b in blocks]
    bad = {("down", 1, 256, 688): {"col_mfma": "DFK_ERR_HIP"}}
    entries = {e["op"]: e for e in tune.build_table(blocks, per, ineligible=bad)}
    assert entries["gate_up"]["winner"] == "col_mfma"
    assert entries["down"]["winner"] != "col_mfma"
    assert entries["down"]["ineligible"] == {"col_mfma": "DFK_ERR_HIP"}
