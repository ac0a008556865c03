"""The C ABI on the host: symbols, argument checks, the scheduler's table logic.

No test here launches a kernel: every call either fails validation before any
HIP call or is host-only (dfk_schedule_select and the table functions).
"""
import ctypes
import json
import os
import re

import pytest

import swiglu_mlp_amd as dfk
from swiglu_mlp_amd import Layout, Status

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dfk.h")

# Fake device addresses: never dereferenced, because every call below fails
# validation first.  A is 16-byte aligned, MIS is not.
A = 0x10000
MIS = 0x10008
NULL = None


@pytest.fixture(scope="module")
def L():
    return dfk.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dfk_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_exported_set():
    assert header_functions() == sorted(dfk.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    for name in header_functions():
        assert hasattr(L, name), f"libdfk.so does not export {name}"


def test_strings(L):
    for s in Status:
        text = dfk.status_string(s)
        assert text.startswith("DFK_")
    assert dfk.status_string(99) == "DFK_ERR_UNKNOWN"
    names = [dfk.layout_name(l) for l in Layout]
    assert names == ["auto", "row", "col", "row_valu", "col_valu", "row_mfma", "col_mfma", "row_persistent"]
    assert dfk.layout_name(42) == "invalid"
    assert "gfx950" in dfk.version()


GU_OK = dict(x=A, wg=A, wu=A, h=A, B=1, dm=256, dff=688, layout=0)


def gate_up(L, x=A, wg=A, wu=A, h=A, B=1, dm=256, dff=688, layout=0):
    return L.dfk_gate_up_silu_mul(x, wg, wu, h, B, dm, dff, layout, None)


def down(L, h=A, wd=A, out=A, B=1, dm=256, dff=688, layout=0):
    return L.dfk_down_proj(h, wd, out, B, dm, dff, layout, None)


def mlp(L, x=A, wg=A, wu=A, wd=A, out=A, B=1, dm=256, dff=688, layout=0):
    return L.dfk_swiglu_mlp(x, wg, wu, wd, out, B, dm, dff, layout, None)


def mlp_noalloc(L, x=A, wg=A, wu=A, wd=A, out=A, B=1, dm=256, dff=688, layout=0):
    return L.dfk_swiglu_mlp_noalloc(x, wg, wu, wd, out, B, dm, dff, layout, None)


def norm_gate_up(L, x=A, gain=A, eps=1e-5, wg=A, wu=A, h=A, B=1, dm=256, dff=688, layout=0):
    return L.dfk_rmsnorm_gate_up_silu_mul(x, gain, eps, wg, wu, h, B, dm, dff, layout, None)


def norm_mlp(L, x=A, gain=A, eps=1e-5, wg=A, wu=A, wd=A, out=A, B=1, dm=256, dff=688, layout=0):
    return L.dfk_rmsnorm_swiglu_mlp(x, gain, eps, wg, wu, wd, out, B, dm, dff, layout, None)


def gu_packed(L, x=A, wgu=A, h=A, B=1, dm=256, dff=688, packing=0, layout=0):
    return L.dfk_gate_up_silu_mul_packed(x, wgu, h, B, dm, dff, packing, layout, None)


def mlp_packed(L, x=A, wgu=A, wd=A, out=A, B=1, dm=256, dff=688, packing=1, layout=0):
    return L.dfk_swiglu_mlp_packed(x, wgu, wd, out, B, dm, dff, packing, layout, None)


def gu_fp8(L, x=A, qg=A, sg=A, qu=A, su=A, h=A, B=1, dm=256, dff=688, layout=0):
    return L.dfk_gate_up_silu_mul_fp8(x, qg, sg, qu, su, h, B, dm, dff, layout, None)


def down_fp8(L, h=A, qd=A, sd=A, out=A, B=1, dm=256, dff=688, layout=0):
    return L.dfk_down_proj_fp8(h, qd, sd, out, B, dm, dff, layout, None)


def mlp_fp8(L, x=A, qg=A, sg=A, qu=A, su=A, qd=A, sd=A, out=A, B=1, dm=256, dff=688, layout=0):
    return L.dfk_swiglu_mlp_fp8(x, qg, sg, qu, su, qd, sd, out, B, dm, dff, layout, None)


FP8_FNS = [gu_fp8, down_fp8, mlp_fp8]


@pytest.mark.parametrize("fn", FP8_FNS, ids=["gu_fp8", "down_fp8", "mlp_fp8"])
def test_fp8_invalid_arguments(L, fn):
    import inspect
    params = inspect.signature(fn).parameters
    for p in [p for p in params if p in ("x", "qg", "qu", "qd", "h", "out")]:
        assert fn(L, **{p: NULL}) == Status.INVALID_ARG, p
        assert fn(L, **{p: MIS}) == Status.MISALIGNED, p
    for p in [p for p in params if p in ("sg", "su", "sd")]:
        assert fn(L, **{p: NULL}) == Status.INVALID_ARG, p
        assert fn(L, **{p: A + 2}) == Status.MISALIGNED, p
    assert fn(L, B=0) == Status.INVALID_ARG
    assert fn(L, B=257) == Status.UNSUPPORTED
    assert fn(L, layout=8) == Status.INVALID_ARG


def rmsnorm(L, x=A, gain=A, eps=1e-5, out=A, B=1, dm=256):
    return L.dfk_rmsnorm(x, gain, eps, out, B, dm, None)


@pytest.mark.parametrize("fn", [gate_up, down, mlp, mlp_noalloc, norm_gate_up, norm_mlp, gu_packed, mlp_packed],
                         ids=["gate_up", "down", "mlp", "mlp_noalloc", "norm_gate_up", "norm_mlp", "gu_packed",
                              "mlp_packed"])
def test_invalid_arguments(L, fn):
    import inspect
    ptrs = [p for p in inspect.signature(fn).parameters
            if p in ("x", "gain", "wg", "wu", "wgu", "wd", "h", "out")]
    for p in ptrs:
        assert fn(L, **{p: NULL}) == Status.INVALID_ARG, p
        assert fn(L, **{p: MIS}) == Status.MISALIGNED, p
    assert fn(L, B=0) == Status.INVALID_ARG
    assert fn(L, B=-3) == Status.INVALID_ARG
    assert fn(L, dm=0) == Status.INVALID_ARG
    assert fn(L, dff=-8) == Status.INVALID_ARG
    assert fn(L, B=257) == Status.UNSUPPORTED
    assert fn(L, dm=260) == Status.UNSUPPORTED
    assert fn(L, dff=690) == Status.UNSUPPORTED
    assert fn(L, dm=65536, dff=32768) == Status.UNSUPPORTED  # d_model*d_ff >= 2^31
    assert fn(L, layout=8) == Status.INVALID_ARG
    assert fn(L, layout=-1) == Status.INVALID_ARG
    # validation order: a null pointer is reported before a bad size
    assert fn(L, B=0, **{ptrs[0]: NULL}) == Status.INVALID_ARG


@pytest.mark.parametrize("fn", [rmsnorm, norm_gate_up, norm_mlp], ids=["rmsnorm", "norm_gate_up", "norm_mlp"])
def test_invalid_eps(L, fn):
    for eps in (-1e-6, float("nan"), float("inf"), -float("inf")):
        assert fn(L, eps=eps) == Status.INVALID_ARG, eps


@pytest.mark.parametrize("fn", [gu_packed, mlp_packed], ids=["gu_packed", "mlp_packed"])
def test_invalid_packing(L, fn):
    for packing in (-1, 2, 7):
        assert fn(L, packing=packing) == Status.INVALID_ARG, packing


def test_rmsnorm_invalid_arguments(L):
    for p in ("x", "gain", "out"):
        assert rmsnorm(L, **{p: NULL}) == Status.INVALID_ARG, p
        assert rmsnorm(L, **{p: MIS}) == Status.MISALIGNED, p
    assert rmsnorm(L, B=0) == Status.INVALID_ARG
    assert rmsnorm(L, dm=-8) == Status.INVALID_ARG
    assert rmsnorm(L, B=257) == Status.UNSUPPORTED
    assert rmsnorm(L, dm=260) == Status.UNSUPPORTED


def test_schedule_select_argument_checks(L):
    g, d = ctypes.c_int(), ctypes.c_int()
    assert L.dfk_schedule_select(1, 4096, 14336, None, ctypes.byref(d)) == Status.INVALID_ARG
    assert L.dfk_schedule_select(1, 4096, 14336, ctypes.byref(g), None) == Status.INVALID_ARG
    assert L.dfk_schedule_select(0, 4096, 14336, ctypes.byref(g), ctypes.byref(d)) == Status.INVALID_ARG
    assert L.dfk_schedule_select(300, 4096, 14336, ctypes.byref(g), ctypes.byref(d)) == Status.UNSUPPORTED
    assert L.dfk_schedule_select(1, 4095, 14336, ctypes.byref(g), ctypes.byref(d)) == Status.UNSUPPORTED


# ----------------------------------------------------------------- tables --

def lib_versions():
    from swiglu_mlp_amd import tune
    return tune.library_versions()


def write_table(path, entries, arch="gfx950", fmt="dfk-tuning-v2", versions=None):
    lib, rocm = versions or lib_versions()
    with open(path, "w") as f:
        json.dump({"format": fmt, "arch": arch, "lib_version": lib, "rocm_version": rocm, "entries": entries}, f)
    return str(path)


def entry(op, B, dm, dff, winner):
    return {"op": op, "B": B, "d_model": dm, "d_ff": dff, "winner": winner,
            "us": {winner: 1.0}}


@pytest.fixture
def restore_table():
    yield
    os.environ.pop("DFK_FORCE_LAYOUT", None)
    try:
        dfk.dfk_load_tuning_table(None)
    except dfk.DfkError:
        pass


def test_table_exact_nearest_and_heuristic(tmp_path, restore_table):
    path = write_table(tmp_path / "t.json", [
        entry("gate_up", 1, 4096, 14336, "col_valu"),
        entry("down", 1, 4096, 14336, "row_mfma"),
        entry("gate_up", 4, 4096, 14336, "row_mfma"),
        entry("down", 4, 4096, 14336, "col_valu"),
        entry("gate_up", 16, 4096, 14336, "row_mfma"),
        entry("down", 16, 4096, 14336, "col_mfma"),
    ])
    dfk.dfk_load_tuning_table(path)
    assert dfk.dfk_tuning_table_source() == path
    S = dfk.dfk_schedule_select
    assert S(1, 4096, 14336) == (Layout.COL_VALU, Layout.ROW_MFMA)       # exact
    assert S(4, 4096, 14336) == (Layout.ROW_MFMA, Layout.COL_VALU)       # exact
    assert S(2, 4096, 14336) == (Layout.ROW_MFMA, Layout.COL_VALU)       # nearest tuned B >= 2 is 4
    assert S(9, 4096, 14336) == (Layout.ROW_MFMA, Layout.COL_MFMA)       # -> 16
    assert S(64, 4096, 14336) == (Layout.ROW_MFMA, Layout.COL_MFMA)      # largest below
    # a VALU winner from a smaller batch cannot serve B > 8: same traversal, MFMA
    path2 = write_table(tmp_path / "t2.json", [entry("gate_up", 8, 4096, 14336, "col_valu"),
                                                entry("down", 8, 4096, 14336, "row_valu")])
    dfk.dfk_load_tuning_table(path2)
    assert S(32, 4096, 14336) == (Layout.COL_MFMA, Layout.ROW_MFMA)
    # untuned shape -> heuristic: VALU rows at small batch, MFMA panels above
    assert S(1, 2048, 5632) == (Layout.ROW_VALU, Layout.ROW_VALU)
    assert S(16, 2048, 5632) == (Layout.COL_MFMA, Layout.COL_MFMA)
    # x too large for the VALU kernel's LDS (B * d_model * 2 > 160 KB) -> MFMA
    assert S(8, 16384, 1024)[0] == Layout.ROW_MFMA


def test_force_layout_env(tmp_path, restore_table):
    path = write_table(tmp_path / "t.json", [entry("gate_up", 1, 4096, 14336, "row_valu"),
                                               entry("down", 1, 4096, 14336, "row_mfma")])
    dfk.dfk_load_tuning_table(path)
    os.environ["DFK_FORCE_LAYOUT"] = "col"
    assert dfk.dfk_schedule_select(1, 4096, 14336) == (Layout.COL_VALU, Layout.COL_MFMA)
    os.environ["DFK_FORCE_LAYOUT"] = "row"
    assert dfk.dfk_schedule_select(1, 4096, 14336) == (Layout.ROW_VALU, Layout.ROW_MFMA)


_V = '"lib_version": "%s", "rocm_version": "%s"'


@pytest.mark.parametrize("content", [
    "not json", '{"format": "dfk-tuning-v2", "arch": "gfx950", %V}',
    '{"format": "other", "arch": "gfx950", %V, "entries": []}',
    '{"format": "dfk-tuning-v1", "arch": "gfx950", "entries": []}',
    '{"format": "dfk-tuning-v2", "arch": "gfx950", "entries": []}',
    '{"format": "dfk-tuning-v2", "arch": "gfx942", %V, "entries": []}',
    '{"format": "dfk-tuning-v2", "arch": "gfx950", %V, "entries": [{"op": "gate_up"}]}',
    '{"format": "dfk-tuning-v2", "arch": "gfx950", %V, "entries": [{"op": "x", "B": 1, "d_model": 8, "d_ff": 8, "winner": "row_valu"}]}',
    '{"format": "dfk-tuning-v2", "arch": "gfx950", %V, "entries": [{"op": "down", "B": 1, "d_model": 8, "d_ff": 8, "winner": "diag"}]}',
    '{"format": "dfk-tuning-v2", "arch": "gfx950", %V, "entries": [{"op": "gate_up_fp8", "B": 1, "d_model": 16, "d_ff": 16, "winner": "col_valu"}]}',
])
def test_bad_table_falls_back_to_heuristic(tmp_path, content, restore_table):
    p = tmp_path / "bad.json"
    p.write_text(content.replace("%V", _V % lib_versions()))
    with pytest.raises(dfk.DfkError) as e:
        dfk.dfk_load_tuning_table(str(p))
    assert e.value.status == Status.INVALID_ARG
    assert dfk.dfk_tuning_table_source() == "heuristic"
    assert dfk.dfk_schedule_select(1, 4096, 14336) == (Layout.ROW_VALU, Layout.ROW_VALU)


@pytest.mark.parametrize("which", ["lib", "rocm"])
def test_table_for_another_version_is_not_used(tmp_path, which, restore_table):
    """A table tuned for another library or HIP version falls back to the
    heuristic, and the table source names the mismatch (re-tune then)."""
    lib, rocm = lib_versions()
    vers = ("0.0.1", rocm) if which == "lib" else (lib, "1.2.3")
    path = write_table(tmp_path / "old.json", [entry("gate_up", 1, 4096, 14336, "col_mfma"),
                                                entry("down", 1, 4096, 14336, "col_mfma")], versions=vers)
    with pytest.raises(dfk.DfkError):
        dfk.dfk_load_tuning_table(path)
    src = dfk.dfk_tuning_table_source()
    assert src.startswith("heuristic (table ") and path in src and (vers[0] in src and vers[1] in src)
    assert dfk.dfk_schedule_select(1, 4096, 14336) == (Layout.ROW_VALU, Layout.ROW_VALU)


def test_fp8_entries_load_beside_bf16(tmp_path, restore_table):
    """FP8 entries (gate_up_fp8 / down_fp8) load with the bf16 ones and leave
    the bf16 schedule alone."""
    path = write_table(tmp_path / "t.json", [entry("gate_up", 1, 4096, 14336, "row_valu"),
                                               entry("down", 1, 4096, 14336, "row_valu"),
                                               entry("gate_up_fp8", 1, 4096, 14336, "col_mfma"),
                                               entry("down_fp8", 1, 4096, 14336, "row_mfma")])
    dfk.dfk_load_tuning_table(path)
    assert dfk.dfk_tuning_table_source() == path
    assert dfk.dfk_schedule_select(1, 4096, 14336) == (Layout.ROW_VALU, Layout.ROW_VALU)


def test_missing_table(tmp_path, restore_table):
    with pytest.raises(dfk.DfkError):
        dfk.dfk_load_tuning_table(str(tmp_path / "nope.json"))
    assert dfk.dfk_tuning_table_source() == "heuristic"


def test_installed_table_parses(restore_table):
    """The table shipped with the package (if any) loads and names only known variants."""
    if not os.path.exists(dfk.TUNING_TABLE):
        pytest.skip("no tuning table installed yet")
    t = json.load(open(dfk.TUNING_TABLE))
    assert (t["lib_version"], t["rocm_version"]) == lib_versions(), "the installed table is stale: re-tune"
    dfk.dfk_load_tuning_table(dfk.TUNING_TABLE)
    assert dfk.dfk_tuning_table_source() == dfk.TUNING_TABLE
    for e in t["entries"]:
        if e["op"].endswith("_fp8"):
            continue  # the FP8 entry points' AUTO reads these; no public query
        g, d = dfk.dfk_schedule_select(e["B"], e["d_model"], e["d_ff"])
        got = g if e["op"] == "gate_up" else d
        assert dfk.layout_name(got) == e["winner"]


def test_stream_read_argument_checks(L):
    L.dfk_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert L.dfk_stream_read(NULL, 1024, A, None) == Status.INVALID_ARG
    assert L.dfk_stream_read(A, 1024, NULL, None) == Status.INVALID_ARG
    assert L.dfk_stream_read(A, 0, A, None) == Status.INVALID_ARG
    assert L.dfk_stream_read(A, 1000, A, None) == Status.UNSUPPORTED
    assert L.dfk_stream_read(MIS, 1024, A, None) == Status.MISALIGNED
    assert L.dfk_stream_read(A, 1024, A + 2, None) == Status.MISALIGNED
