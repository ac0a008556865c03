"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every entry point x every variant on small ragged shapes (several tiles and a
ragged tail in each dimension), exact pins (worked example, integer inputs),
invariants (zeros, linearity in W_down, batch rows, neuron permutation,
determinism) and the full-size workloads in the configuration the benchmark
times.  Tolerances: y normwise max <= 1e-2 per row and mean <= 2e-3; h 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
import swiglu_mlp_amd as dfk
from swiglu_mlp_amd import Layout, Status, inputs
from tests import helpers as H
from tests import oracle_pins

pytestmark = pytest.mark.gpu

ENGINE_LAYOUTS = [Layout.ROW_VALU, Layout.COL_VALU, Layout.ROW_MFMA, Layout.COL_MFMA]
ALL_LAYOUTS = ENGINE_LAYOUTS + [Layout.ROW, Layout.COL, Layout.AUTO]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dfk.lib()  # the HIP library must load: there is no fallback
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def valu_ok(op, B, d_model):
    if B > 8:
        return False
    return not (op == "gate_up" and B * d_model * 2 > 160 * 1024)


def layouts_for(op, B, d_model):
    out = []
    for l in ALL_LAYOUTS:
        if l in (Layout.ROW_VALU, Layout.COL_VALU) and not valu_ok(op, B, d_model):
            continue
        out.append(l)
    return out


def to_dev(L, dev):
    return {k: H.dev_bf16(getattr(L, k), dev) for k in ("x", "w_gate", "w_up", "w_down")}


def gpu_gate_up(T, layout):
    h = dfk.dfk_gate_up_silu_mul(T["x"], T["w_gate"], T["w_up"], layout=layout)
    torch.cuda.synchronize()
    return h.double().cpu().numpy()


def gpu_down(h_np, wd, layout, dev):
    y = dfk.dfk_down_proj(H.dev_f32(h_np, dev), wd, layout=layout)
    torch.cuda.synchronize()
    return y


def gpu_mlp(T, layout):
    y = dfk.dfk_swiglu_mlp(T["x"], T["w_gate"], T["w_up"], T["w_down"], layout=layout)
    torch.cuda.synchronize()
    return y


# shapes (B, d_model, d_ff): tiny workload, ragged chunk counts (d_model/8 not
# a multiple of 64), row counts not a multiple of any tile, batch above and
# below every tile boundary, and the largest batch (256)
SMALL_SHAPES = [
    (1, 256, 688), (1, 520, 1000), (2, 264, 72), (3, 1032, 200), (5, 136, 264),
    (8, 8, 8), (8, 520, 1000), (13, 128, 136), (16, 520, 1000), (17, 264, 456),
    (33, 1032, 200), (64, 136, 264), (256, 64, 48),
    # K long enough for the workgroup-cooperative kernels: ragged stage counts
    # (shifted last stages), a two-way K split with a short last split, and a
    # ragged last row tile
    (2, 4104, 264), (4, 264, 4104), (5, 600, 1096), (16, 1032, 2056),
    # h past the LDS limit: the vector-ALU down walk over K panels (2, 2 and
    # 5 panels, ragged last panel)
    (3, 136, 11008), (8, 64, 4112), (5, 264, 28680),
]


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "B%d_%dx%d" % s)
def test_small_shapes_all_variants(dev, orc, shape):
    B, dm, dff = shape
    L = inputs.tiny_layer() if shape == (1, 256, 688) else inputs.random_layer(B, dm, dff, seed=7000 + B + dm)
    T = to_dev(L, dev)
    _, _, h_ref = orc.gate_up(L.x, L.w_gate, L.w_up)
    y_ref, _ = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    h_in = inputs.h_like(B, dff, seed=7100 + B)
    yd_ref = orc.down(h_in, L.w_down)
    for layout in layouts_for("gate_up", B, dm):
        H.assert_h_close(gpu_gate_up(T, layout), h_ref, f"gate_up {layout.name} {shape}")
        H.assert_y_close(H.host_bf16_as_f64(gpu_mlp(T, layout)), y_ref, f"mlp {layout.name} {shape}")
    for layout in layouts_for("down", B, dm):
        y = gpu_down(h_in, T["w_down"], layout, dev)
        H.assert_y_close(H.host_bf16_as_f64(y), yd_ref, f"down {layout.name} {shape}")


# Seeded random shapes (d_model and d_ff multiples of 8 from 8 to 3072, B from
# 1 to 64, a few up to 256): every plan rule's boundary is crossed somewhere
# (chunks per lane and waves per workgroup of the h-in-registers walk, K
# panels, batch tiles, K splits), and every variant of every entry point is
# compared with the oracle.
def _random_shapes(n=24, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 20, 33, 64, 100, 256] if i % 4 == 0 else
                           [1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 17, 31, 48, 64]))
        dm = 8 * int(rng.integers(1, 385))
        dff = 8 * int(rng.integers(1, 385))
        out.append((B, dm, dff))
    return out


@pytest.mark.parametrize("shape", _random_shapes(), ids=lambda s: "B%d_%dx%d" % s)
def test_random_shapes_all_variants(dev, orc, shape):
    B, dm, dff = shape
    L = inputs.random_layer(B, dm, dff, seed=7700 + B + dm + dff)
    T = to_dev(L, dev)
    _, _, h_ref = orc.gate_up(L.x, L.w_gate, L.w_up)
    y_ref, _ = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    h_in = inputs.h_like(B, dff, seed=7800 + B)
    yd_ref = orc.down(h_in, L.w_down)
    for layout in layouts_for("gate_up", B, dm):
        H.assert_h_close(gpu_gate_up(T, layout), h_ref, f"gate_up {layout.name} {shape}")
        H.assert_y_close(H.host_bf16_as_f64(gpu_mlp(T, layout)), y_ref, f"mlp {layout.name} {shape}")
    for layout in layouts_for("down", B, dm):
        y = gpu_down(h_in, T["w_down"], layout, dev)
        H.assert_y_close(H.host_bf16_as_f64(y), yd_ref, f"down {layout.name} {shape}")


@pytest.mark.parametrize("op", ["gate_up", "down"])
def test_forced_valu_beyond_its_range_is_unsupported(dev, op):
    B, dm, dff = 16, 64, 48
    L = inputs.random_layer(B, dm, dff, seed=1)
    T = to_dev(L, dev)
    for layout in (Layout.ROW_VALU, Layout.COL_VALU):
        with pytest.raises(dfk.DfkError) as e:
            if op == "gate_up":
                dfk.dfk_gate_up_silu_mul(T["x"], T["w_gate"], T["w_up"], layout=layout)
            else:
                h = torch.zeros((B, dff), dtype=torch.float32, device=dev)
                dfk.dfk_down_proj(h, T["w_down"], layout=layout)
        assert e.value.status == Status.UNSUPPORTED


def test_worked_example_bits(dev):
    """x=[1,-2] example padded to 8x8: y must round to exactly 0x3F91, 0x3FA4."""
    x, wg, wu, wd = oracle_pins.worked_example()
    T = {"x": H.dev_bf16(x, dev), "w_gate": H.dev_bf16(wg, dev), "w_up": H.dev_bf16(wu, dev),
         "w_down": H.dev_bf16(wd, dev)}
    for layout in ALL_LAYOUTS:
        bits = H.host_bits(gpu_mlp(T, layout))
        assert list(bits[0]) == [0x3F91, 0x3FA4, 0, 0, 0, 0, 0, 0], layout.name


# Three batch tiles (33 <= B <= 48) with at least 640 row tiles (d_ff >= 10240
# on a 256-CU part): the regular-width staged-x gate-up kernel, whose x block
# is double-buffered.  Odd and even block counts, ragged last block and last
# row tile.
LTS_BT3_SHAPES = [(33, 1032, 10248), (48, 2048, 10240), (40, 520, 14344)]


@pytest.mark.parametrize("shape", LTS_BT3_SHAPES, ids=lambda s: "B%d_%dx%d" % s)
def test_gate_up_three_batch_tiles_wide(dev, orc, shape):
    B, dm, dff = shape
    L = inputs.random_layer(B, dm, dff, seed=7300 + B)
    T = to_dev(L, dev)
    _, _, h_ref = orc.gate_up(L.x, L.w_gate, L.w_up)
    y_ref, _ = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    for layout in (Layout.ROW_MFMA, Layout.ROW, Layout.AUTO):
        H.assert_h_close(gpu_gate_up(T, layout), h_ref, f"gate_up {layout.name} {shape}")
    H.assert_y_close(H.host_bf16_as_f64(gpu_mlp(T, Layout.ROW_MFMA)), y_ref, f"mlp ROW_MFMA {shape}")


# Down at three batch tiles (33 <= B <= 48) with at least one row tile per CU
# (d_model >= 4096 on a 256-CU part): the LDS-transposed staged-h kernel runs
# its four-batch-tile instance with 128-element K blocks, the fourth batch
# tile zero (a ragged last row tile at 4104 rows, a ragged last K block at
# d_ff 2056).  Every output against the oracle, and the plain and padded
# paths against each other through the integer exactness below.
DOWN_BT3_SHAPES = [(33, 4096, 2056), (40, 4104, 2056), (48, 4096, 3080)]


@pytest.mark.parametrize("shape", DOWN_BT3_SHAPES, ids=lambda s: "B%d_%dx%d" % s)
def test_down_three_batch_tiles_wide(dev, orc, shape):
    B, dm, dff = shape
    wd = inputs.randn_bf16((dm, dff), 1.0 / np.sqrt(dff), 7400 + B)
    h_in = inputs.h_like(B, dff, seed=7450 + B)
    want = orc.down(h_in, wd)
    wd_dev = H.dev_bf16(wd, dev)
    for layout in (Layout.COL_MFMA, Layout.COL, Layout.AUTO):
        y = gpu_down(h_in, wd_dev, layout, dev)
        H.assert_y_close(H.host_bf16_as_f64(y), want, f"down {layout.name} {shape}")
    # integer operands: exact in any order, so bit for bit
    hi = inputs.integer_h(B, dff, seed=7480 + B)
    wi = inputs.rand_int_bf16((dm, dff), -1, 1, seed=7490 + B)
    got = H.host_bits(gpu_down(hi, H.dev_bf16(wi, dev), Layout.COL_MFMA, dev))
    assert np.array_equal(got, orc.bf16_rne_array(orc.down(hi, wi))), f"integer {shape}"


# Down column walk with h held in registers (vector ALU, 2 <= B <= 8 where
# h fits the lane's registers): shapes where every workgroup walks several row
# groups, an odd number of them (5 and 3: the two-group turn plus a single
# tail group) and an even number (4), with one or two rows per group, slices
# of one to three chunks per lane and 8- and 16-wave workgroups.  Every output
# against the oracle; integer operands bit for bit.
DOWN_HREG_SHAPES = [(2, 8200, 1000), (2, 6144, 3000), (3, 2048, 9000), (4, 4096, 2056), (8, 4096, 1024)]


@pytest.mark.parametrize("shape", DOWN_HREG_SHAPES, ids=lambda s: "B%d_%dx%d" % s)
def test_down_h_in_registers_walks(dev, orc, shape):
    B, dm, dff = shape
    wd = inputs.randn_bf16((dm, dff), 1.0 / np.sqrt(dff), 7500 + B)
    h_in = inputs.h_like(B, dff, seed=7550 + B)
    want = orc.down(h_in, wd)
    y = gpu_down(h_in, H.dev_bf16(wd, dev), Layout.COL_VALU, dev)
    H.assert_y_close(H.host_bf16_as_f64(y), want, f"down COL_VALU {shape}")
    hi = inputs.integer_h(B, dff, seed=7580 + B)
    wi = inputs.rand_int_bf16((dm, dff), -1, 1, seed=7590 + B)
    got = H.host_bits(gpu_down(hi, H.dev_bf16(wi, dev), Layout.COL_VALU, dev))
    assert np.array_equal(got, orc.bf16_rne_array(orc.down(hi, wi))), f"integer {shape}"


@pytest.mark.parametrize("B", [1, 4, 8, 16, 64])
def test_integer_down_is_bitwise_exact(dev, orc, B):
    """Integer h (|h| <= 256) and W_down in {-1,0,1}: fp32 accumulation is exact
    in any order, so every variant must return RNE_bf16(exact y) bit for bit."""
    dm, dff = 1024, 14336
    h = inputs.integer_h(B, dff, seed=8000 + B)
    wd = inputs.rand_int_bf16((dm, dff), -1, 1, seed=8100 + B)
    want = orc.bf16_rne_array(orc.down(h, wd))
    wd_dev = H.dev_bf16(wd, dev)
    for layout in layouts_for("down", B, dm):
        got = H.host_bits(gpu_down(h, wd_dev, layout, dev))
        assert np.array_equal(got, want), layout.name


@pytest.mark.parametrize("B", [1, 3, 8, 16, 40])
def test_integer_gate_up_only_silu_rounds(dev, orc, B):
    """Integer x and weights in [-2, 2]: g and u are exact in fp32, so h differs
    from the oracle only by the fp32 SiLU and product rounding."""
    L = inputs.integer_layer(B, 2048, 1000, seed=8200 + B)
    T = to_dev(L, dev)
    _, _, h_ref = orc.gate_up(L.x, L.w_gate, L.w_up)
    for layout in layouts_for("gate_up", B, 2048):
        mx, mean = H.normwise(gpu_gate_up(T, layout), h_ref)
        assert mx <= 1e-6 and mean <= 1e-6, (layout.name, mx, mean)


def test_zero_invariants(dev):
    B, dm, dff = 8, 1032, 1000
    L = inputs.random_layer(B, dm, dff, seed=8300)
    T = to_dev(L, dev)
    cases = {"x": "x", "w_gate": "w_gate", "w_up": "w_up", "w_down": "w_down"}
    for name in cases:
        Z = dict(T)
        Z[name] = torch.zeros_like(T[name])
        for layout in layouts_for("gate_up", B, dm):
            y = gpu_mlp(Z, layout)
            assert torch.count_nonzero(y.float()).item() == 0, (name, layout.name)
            if name in ("x", "w_gate", "w_up"):
                h = gpu_gate_up(Z, layout)
                assert np.all(h == 0.0), (name, layout.name)


def bf16_ulp(v: torch.Tensor) -> torch.Tensor:
    """Spacing of bf16 values at |v| (8 significant bits)."""
    e = torch.floor(torch.log2(v.abs().clamp_min(2.0 ** -126)))
    return torch.pow(2.0, e - 7)


def uses_mfma(layout, B):
    return layout in (Layout.ROW_MFMA, Layout.COL_MFMA) or (
        layout in (Layout.ROW, Layout.COL) and B >= 16)


@pytest.mark.parametrize("B", [1, 8, 16])
def test_linearity_in_w_down_bitwise(dev, B):
    """y(2 W_down) = 2 y(W_down) bit for bit on every variant, and
    y(-W_down) = -y(W_down) bit for bit on the IEEE fp32 (VALU) path.  The
    matrix cores' accumulation is not sign-symmetric (isolated in
    test_sign_asymmetry_of_the_accumulators below), so on MFMA variants
    negation holds to one bf16 ulp per element."""
    L = inputs.random_layer(B, 1032, 1000, seed=8400 + B)
    T = to_dev(L, dev)
    T2 = dict(T, w_down=(T["w_down"].float() * 2).to(torch.bfloat16))
    Tn = dict(T, w_down=-T["w_down"])
    for layout in layouts_for("down", B, 1032):
        y = gpu_mlp(T, layout).float()
        assert torch.equal(gpu_mlp(T2, layout).float(), 2 * y), layout.name
        yn = gpu_mlp(Tn, layout).float()
        if layout == Layout.AUTO:
            continue  # AUTO resolves to one of the explicit variants checked here
        if uses_mfma(layout, B):
            assert torch.all((yn + y).abs() <= bf16_ulp(y)), layout.name
        else:
            assert torch.equal(yn, -y), layout.name


# Rows of W_up whose sum u = sum_k W_up[n, k] (x all ones) is the exact value
# 1 + 2^-23 + 2^-24 - 2^-40, just below the fp32 tie between 1 + 2^-23 and
# 1 + 2^-22, so correct rounding gives 0x3f800001; the terms sit in one or
# two 32-element K steps of the matrix-core contraction (and one or two
# 8-element lane chunks of the vector-ALU walk).
_SIGN_ROWS = {
    "a": {0: 1.0, 1: 2.0 ** -23, 32: 2.0 ** -24, 33: -2.0 ** -40},   # two K steps
    "b": {0: -2.0 ** -40, 32: 1.0, 33: 2.0 ** -23, 34: 2.0 ** -24},  # tiny term first
    "c": {0: 1.0, 1: 2.0 ** -23, 2: 2.0 ** -24, 3: -2.0 ** -40},     # one K step, one lane
}
# (u, u with W_up negated) as fp32 bits, measured on MI355X.
_SIGN_BITS = {
    "valu": {"a": (0x3F800001, 0xBF800001), "b": (0x3F800002, 0xBF800002), "c": (0x3F800001, 0xBF800002)},
    "mfma": {"a": (0x3F800001, 0xBF800002), "b": (0x3F800001, 0xBF800002), "c": (0x3F800002, 0xBF800002)},
}


def test_sign_asymmetry_of_the_accumulators(dev):
    """The smallest library calls that show why negating a weight matrix is
    not bit-exact on every engine.  With x = 1 and W_gate[n] = (64, 0, ...),
    g = 64 and SiLU(64) = 64 exactly in fp32, so h / 64 is u's fp32 sum.

    - Vector ALU (bf16 dot2 into an fp32 lane sum, then an fp32 lane
      reduction): row c, whose tiny opposite-signed term shares a dot2 with
      the tie-making term, rounds toward minus infinity (two's complement
      truncation of the aligned addend): 0x3f800001 but 0xbf800002.
    - Matrix cores (v_mfma_f32_16x16x32_bf16): inside one instruction the
      products' tiny term is dropped toward zero (row c: symmetric, tie to
      even), but when the products are added to a non-zero accumulator from
      an earlier K step (rows a, b) the tiny opposite-signed term again
      rounds toward minus infinity: asymmetric.
    - The fp32 FMA of the vector-ALU down projection is IEEE and symmetric
      (test_linearity_in_w_down_bitwise holds negation bit for bit there).
    All of these stay within one ulp of the correctly rounded sum."""
    K, N = 256, 16
    x = torch.ones((1, K), dtype=torch.bfloat16, device=dev)
    wg = torch.zeros((N, K), dtype=torch.float32)
    wg[:, 0] = 64.0
    wu = torch.zeros((N, K), dtype=torch.float32)
    names = sorted(_SIGN_ROWS)
    for n, name in enumerate(names):
        for k, v in _SIGN_ROWS[name].items():
            wu[n, k] = v
    assert torch.equal(wu.to(torch.bfloat16).float(), wu)  # every term is a bf16 value
    wg_d = wg.to(torch.bfloat16).to(dev)
    for engine, layouts in (("valu", [Layout.ROW_VALU, Layout.COL_VALU]),
                            ("mfma", [Layout.ROW_MFMA, Layout.COL_MFMA])):
        for layout in layouts:
            got = {}
            for sign in (1.0, -1.0):
                h = dfk.dfk_gate_up_silu_mul(x, wg_d, (sign * wu).to(torch.bfloat16).to(dev), layout=layout)
                torch.cuda.synchronize()
                u = (h[0].cpu() / 64.0).numpy().astype(np.float32).view(np.uint32)
                got[sign] = u
            for n, name in enumerate(names):
                want = _SIGN_BITS[engine][name]
                assert (int(got[1.0][n]), int(got[-1.0][n])) == want, (layout.name, name, hex(got[1.0][n]),
                                                                         hex(got[-1.0][n]))
            assert np.all(got[1.0][len(names):] == 0) and np.all(got[-1.0][len(names):] == 0)


def test_run_to_run_determinism(dev):
    L = inputs.random_layer(4, 4096, 3000, seed=8500)
    T = to_dev(L, dev)
    for layout in layouts_for("gate_up", 4, 4096):
        a = H.host_bits(gpu_mlp(T, layout))
        b = H.host_bits(gpu_mlp(T, layout))
        h1 = gpu_gate_up(T, layout)
        h2 = gpu_gate_up(T, layout)
        assert np.array_equal(a, b) and np.array_equal(h1, h2), layout.name


@pytest.mark.parametrize("B", [3, 20])
def test_batch_rows_are_independent(dev, orc, B):
    L = inputs.random_layer(B, 1032, 1000, seed=8600 + B)
    T = to_dev(L, dev)
    y = H.host_bf16_as_f64(gpu_mlp(T, Layout.AUTO))
    for b in range(B):
        Tb = dict(T, x=T["x"][b:b + 1].contiguous())
        yb = H.host_bf16_as_f64(gpu_mlp(Tb, Layout.AUTO))
        H.assert_y_close(yb, y[b:b + 1], f"row {b}")


def test_neuron_permutation_invariance(dev):
    B = 5
    L = inputs.random_layer(B, 1032, 1000, seed=8700)
    T = to_dev(L, dev)
    perm = torch.from_numpy(np.random.default_rng(8701).permutation(1000)).to(dev)
    Tp = dict(T, w_gate=T["w_gate"][perm].contiguous(), w_up=T["w_up"][perm].contiguous(),
              w_down=T["w_down"][:, perm].contiguous())
    for layout in layouts_for("gate_up", B, 1032):
        y = H.host_bf16_as_f64(gpu_mlp(T, layout))
        yp = H.host_bf16_as_f64(gpu_mlp(Tp, layout))
        H.assert_y_close(yp, y, layout.name)


def test_side_stream_and_workspace_growth(dev, orc):
    """Calls on a side stream, COL scratch growing from a small to a large shape."""
    s = torch.cuda.Stream(device=dev)
    for (B, dm, dff) in [(1, 64, 48), (16, 4096, 3000), (2, 520, 1000)]:
        L = inputs.random_layer(B, dm, dff, seed=8800 + B)
        T = to_dev(L, dev)
        y_ref, _ = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            y = dfk.dfk_swiglu_mlp(T["x"], T["w_gate"], T["w_up"], T["w_down"], layout=Layout.COL)
        s.synchronize()
        H.assert_y_close(H.host_bf16_as_f64(y), y_ref, f"side stream {B},{dm},{dff}")


# ------------------------------------------------------------ full sizes --

@pytest.fixture(scope="module")
def llama8b(dev):
    L = inputs.llama8b_layer(8)
    return L, to_dev(L, dev)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64])
def test_llama8b_layer(dev, orc, llama8b, B):
    """Every batch row of every variant against the oracle: the full-size
    grids, K splits and batch tiles differ from the small shapes'."""
    L8, T8 = llama8b
    x = inputs.randn_bf16((B, 4096), 1.0, 1100 + B)
    T = dict(T8, x=H.dev_bf16(x, dev))
    y_ref, h_ref = orc.mlp(x, L8.w_gate, L8.w_up, L8.w_down)
    for layout in layouts_for("gate_up", B, 4096):
        H.assert_h_close(gpu_gate_up(T, layout), h_ref, f"8B gate_up B={B} {layout.name}")
        mx, mean = H.assert_y_close(H.host_bf16_as_f64(gpu_mlp(T, layout)), y_ref, f"8B B={B} {layout.name}")
        print(f"8B B={B} {layout.name}: max {mx:.2e} mean {mean:.2e}")


@pytest.fixture(scope="module")
def llama70b(dev):
    L = inputs.llama70b_layer(1)
    return L, to_dev(L, dev)


@pytest.mark.parametrize("B", [1, 4, 16, 32, 64])
def test_llama70b_layer(dev, orc, llama70b, B):
    """Every batch row (all four 16-row batch tiles at B = 64) of every
    variant against the oracle; at B = 64 the oracle is ~45 G fp64
    multiply-adds, a few seconds on the host cores."""
    L7, T7 = llama70b
    x = inputs.randn_bf16((B, 8192), 1.0, 4100 + B)
    T = dict(T7, x=H.dev_bf16(x, dev))
    y_ref, h_ref = orc.mlp(x, L7.w_gate, L7.w_up, L7.w_down)
    for layout in layouts_for("gate_up", B, 8192):
        H.assert_h_close(gpu_gate_up(T, layout), h_ref, f"70B gate_up B={B} {layout.name}")
        y = H.host_bf16_as_f64(gpu_mlp(T, layout))
        mx, mean = H.assert_y_close(y, y_ref, f"70B B={B} {layout.name}")
        print(f"70B B={B} {layout.name}: max {mx:.2e} mean {mean:.2e}")


@pytest.mark.parametrize("s", range(len(inputs.SWEEP_SHAPES)))
def test_shape_sweep_auto(dev, orc, s):
    """Every (d_model, d_ff) x batch of the scheduler sweep, through AUTO,
    every batch row against the oracle."""
    dm, dff = inputs.SWEEP_SHAPES[s]
    base = inputs.sweep_layer(s, 1)
    T0 = to_dev(base, dev)
    for B in inputs.SWEEP_BATCHES:
        x = inputs.randn_bf16((B, dm), 1.0, 5000 + 100 * s + 10 + B)
        y_ref, _ = orc.mlp(x, base.w_gate, base.w_up, base.w_down)
        T = dict(T0, x=H.dev_bf16(x, dev))
        y = H.host_bf16_as_f64(gpu_mlp(T, Layout.AUTO))
        H.assert_y_close(y, y_ref, f"sweep {dm}x{dff} B={B}")


def test_llama8b_32_layer_stack(dev, orc):
    """The chained 32-layer stack, teacher-forced from the oracle: layer l's GPU
    call gets the oracle's x_l (the oracle chain applies the RMS rescale), so
    each layer is compared on identical inputs."""
    x = inputs.stack_x0(1)
    worst = 0.0
    for l in range(32):
        wg, wu, wd = inputs.stack_layer_weights_device(l, dev)
        bits = {k: H.host_bits(t) for k, t in (("w_gate", wg), ("w_up", wu), ("w_down", wd))}
        y_ref, _ = orc.mlp(x, bits["w_gate"], bits["w_up"], bits["w_down"])
        y = dfk.dfk_swiglu_mlp(H.dev_bf16(x, dev), wg, wu, wd)
        torch.cuda.synchronize()
        mx, mean = H.assert_y_close(H.host_bf16_as_f64(y), y_ref, f"stack layer {l}")
        worst = max(worst, mean)
        x = orc.rms_rescale(orc.bf16_rne_array(y_ref), eps=1e-6)
        del wg, wu, wd
    print(f"32-layer stack: worst per-layer normwise mean {worst:.2e}")
