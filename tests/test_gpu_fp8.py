"""GPU parity of the weight-only FP8 entry points (dfk_*_fp8) against the
fp64 oracle over the dequantized weights W = s[row] * e4m3(q).

- Every code and its byte position: one-hot h (or x) picks out one column of
  the codes, so y is s * e4m3(q) itself, exact in bf16 for power-of-two
  scales (bit for bit against the oracle), and h is SiLU(1) * that value.
- Ragged shapes (chunk counts not a multiple of 64, a single chunk, h past the
  LDS limit, so K panels), batches 1 to 128 on the vector-ALU (B <= 8) and
  matrix-core variants, the Llama-3-8B layer shape: h within 1e-4 and y
  within the usual normwise bars of the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import swiglu_mlp_amd as dfk
from swiglu_mlp_amd import Layout, Status, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu

LAYOUTS = [Layout.AUTO, Layout.ROW, Layout.COL, Layout.ROW_VALU, Layout.ROW_MFMA, Layout.COL_MFMA]


def layouts_for(B):
    return [l for l in LAYOUTS if B <= 8 or l != Layout.ROW_VALU]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dfk.lib()  # the HIP library must load: there is no fallback
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def code_matrix(rows, cols, shift=0):
    """Row r, column c holds code (r + c + shift) % 256; NaN codes become 0."""
    q = ((np.arange(rows)[:, None] + np.arange(cols)[None, :] + shift) % 256).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0
    return q


@pytest.mark.parametrize("B", [1, 2, 3, 4, 6, 8, 20])
@pytest.mark.parametrize("layout", [Layout.ROW_VALU, Layout.COL_VALU, Layout.ROW_MFMA, Layout.COL_MFMA])
def test_every_code_through_down(dev, orc, B, layout):
    if layout == Layout.ROW_VALU and B > 8:
        pytest.skip("the vector-ALU FP8 row walk takes B <= 8")
    if layout == Layout.COL_VALU and B > 4:
        pytest.skip("the FP8 down column walk (h in registers) takes B <= 4")
    M = K = 256
    q = code_matrix(M, K)
    s = np.array([2.0 ** -(m % 4) for m in range(M)], dtype=np.float32)
    for k0 in (0, 1, 2, 3, 5, 8, 13, 15, 16, 17, 255):
        h = np.zeros((B, K), dtype=np.float32)
        for b in range(B):
            h[b, (k0 + 7 * b) % K] = 1.0
        want = orc.bf16_rne_array(orc.down_fp8(h.astype(np.float64), q, s))
        y = dfk.dfk_down_proj_fp8(to_dev(h, dev), to_dev(q, dev), to_dev(s, dev), layout=layout)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(H.host_bits(y), want, err_msg=f"k0={k0}")


@pytest.mark.parametrize("layout", [Layout.ROW_VALU, Layout.ROW_MFMA, Layout.COL_MFMA])
def test_every_code_through_gate_up(dev, orc, layout):
    N = K = 256
    qu = code_matrix(N, K, shift=3)
    qg = np.full((N, K), 0x38, dtype=np.uint8)  # every gate weight 1.0
    sg = np.ones(N, dtype=np.float32)
    su = np.array([2.0 ** -(n % 3) for n in range(N)], dtype=np.float32)
    for k0 in (0, 1, 4, 9, 15, 16, 100, 255):
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k0] = 1.0
        xb = inputs.to_bf16_bits(torch.from_numpy(x))
        want = orc.gate_up_fp8(xb, qg, sg, qu, su)
        h = dfk.dfk_gate_up_silu_mul_fp8(H.dev_bf16(xb, dev), to_dev(qg, dev), to_dev(sg, dev), to_dev(qu, dev),
                                         to_dev(su, dev), layout=layout)
        torch.cuda.synchronize()
        got = h.double().cpu().numpy()
        np.testing.assert_allclose(got, want, rtol=5e-7, atol=0, err_msg=f"k0={k0}")


# (B, d_model, d_ff): the tiny workload's shape, ragged 16-byte chunk counts,
# a single chunk, every batch, h beyond the LDS limit at B = 4
SHAPES = [(1, 256, 688), (1, 528, 1008), (2, 272, 80), (3, 1040, 208), (4, 144, 272), (2, 16, 16),
          (4, 4112, 272), (4, 64, 8208), (1, 2064, 4112), (5, 528, 1008), (6, 272, 4112), (7, 1040, 208),
          (8, 144, 8208), (8, 16, 16), (16, 528, 1008), (17, 272, 464), (40, 1040, 208), (64, 144, 272),
          (128, 64, 48)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_%dx%d" % s)
def test_fp8_small_shapes(dev, orc, shape):
    B, dm, dff = shape
    L = inputs.fp8_layer(B, dm, dff, seed=9400 + B + dm, std=0.05)
    d = {k: (H.dev_bf16(v, dev) if k == "x" else to_dev(v, dev)) for k, v in L.items()}
    y_ref, h_ref = orc.mlp_fp8(L["x"], L["q_gate"], L["s_gate"], L["q_up"], L["s_up"], L["q_down"], L["s_down"])
    h_in = inputs.h_like(B, dff, seed=9450 + B)
    yd_ref = orc.down_fp8(h_in.astype(np.float64), L["q_down"], L["s_down"])
    for layout in layouts_for(B):
        what = f"{layout.name} {shape}"
        h = dfk.dfk_gate_up_silu_mul_fp8(d["x"], d["q_gate"], d["s_gate"], d["q_up"], d["s_up"], layout=layout)
        y = dfk.dfk_swiglu_mlp_fp8(d["x"], d["q_gate"], d["s_gate"], d["q_up"], d["s_up"], d["q_down"],
                                   d["s_down"], layout=layout)
        yd = dfk.dfk_down_proj_fp8(H.dev_f32(h_in, dev), d["q_down"], d["s_down"], layout=layout)
        torch.cuda.synchronize()
        H.assert_h_close(h.double().cpu().numpy(), h_ref, f"gate_up_fp8 {what}")
        H.assert_y_close(H.host_bf16_as_f64(y), y_ref, f"mlp_fp8 {what}")
        H.assert_y_close(H.host_bf16_as_f64(yd), yd_ref, f"down_fp8 {what}")
    if B <= 4:
        # the down column walk with h held in registers (fits every shape here)
        yd = dfk.dfk_down_proj_fp8(H.dev_f32(h_in, dev), d["q_down"], d["s_down"], layout=Layout.COL_VALU)
        torch.cuda.synchronize()
        H.assert_y_close(H.host_bf16_as_f64(yd), yd_ref, f"down_fp8 COL_VALU {shape}")


# FP8 down column walk with h in registers where every workgroup walks several
# row groups (odd and even counts, one or two rows per group, 8- and 16-wave
# workgroups), and the Llama-3-8B down shape: against the oracle, and integer
# codes with power-of-two scales bit for bit.
DOWN_HREG_F8_SHAPES = [(1, 4096, 14336), (2, 4096, 14336), (3, 4096, 14336), (4, 4096, 14336),
                       (2, 8192, 4096), (3, 6144, 3008), (4, 2048, 9008)]


@pytest.mark.parametrize("shape", DOWN_HREG_F8_SHAPES, ids=lambda s: "B%d_%dx%d" % s)
def test_fp8_down_h_in_registers(dev, orc, shape):
    B, dm, dff = shape
    rng = np.random.default_rng(9600 + B + dm)
    q = rng.integers(0, 256, size=(dm, dff), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0  # no NaN codes
    s = (2.0 ** rng.integers(-3, 1, size=dm)).astype(np.float32)
    qd, sd = to_dev(q, dev), to_dev(s, dev)
    h_in = inputs.h_like(B, dff, seed=9650 + B)
    want = orc.down_fp8(h_in.astype(np.float64), q, s)
    y = dfk.dfk_down_proj_fp8(H.dev_f32(h_in, dev), qd, sd, layout=Layout.COL_VALU)
    torch.cuda.synchronize()
    H.assert_y_close(H.host_bf16_as_f64(y), want, f"down_fp8 COL_VALU {shape}")
    # small integer h and codes of small integers (|e4m3| <= 4): every sum exact
    qi = rng.choice(np.array([0x00, 0x38, 0xB8, 0x40, 0xC0, 0x48, 0xC8], dtype=np.uint8), size=(dm, dff))
    hi = inputs.integer_h(B, dff, seed=9680 + B, bound=64)
    got = dfk.dfk_down_proj_fp8(H.dev_f32(hi, dev), to_dev(qi, dev), sd, layout=Layout.COL_VALU)
    torch.cuda.synchronize()
    exact = orc.bf16_rne_array(orc.down_fp8(hi.astype(np.float64), qi, s))
    np.testing.assert_array_equal(H.host_bits(got), exact, err_msg=f"integer {shape}")


def _hreg_f8_fits(B, d_ff):
    """Whether the FP8 down column walk takes the shape: some workgroup width
    (8, 16 or 4 waves) leaves a lane J <= 8 chunks of h with J * 16 * B <= 64
    registers (16 waves only up to J = 4)."""
    if B > 4:
        return False
    c16 = d_ff // 16
    for w in (8, 16, 4):
        J = -(-(-(-c16 // w)) // 64)
        if J <= 8 and J * 16 * B <= 64 and (w <= 8 or J <= 4):
            return True
    return False


# Seeded random shapes (multiples of 16 up to 3072, B up to 128): every FP8
# variant, and the down column walk wherever it takes the shape (else it must
# refuse it), against the oracle.
def _random_fp8_shapes(n=16, seed=20261205):
    rng = np.random.default_rng(seed)
    return [(int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 17, 40, 64, 128])), 16 * int(rng.integers(1, 193)),
             16 * int(rng.integers(1, 193))) for _ in range(n)]


@pytest.mark.parametrize("shape", _random_fp8_shapes(), ids=lambda s: "B%d_%dx%d" % s)
def test_fp8_random_shapes(dev, orc, shape):
    B, dm, dff = shape
    L = inputs.fp8_layer(B, dm, dff, seed=9700 + B + dm, std=0.05)
    d = {k: (H.dev_bf16(v, dev) if k == "x" else to_dev(v, dev)) for k, v in L.items()}
    y_ref, h_ref = orc.mlp_fp8(L["x"], L["q_gate"], L["s_gate"], L["q_up"], L["s_up"], L["q_down"], L["s_down"])
    h_in = inputs.h_like(B, dff, seed=9750 + B)
    yd_ref = orc.down_fp8(h_in.astype(np.float64), L["q_down"], L["s_down"])
    for layout in layouts_for(B):
        what = f"{layout.name} {shape}"
        h = dfk.dfk_gate_up_silu_mul_fp8(d["x"], d["q_gate"], d["s_gate"], d["q_up"], d["s_up"], layout=layout)
        y = dfk.dfk_swiglu_mlp_fp8(d["x"], d["q_gate"], d["s_gate"], d["q_up"], d["s_up"], d["q_down"],
                                   d["s_down"], layout=layout)
        yd = dfk.dfk_down_proj_fp8(H.dev_f32(h_in, dev), d["q_down"], d["s_down"], layout=layout)
        torch.cuda.synchronize()
        H.assert_h_close(h.double().cpu().numpy(), h_ref, f"gate_up_fp8 {what}")
        H.assert_y_close(H.host_bf16_as_f64(y), y_ref, f"mlp_fp8 {what}")
        H.assert_y_close(H.host_bf16_as_f64(yd), yd_ref, f"down_fp8 {what}")
    if _hreg_f8_fits(B, dff):
        yd = dfk.dfk_down_proj_fp8(H.dev_f32(h_in, dev), d["q_down"], d["s_down"], layout=Layout.COL_VALU)
        torch.cuda.synchronize()
        H.assert_y_close(H.host_bf16_as_f64(yd), yd_ref, f"down_fp8 COL_VALU {shape}")
    else:
        with pytest.raises(dfk.DfkError) as e:
            dfk.dfk_down_proj_fp8(H.dev_f32(h_in, dev), d["q_down"], d["s_down"], layout=Layout.COL_VALU)
        assert e.value.status == Status.UNSUPPORTED, shape


# FP8 gate-up row traversal at one batch tile with many row tiles (at least
# five per CU on a 256-CU device: the staged-x kernel with 128-element K
# blocks), ragged K blocks and a partial batch tile, against the oracle.
MANY_ROWS_F8_SHAPES = [(1, 272, 28688), (5, 1040, 28688), (16, 528, 20496)]


@pytest.mark.parametrize("shape", MANY_ROWS_F8_SHAPES, ids=lambda s: "B%d_%dx%d" % s)
def test_fp8_gate_up_one_tile_many_rows(dev, orc, shape):
    B, dm, dff = shape
    L = inputs.fp8_layer(B, dm, dff, seed=9800 + B + dm, std=0.05)
    d = {k: (H.dev_bf16(v, dev) if k == "x" else to_dev(v, dev)) for k, v in L.items()}
    _, h_ref = orc.mlp_fp8(L["x"], L["q_gate"], L["s_gate"], L["q_up"], L["s_up"], L["q_down"], L["s_down"])
    for layout in (Layout.ROW_MFMA, Layout.COL_MFMA, Layout.AUTO):
        h = dfk.dfk_gate_up_silu_mul_fp8(d["x"], d["q_gate"], d["s_gate"], d["q_up"], d["s_up"], layout=layout)
        torch.cuda.synchronize()
        H.assert_h_close(h.double().cpu().numpy(), h_ref, f"gate_up_fp8 {layout.name} {shape}")


@pytest.mark.parametrize("B", [1, 2, 3, 4, 8, 16, 64])
def test_fp8_llama8b_shape(dev, orc, B):
    L = inputs.fp8_layer(B, 4096, 14336, seed=9300, std=0.02)
    d = {k: (H.dev_bf16(v, dev) if k == "x" else to_dev(v, dev)) for k, v in L.items()}
    y_ref, h_ref = orc.mlp_fp8(L["x"], L["q_gate"], L["s_gate"], L["q_up"], L["s_up"], L["q_down"], L["s_down"])
    y = dfk.dfk_swiglu_mlp_fp8(d["x"], d["q_gate"], d["s_gate"], d["q_up"], d["s_up"], d["q_down"], d["s_down"])
    h = dfk.dfk_gate_up_silu_mul_fp8(d["x"], d["q_gate"], d["s_gate"], d["q_up"], d["s_up"])
    torch.cuda.synchronize()
    H.assert_h_close(h.double().cpu().numpy(), h_ref, f"gate_up_fp8 8B B={B}")
    H.assert_y_close(H.host_bf16_as_f64(y), y_ref, f"mlp_fp8 8B B={B}")


def test_fp8_unsupported(dev):
    def mk(B, dm, dff):
        L = inputs.fp8_layer(B, dm, dff, seed=1, std=0.1)
        return {k: (H.dev_bf16(v, dev) if k == "x" else to_dev(v, dev)) for k, v in L.items()}

    cases = [(mk(129, 64, 48), Layout.AUTO), (mk(9, 64, 48), Layout.ROW_VALU), (mk(1, 72, 48), Layout.AUTO),
             (mk(1, 64, 40), Layout.AUTO)]
    cases += [(mk(1, 64, 48), l) for l in (Layout.COL_VALU, Layout.ROW_PERSISTENT)]
    # the down column walk takes B <= 4
    d5 = mk(5, 64, 48)
    with pytest.raises(dfk.DfkError) as e:
        dfk.dfk_down_proj_fp8(torch.zeros((5, 48), dtype=torch.float32, device=dev), d5["q_down"], d5["s_down"],
                              layout=Layout.COL_VALU)
    assert e.value.status == Status.UNSUPPORTED
    for d, layout in cases:
        with pytest.raises(dfk.DfkError) as e:
            dfk.dfk_swiglu_mlp_fp8(d["x"], d["q_gate"], d["s_gate"], d["q_up"], d["s_up"], d["q_down"],
                                   d["s_down"], layout=layout)
        assert e.value.status == Status.UNSUPPORTED, (tuple(d["x"].shape), layout)
