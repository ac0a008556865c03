"""GPU parity of the RMS normalization ahead of gate-up, through the C ABI.

dfk_rmsnorm must equal the oracle bit for bit: both sides sum squares in fp64
and round (x * inv) * gain from fp64 to bf16 once, so they can differ only
where that fp64 value lies within a few fp64 ulps of a bf16 rounding boundary
(about 2^-44 of random cases; none of the seeded cases here).  The fused
entry points must equal dfk_rmsnorm followed by the plain entry point with the
same variant bit for bit (the fused kernels normalize in the same order), and
the oracle chain rmsnorm -> gate_up (-> down) to the usual normwise bars.
"""
import numpy as np
import pytest
import torch

import oracle
import swiglu_mlp_amd as dfk
from swiglu_mlp_amd import Layout, Status, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu

ALL_LAYOUTS = [Layout.ROW_VALU, Layout.COL_VALU, Layout.ROW_MFMA, Layout.COL_MFMA, Layout.ROW, Layout.COL,
               Layout.AUTO]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dfk.lib()  # the HIP library must load: there is no fallback
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def layouts_for(B, d_model):
    valu = B <= 8 and B * d_model * 2 + B * 64 <= 160 * 1024
    return [l for l in ALL_LAYOUTS if valu or l not in (Layout.ROW_VALU, Layout.COL_VALU)]


def gpu_rmsnorm(x, gain, eps, dev):
    out = dfk.dfk_rmsnorm(H.dev_bf16(x, dev), H.dev_bf16(gain, dev), eps)
    torch.cuda.synchronize()
    return H.host_bits(out)


# (B, d_model, x std, eps): one chunk, ragged chunk counts, the layer widths,
# the largest batch, activations far from unit scale
NORM_CASES = [
    (1, 8, 1.0, 1e-5), (1, 4096, 1.0, 1e-5), (3, 520, 1.0, 1e-6), (8, 1032, 30.0, 1e-5),
    (64, 136, 1e-3, 1e-5), (256, 64, 1.0, 1e-6), (2, 8192, 1.0, 1e-5), (5, 16392, 0.2, 1e-5),
]


@pytest.mark.parametrize("case", NORM_CASES, ids=lambda c: "B%d_d%d_s%g_e%g" % c)
def test_rmsnorm_bitwise(dev, orc, case):
    B, dm, std, eps = case
    x = inputs.randn_bf16((B, dm), std, seed=9000 + B + dm)
    gain = inputs.norm_gain(dm, seed=9100 + dm)
    got = gpu_rmsnorm(x, gain, eps, dev)
    want = orc.rmsnorm(x, gain, eps)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{bad.shape[0]} mismatches, first at {bad[0]}: {got[tuple(bad[0])]:#06x} vs " \
                          f"{want[tuple(bad[0])]:#06x}"


def _bits_of(values):
    return inputs.to_bf16_bits(torch.tensor(values, dtype=torch.float32))


def test_rmsnorm_degenerate_rows(dev, orc):
    """Zero rows, one nonzero element, values whose squares overflow fp32,
    bf16 subnormal inputs and outputs, gains with zeros and negatives, and
    exact rounding ties."""
    dm = 64
    rows = np.zeros((7, dm), dtype=np.float32)
    rows[1, 17] = -3.0                                     # one nonzero: xn = -gain * dm^0.5 (eps aside)
    rows[2, :] = 1.0e30                                    # x^2 overflows fp32, not fp64
    rows[2, ::3] = -2.5e30
    rows[3, :] = 1.0e-39                                   # bf16 subnormals
    rows[3, 1::2] = -3.0e-39
    rows[4, :] = np.linspace(-4.0, 4.0, dm)
    rows[5, :] = 0.5                                       # all equal: xn = gain / sqrt(0.25 + eps)
    # mean square exactly 1 (16 x 1.5^2 + 28 x 1^2 = 64): with eps = 0, inv = 1
    # and 1.5 * (1 + 2^-7) = 1.51171875 lies exactly halfway between two bf16
    # values (ties to even: 0x3FC2)
    ties = np.arange(0, 64, 4)
    rows[6, ties] = 1.5
    rows[6, ties[::2]] = -1.5
    rest = np.setdiff1d(np.arange(dm), ties)[:28]
    rows[6, rest] = 1.0
    rows[6, rest[1::3]] = -1.0
    x = inputs.to_bf16_bits(torch.from_numpy(rows))
    g = np.ones(dm, dtype=np.float32)
    g[::5] = 0.0
    g[1::7] = -1.75
    g[2::11] = 3.0e-38
    g[ties] = 1.0078125
    gain = _bits_of(g)
    for eps in (1e-5, 1.0, 0.0):
        if eps == 0.0:
            xe, ge = x[1:], gain  # eps = 0 with a zero row gives NaN on both sides; leave it out
        else:
            xe, ge = x, gain
        got = gpu_rmsnorm(xe, ge, eps, dev)
        want = orc.rmsnorm(xe, ge, eps)
        np.testing.assert_array_equal(got, want, err_msg=f"eps={eps}")
    # the zero row normalizes to zeros (of the gain's sign)
    z = gpu_rmsnorm(x[:1], gain, 1e-5, dev)[0]
    assert np.all((z & 0x7FFF) == 0)
    # the ties round to even
    t6 = gpu_rmsnorm(x[6:7], gain, 0.0, dev)[0]
    assert set(t6[ties[1::2]].tolist()) == {0x3FC2} and set(t6[ties[::2]].tolist()) == {0xBFC2}


def test_rmsnorm_rejects_bad_eps(dev):
    x = H.dev_bf16(inputs.randn_bf16((1, 64), 1.0, seed=1), dev)
    g = H.dev_bf16(inputs.norm_gain(64, seed=2), dev)
    for eps in (-1.0, float("nan"), float("inf")):
        with pytest.raises(dfk.DfkError) as e:
            dfk.dfk_rmsnorm(x, g, eps)
        assert e.value.status == Status.INVALID_ARG


NG_SHAPES = [(1, 256, 688), (1, 520, 1000), (3, 1032, 200), (8, 520, 1000), (13, 128, 136), (17, 264, 456),
             (64, 136, 264), (2, 4104, 264), (5, 600, 1096)]


@pytest.mark.parametrize("shape", NG_SHAPES, ids=lambda s: "B%d_%dx%d" % s)
def test_rmsnorm_gate_up_and_mlp_all_variants(dev, orc, shape):
    B, dm, dff = shape
    eps = 1e-5
    L = inputs.random_layer(B, dm, dff, seed=9500 + B + dm)
    gain = inputs.norm_gain(dm, seed=9600 + dm)
    xn = orc.rmsnorm(L.x, gain, eps)
    _, _, h_ref = orc.gate_up(xn, L.w_gate, L.w_up)
    y_ref, _ = orc.mlp(xn, L.w_gate, L.w_up, L.w_down)
    x_d, g_d = H.dev_bf16(L.x, dev), H.dev_bf16(gain, dev)
    wg, wu, wd = H.dev_bf16(L.w_gate, dev), H.dev_bf16(L.w_up, dev), H.dev_bf16(L.w_down, dev)
    for layout in layouts_for(B, dm):
        what = f"{layout.name} {shape}"
        h = dfk.dfk_rmsnorm_gate_up_silu_mul(x_d, g_d, eps, wg, wu, layout=layout)
        xn_d = dfk.dfk_rmsnorm(x_d, g_d, eps)
        h2 = dfk.dfk_gate_up_silu_mul(xn_d, wg, wu, layout=layout)
        y = dfk.dfk_rmsnorm_swiglu_mlp(x_d, g_d, eps, wg, wu, wd, layout=layout)
        y2 = dfk.dfk_swiglu_mlp(xn_d, wg, wu, wd, layout=layout)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(H.host_bits(xn_d), xn, err_msg=f"rmsnorm {what}")
        assert torch.equal(h.view(torch.int32), h2.view(torch.int32)), f"fused vs composed h {what}"
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), f"fused vs composed y {what}"
        H.assert_h_close(h.double().cpu().numpy(), h_ref, f"rmsnorm gate_up {what}")
        H.assert_y_close(H.host_bf16_as_f64(y), y_ref, f"rmsnorm mlp {what}")


@pytest.mark.parametrize("B", [1, 4, 8, 16])
def test_rmsnorm_mlp_llama8b_shape(dev, orc, B):
    """The 8B layer shape in the scheduler's configuration (AUTO)."""
    eps = 1e-5
    L = inputs.llama8b_layer(B)
    gain = inputs.norm_gain(L.d_model, seed=9700)
    xn = orc.rmsnorm(L.x, gain, eps)
    y_ref, h_ref = orc.mlp(xn, L.w_gate, L.w_up, L.w_down)
    x_d, g_d = H.dev_bf16(L.x, dev), H.dev_bf16(gain, dev)
    wg, wu, wd = H.dev_bf16(L.w_gate, dev), H.dev_bf16(L.w_up, dev), H.dev_bf16(L.w_down, dev)
    h = dfk.dfk_rmsnorm_gate_up_silu_mul(x_d, g_d, eps, wg, wu)
    y = dfk.dfk_rmsnorm_swiglu_mlp(x_d, g_d, eps, wg, wu, wd)
    torch.cuda.synchronize()
    H.assert_h_close(h.double().cpu().numpy(), h_ref, f"rmsnorm gate_up 8B B={B}")
    H.assert_y_close(H.host_bf16_as_f64(y), y_ref, f"rmsnorm mlp 8B B={B}")
