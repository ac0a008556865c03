"""GPU parity of the packed gate/up weight layouts (dfk_*_packed).

Packing moves only the weights' addresses: each output is summed in the same
order as with separate W_gate / W_up, so h and y must equal the unpacked
entry points bit for bit, for every variant, and the oracle to the usual
normwise bars.
"""
import pytest
import torch

import oracle
import swiglu_mlp_amd as dfk
from swiglu_mlp_amd import Layout, Packing, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu

LAYOUTS = [Layout.ROW_VALU, Layout.COL_VALU, Layout.ROW_MFMA, Layout.COL_MFMA, Layout.ROW, Layout.COL,
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
    valu = B <= 8 and B * d_model * 2 <= 160 * 1024
    return [l for l in LAYOUTS if valu or l not in (Layout.ROW_VALU, Layout.COL_VALU)]


# ragged chunk and row counts, every engine's batch range, staged and
# K-panel kernels (B 17, 40), the tiny workload
SHAPES = [(1, 256, 688), (1, 520, 1000), (3, 1032, 200), (5, 600, 1096), (8, 136, 264), (16, 1032, 2056),
          (17, 264, 456), (40, 520, 1000)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_%dx%d" % s)
def test_packed_equals_separate(dev, orc, shape):
    B, dm, dff = shape
    L = inputs.tiny_layer() if shape == (1, 256, 688) else inputs.random_layer(B, dm, dff, seed=9800 + B + dm)
    x, wg, wu, wd = (H.dev_bf16(a, dev) for a in (L.x, L.w_gate, L.w_up, L.w_down))
    _, _, h_ref = orc.gate_up(L.x, L.w_gate, L.w_up)
    y_ref, _ = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    packed = {p: dfk.pack_gate_up(wg, wu, p) for p in Packing}
    for layout in layouts_for(B, dm):
        h = dfk.dfk_gate_up_silu_mul(x, wg, wu, layout=layout)
        y = dfk.dfk_swiglu_mlp(x, wg, wu, wd, layout=layout)
        for p, wgu in packed.items():
            what = f"{p.name} {layout.name} {shape}"
            hp = dfk.dfk_gate_up_silu_mul_packed(x, wgu, p, layout=layout)
            yp = dfk.dfk_swiglu_mlp_packed(x, wgu, wd, p, layout=layout)
            torch.cuda.synchronize()
            assert torch.equal(hp.view(torch.int32), h.view(torch.int32)), f"h {what}"
            assert torch.equal(yp.view(torch.int16), y.view(torch.int16)), f"y {what}"
            H.assert_h_close(hp.double().cpu().numpy(), h_ref, f"h vs oracle {what}")
            H.assert_y_close(H.host_bf16_as_f64(yp), y_ref, f"y vs oracle {what}")


@pytest.mark.parametrize("B", [1, 4, 8])
def test_packed_llama8b_shape(dev, orc, B):
    L = inputs.llama8b_layer(B)
    x, wg, wu, wd = (H.dev_bf16(a, dev) for a in (L.x, L.w_gate, L.w_up, L.w_down))
    y_ref, _ = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    y = dfk.dfk_swiglu_mlp(x, wg, wu, wd)
    for p in Packing:
        yp = dfk.dfk_swiglu_mlp_packed(x, dfk.pack_gate_up(wg, wu, p), wd, p)
        torch.cuda.synchronize()
        assert torch.equal(yp.view(torch.int16), y.view(torch.int16)), p.name
        H.assert_y_close(H.host_bf16_as_f64(yp), y_ref, f"8B B={B} {p.name}")


def test_packed_persistent(dev):
    L = inputs.random_layer(1, 520, 1000, seed=9850)
    x, wg, wu, wd = (H.dev_bf16(a, dev) for a in (L.x, L.w_gate, L.w_up, L.w_down))
    y = dfk.dfk_swiglu_mlp(x, wg, wu, wd, layout=Layout.ROW_VALU)
    yp = dfk.dfk_swiglu_mlp_packed(x, dfk.pack_gate_up(wg, wu, Packing.BLOCKED), wd, Packing.BLOCKED,
                                   layout=Layout.ROW_PERSISTENT)
    torch.cuda.synchronize()
    assert torch.equal(yp.view(torch.int16), y.view(torch.int16))
    with pytest.raises(dfk.DfkError) as e:
        dfk.dfk_swiglu_mlp_packed(x, dfk.pack_gate_up(wg, wu, Packing.INTERLEAVED), wd, Packing.INTERLEAVED,
                                  layout=Layout.ROW_PERSISTENT)
    assert e.value.status == dfk.Status.UNSUPPORTED
