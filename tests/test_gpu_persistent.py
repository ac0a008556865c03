"""GPU parity of the persistent MLP kernel (DFK_LAYOUT_ROW_PERSISTENT).

The persistent kernel runs the vector-ALU gate-up and down row walks in one
cooperative launch with a grid barrier between them.  Each output row is
summed in the same order as in the two-kernel row path (a lane's chunks in
order, then the same DPP reduction), so y must equal dfk_swiglu_mlp with
ROW_VALU bit for bit, and the oracle to the usual normwise bar.  Repeated
launches reuse the barrier state, so every case runs several times in a row
and after other work on the same stream.
"""
import numpy as np
import pytest
import torch

import oracle
import swiglu_mlp_amd as dfk
from swiglu_mlp_amd import Layout, Status, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu

P = Layout.ROW_PERSISTENT


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dfk.lib()  # the HIP library must load: there is no fallback
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def to_dev(L, dev):
    return [H.dev_bf16(a, dev) for a in (L.x, L.w_gate, L.w_up, L.w_down)]


# (B, d_model, d_ff): the tiny workload, ragged chunk and row counts, a single
# 16-byte chunk, every supported batch, the 8B and 70B layer shapes
SHAPES = [(1, 256, 688), (1, 520, 1000), (2, 264, 72), (3, 1032, 200), (4, 136, 264), (1, 8, 8),
          (2, 4104, 264), (4, 600, 1096)]
BIG = [(1, 4096, 14336), (2, 4096, 14336), (1, 8192, 28672)]


def check_shape(dev, orc, shape, L, reps=3):
    x, wg, wu, wd = to_dev(L, dev)
    y_ref, _ = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    want = dfk.dfk_swiglu_mlp(x, wg, wu, wd, layout=Layout.ROW_VALU)
    torch.cuda.synchronize()
    H.assert_y_close(H.host_bf16_as_f64(want), y_ref, f"two-kernel row {shape}")
    for r in range(reps):
        out = torch.full_like(want, float("nan"))
        dfk.dfk_swiglu_mlp(x, wg, wu, wd, out, layout=P)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"persistent {shape} rep {r}"
        # other work on the stream between launches
        dfk.dfk_swiglu_mlp(x, wg, wu, wd, layout=Layout.COL_MFMA)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_%dx%d" % s)
def test_persistent_small(dev, orc, shape):
    B, dm, dff = shape
    L = inputs.tiny_layer() if shape == (1, 256, 688) else inputs.random_layer(B, dm, dff, seed=9900 + B + dm)
    check_shape(dev, orc, shape, L)


@pytest.mark.parametrize("shape", BIG, ids=lambda s: "B%d_%dx%d" % s)
def test_persistent_layer_shapes(dev, orc, shape):
    B, dm, dff = shape
    L = inputs.llama8b_layer(B) if dm == 4096 else inputs.llama70b_layer(B)
    check_shape(dev, orc, shape, L, reps=2)


def test_persistent_unsupported(dev):
    def mk(B, dm, dff):
        return [torch.zeros(s, dtype=torch.bfloat16, device=dev)
                for s in ((B, dm), (dff, dm), (dff, dm), (dm, dff))]

    for B, dm, dff in ((5, 64, 48), (3, 4096, 14336), (2, 64, 32776)):  # batch, then h beyond LDS
        x, wg, wu, wd = mk(B, dm, dff)
        with pytest.raises(dfk.DfkError) as e:
            dfk.dfk_swiglu_mlp(x, wg, wu, wd, layout=P)
        assert e.value.status == Status.UNSUPPORTED, (B, dm, dff)
    x, wg, wu, wd = mk(1, 64, 48)
    with pytest.raises(dfk.DfkError) as e:
        dfk.dfk_gate_up_silu_mul(x, wg, wu, layout=P)
    assert e.value.status == Status.UNSUPPORTED
    with pytest.raises(dfk.DfkError) as e:
        dfk.dfk_down_proj(torch.zeros((1, 48), dtype=torch.float32, device=dev), wd, layout=P)
    assert e.value.status == Status.UNSUPPORTED
    g = torch.ones(64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(dfk.DfkError) as e:
        dfk.dfk_rmsnorm_swiglu_mlp(x, g, 1e-5, wg, wu, wd, layout=P)
    assert e.value.status == Status.UNSUPPORTED


def test_persistent_refused_under_capture(dev, orc):
    """A stream being captured gets DFK_ERR_UNSUPPORTED (nothing enqueued);
    the captured two-kernel call still replays correctly."""
    L = inputs.random_layer(1, 520, 1000, seed=9950)
    x, wg, wu, wd = to_dev(L, dev)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):  # creates the stream's workspace (no allocation under capture)
        want = dfk.dfk_swiglu_mlp(x, wg, wu, wd, layout=Layout.ROW_VALU)
    s.synchronize()
    out = torch.empty_like(want)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    refused = None
    with torch.cuda.graph(graph, stream=s):
        try:
            dfk.dfk_swiglu_mlp(x, wg, wu, wd, out, layout=P)
        except dfk.DfkError as e:
            refused = e.status
        dfk.dfk_swiglu_mlp(x, wg, wu, wd, out, layout=Layout.ROW_VALU)
    assert refused == Status.UNSUPPORTED
    for _ in range(2):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16))
