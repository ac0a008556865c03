"""Chained MLP calls captured into one HIP graph: the launch-gap removal path
for stacked layers.  Once a stream's workspace exists the library's calls do
no allocation and no synchronisation, so they capture.  Every replay, with
eager work and synchronisations between replays, must reproduce the eager
chain bit for bit (the kernels are deterministic) and match the fp64 oracle
on seeded inputs.  The library's workspace may grow after a capture (a later
eager call of a larger shape on the same stream): the graph keeps the buffer
it captured, which growth never frees, so its replays stay correct."""
import numpy as np
import pytest
import torch

import oracle
import swiglu_mlp_amd as dfk
from swiglu_mlp_amd import Layout, Status, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def _layers(L, dm, dff, seed, dev):
    return [(inputs.randn_bf16_device((dff, dm), 0.02, seed + 10 * l + 1, dev),
             inputs.randn_bf16_device((dff, dm), 0.02, seed + 10 * l + 2, dev),
             inputs.randn_bf16_device((dm, dff), 0.02, seed + 10 * l + 3, dev)) for l in range(L)]


def _oracle_y(orc, x, w):
    """The oracle's y for bf16 device tensors x and w = (W_gate, W_up, W_down)."""
    y, _ = orc.mlp(H.host_bits(x), *(H.host_bits(t) for t in w))
    return y


CASES = [
    (1, 4096, 14336, 4, Layout.AUTO),      # the 8B layer shape, the scheduler's variants
    (16, 1032, 2056, 3, Layout.COL_MFMA),  # down through K panels + the reduce kernel
    (40, 520, 1000, 3, Layout.AUTO),       # staged kernels, K split + reduce
    (5, 600, 1096, 3, Layout.ROW_MFMA),    # LDS-transposed gate-up, cooperative down
]


@pytest.mark.parametrize("B,dm,dff,L,layout", CASES)
def test_graph_replays_match_eager(B, dm, dff, L, layout):
    dev = torch.device("cuda:0")
    layers = _layers(L, dm, dff, 8000 + B, dev)
    x0 = inputs.randn_bf16_device((B, dm), 1.0, 8500 + B, dev)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    # eager chain on s (this also creates the library's workspace for s)
    with torch.cuda.stream(s):
        ref, cur = [], x0
        for w in layers:
            cur = dfk.dfk_swiglu_mlp(cur, *w, layout=layout)
            ref.append(cur)
    s.synchronize()
    x_in = x0.clone()
    outs = [torch.empty((B, dm), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    junk_out = torch.empty((B, dm), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        cur = x_in
        for w, o in zip(layers, outs):
            dfk.dfk_swiglu_mlp(cur, *w, out=o, layout=layout)
            cur = o
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        # eager library work on the same stream between replays
        with torch.cuda.stream(s):
            dfk.dfk_swiglu_mlp(x0, *layers[-1], out=junk_out, layout=layout)
        s.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(outs[l], ref[l]), f"replay {r}, layer {l}"


@pytest.mark.parametrize("B,dm,dff,L,layout", CASES)
def test_graph_replays_match_oracle(orc, B, dm, dff, L, layout):
    """L calls on seeded inputs (one input buffer per layer) captured into one
    graph: every replay of every layer against the fp64 oracle."""
    dev = torch.device("cuda:0")
    layers = _layers(L, dm, dff, 8100 + B, dev)
    xs = [inputs.randn_bf16_device((B, dm), 1.0, 8600 + 10 * B + l, dev) for l in range(L)]
    want = [_oracle_y(orc, x, w) for x, w in zip(xs, layers)]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):  # creates the stream's workspace
        for x, w in zip(xs, layers):
            dfk.dfk_swiglu_mlp(x, *w, layout=layout)
    s.synchronize()
    outs = [torch.empty((B, dm), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for x, w, o in zip(xs, layers, outs):
            dfk.dfk_swiglu_mlp(x, *w, out=o, layout=layout)
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        with torch.cuda.stream(s):
            dfk.dfk_swiglu_mlp(xs[0], *layers[0], layout=layout)
        s.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            H.assert_y_close(H.host_bf16_as_f64(outs[l]), want[l], f"replay {r} layer {l} {layout.name}")


def test_graph_survives_workspace_growth(orc):
    """Capture the Llama-3-8B layer at B = 1, then grow the same stream's
    workspace with an eager Llama-3-70B B = 64 call: the graph still holds the
    buffer it captured (retired, not freed), so its replay matches the oracle
    and the eager result bit for bit.  The 70B call itself is checked too."""
    dev = torch.device("cuda:0")
    w8 = _layers(1, 4096, 14336, 8200, dev)[0]
    x8 = inputs.randn_bf16_device((1, 4096), 1.0, 8210, dev)
    want8 = _oracle_y(orc, x8, w8)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        eager8 = dfk.dfk_swiglu_mlp(x8, *w8)
    s.synchronize()
    H.assert_y_close(H.host_bf16_as_f64(eager8), want8, "8B B=1 eager")
    out8 = torch.empty_like(eager8)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dfk.dfk_swiglu_mlp(x8, *w8, out=out8)
    w70 = _layers(1, 8192, 28672, 8300, dev)[0]
    x70 = inputs.randn_bf16_device((64, 8192), 1.0, 8310, dev)
    with torch.cuda.stream(s):
        y70 = dfk.dfk_swiglu_mlp(x70, *w70)  # needs a larger workspace: it grows
    s.synchronize()
    for r in range(3):
        out8.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        with torch.cuda.stream(s):  # the grown workspace in use on the stream too
            dfk.dfk_swiglu_mlp(x70, *w70, out=y70)
        torch.cuda.synchronize()
        assert torch.equal(out8.view(torch.int16), eager8.view(torch.int16)), f"replay {r}"
        H.assert_y_close(H.host_bf16_as_f64(out8), want8, f"8B B=1 replay {r} after growth")
    H.assert_y_close(H.host_bf16_as_f64(y70), _oracle_y(orc, x70, w70), "70B B=64 on the grown workspace")
    del g, w70


def test_growth_inside_capture_is_refused(orc):
    """A call that would have to grow the workspace while its stream is being
    captured returns DFK_ERR_UNSUPPORTED and enqueues nothing; a call that
    fits is captured as usual and its replays match the oracle."""
    dev = torch.device("cuda:0")
    small = _layers(1, 264, 456, 8400, dev)[0]
    big = _layers(1, 2048, 5632, 8410, dev)[0]
    xs = inputs.randn_bf16_device((2, 264), 1.0, 8420, dev)
    xb = inputs.randn_bf16_device((64, 2048), 1.0, 8421, dev)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dfk.dfk_swiglu_mlp(xs, *small)  # the stream's first workspace: the minimum size
    s.synchronize()
    outs = torch.empty((2, 264), dtype=torch.bfloat16, device=dev)
    outb = torch.empty((64, 2048), dtype=torch.bfloat16, device=dev)
    g = torch.cuda.CUDAGraph()
    refused = None
    with torch.cuda.graph(g, stream=s):
        try:
            dfk.dfk_swiglu_mlp(xb, *big, out=outb, layout=Layout.COL_MFMA)
        except dfk.DfkError as e:
            refused = e
        dfk.dfk_swiglu_mlp(xs, *small, out=outs)
    assert refused is not None and refused.status == Status.UNSUPPORTED
    want = _oracle_y(orc, xs, small)
    for r in range(2):
        outs.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        H.assert_y_close(H.host_bf16_as_f64(outs), want, f"replay {r}")
    # outside the capture the same large call grows the workspace and runs
    with torch.cuda.stream(s):
        dfk.dfk_swiglu_mlp(xb, *big, out=outb, layout=Layout.COL_MFMA)
    s.synchronize()
    H.assert_y_close(H.host_bf16_as_f64(outb), _oracle_y(orc, xb, big), "large call after the capture")


@pytest.mark.parametrize("kind,B", [("rmsnorm", 1), ("rmsnorm", 8), ("rmsnorm", 24), ("fp8", 1), ("fp8", 4),
                                    ("packed", 2), ("packed", 20)])
def test_graph_replays_other_entry_points(kind, B):
    """The RMS-normalized, FP8-weight and packed-weight MLPs captured the same
    way: every replay equals the eager call bit for bit."""
    import numpy as np
    dev = torch.device("cuda:0")
    dm, dff = 1040, 2064
    x = inputs.randn_bf16_device((B, dm), 1.0, 8700 + B, dev)
    if kind == "fp8":
        L = inputs.fp8_layer(B, dm, dff, seed=8800 + B, std=0.05)
        args = [torch.from_numpy(np.ascontiguousarray(L[k])).to(dev)
                for k in ("q_gate", "s_gate", "q_up", "s_up", "q_down", "s_down")]
        call = lambda out: dfk.dfk_swiglu_mlp_fp8(x, *args, out=out)
    else:
        wg, wu, wd = _layers(1, dm, dff, 8900 + B, dev)[0]
        if kind == "rmsnorm":
            gain = inputs.randn_bf16_device((dm,), 0.1, 8950, dev).add_(1.0)
            call = lambda out: dfk.dfk_rmsnorm_swiglu_mlp(x, gain, 1e-5, wg, wu, wd, out=out)
        else:
            wgu = dfk.pack_gate_up(wg, wu, dfk.Packing.INTERLEAVED)
            call = lambda out: dfk.dfk_swiglu_mlp_packed(x, wgu, wd, dfk.Packing.INTERLEAVED, out=out)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    ref = torch.empty((B, dm), dtype=torch.bfloat16, device=dev)
    with torch.cuda.stream(s):  # creates the stream's workspace
        call(ref)
    s.synchronize()
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(out)
    junk = torch.empty_like(ref)
    for r in range(3):
        out.fill_(float("nan"))
        with torch.cuda.stream(s):
            call(junk)
        s.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{kind} B={B} replay {r}"
