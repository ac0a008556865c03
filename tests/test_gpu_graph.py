"""Chained MLP calls captured into one HIP graph: the launch-gap removal path
for stacked layers.  Once a stream's workspace exists the library's calls do
no allocation and no synchronisation, so they capture; every replay, with
eager work and synchronisations between replays, must reproduce the eager
chain bit for bit (the kernels are deterministic)."""
import pytest
import torch

import swiglu_mlp_amd as dfk
from swiglu_mlp_amd import Layout, inputs

pytestmark = pytest.mark.gpu


def _layers(L, dm, dff, seed, dev):
    return [(inputs.randn_bf16_device((dff, dm), 0.02, seed + 10 * l + 1, dev),
             inputs.randn_bf16_device((dff, dm), 0.02, seed + 10 * l + 2, dev),
             inputs.randn_bf16_device((dm, dff), 0.02, seed + 10 * l + 3, dev)) for l in range(L)]


@pytest.mark.parametrize("B,dm,dff,L,layout", [
    (1, 4096, 14336, 4, Layout.AUTO),      # the 8B layer shape, the scheduler's variants
    (16, 1032, 2056, 3, Layout.COL_MFMA),  # down through K panels + the reduce kernel
    (40, 520, 1000, 3, Layout.AUTO),       # staged kernels, K split + reduce
    (5, 600, 1096, 3, Layout.ROW_MFMA),    # LDS-transposed gate-up, cooperative down
])
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
