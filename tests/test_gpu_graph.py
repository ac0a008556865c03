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
