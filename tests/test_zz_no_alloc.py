"""dfk_swiglu_mlp_noalloc: the whole MLP with h and the split sums in the
library's static device scratch, so the call allocates nothing.  Two calls in
a row on one device, the second smaller (the buffer keeps the first call's
contents), each against the allocating entry point bit for bit (same kernels)
and against the fp64 oracle; a call that needs more than the buffer is
refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import swiglu_mlp_amd as dfk
from swiglu_mlp_amd import Layout, Status, inputs
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _case(B, dm, dff, seed, dev):
    w = tuple(inputs.randn_bf16_device(shape, 0.02, seed + i, dev)
              for i, shape in enumerate(((dff, dm), (dff, dm), (dm, dff)), start=1))
    return inputs.randn_bf16_device((B, dm), 1.0, seed, dev), w


_ORACLE_Y = {}  # (B, d_model, d_ff, seed) -> the oracle's y, shared by the layouts


@pytest.mark.parametrize("layout", [Layout.AUTO, Layout.COL_MFMA, Layout.ROW])
def test_noalloc_matches_allocating_call_and_oracle(layout):
    dev = torch.device("cuda:0")
    orc = oracle.get()
    # first the largest supported workload (the 70B layer at B = 64: h and
    # the split sums fill most of the buffer), then a smaller one
    for (B, dm, dff, seed) in [(64, 8192, 28672, 9900), (3, 4096, 14336, 9910)]:
        print(f"noalloc {layout.name} B={B} {dm}x{dff}", flush=True)
        x, w = _case(B, dm, dff, seed, dev)
        out = torch.full((B, dm), float("nan"), dtype=torch.bfloat16, device=dev)
        dfk.dfk_swiglu_mlp_noalloc(x, *w, out=out, layout=layout)
        ref = dfk.dfk_swiglu_mlp(x, *w, layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (layout.name, B)
        key = (B, dm, dff, seed)
        if key not in _ORACLE_Y:
            _ORACLE_Y[key] = orc.mlp(H.host_bits(x), *(H.host_bits(t) for t in w))[0]
        y_ref = _ORACLE_Y[key]
        H.assert_y_close(H.host_bf16_as_f64(out), y_ref, f"noalloc {layout.name} B={B}")
        del w


def test_noalloc_refuses_beyond_its_buffer():
    dev = torch.device("cuda:0")
    B, dm, dff = 256, 8, 70000  # h alone is 71.7 MB > 64 MiB
    x = torch.zeros((B, dm), dtype=torch.bfloat16, device=dev)
    wg = torch.zeros((dff, dm), dtype=torch.bfloat16, device=dev)
    wd = torch.zeros((dm, dff), dtype=torch.bfloat16, device=dev)
    out = torch.full((B, dm), 7.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(dfk.DfkError) as e:
        dfk.dfk_swiglu_mlp_noalloc(x, wg, wg, wd, out=out)
    assert e.value.status == Status.UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out.float() == 7.0)  # nothing was enqueued
    # the shape itself is served: the allocating entry point runs it
    y = dfk.dfk_swiglu_mlp(x, wg, wg, wd)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y.float()).item() == 0
    with pytest.raises(dfk.DfkError) as e:
        dfk.dfk_swiglu_mlp_noalloc(x[:1], wg, wg, wd, out=out[:1], layout=Layout.ROW_PERSISTENT)
    assert e.value.status == Status.UNSUPPORTED
