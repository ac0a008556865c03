"""Shared test helpers: device transfer of bf16 bit patterns and parity metrics."""
from __future__ import annotations

import numpy as np

from swiglu_mlp_amd import inputs

# Parity bar on y (bf16 output, fp32 accumulation): normwise max relative error
# per batch row <= 1e-2 and normwise mean relative error <= 2e-3.
Y_MAX_REL = 1e-2
Y_MEAN_REL = 2e-3
# Bar on h (fp32, no bf16 rounding): two orders of magnitude tighter.
H_MAX_REL = 1e-4
H_MEAN_REL = 1e-4


def dev_bf16(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def dev_f32(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_bf16_as_f64(t) -> np.ndarray:
    return inputs.bits_to_float32(host_bits(t)).astype(np.float64)


def normwise(actual, ref):
    """(max over rows of max|d| / max|ref|, sum|d| / sum|ref|); zero references
    fall back to absolute error."""
    a = np.asarray(actual, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    d = np.abs(a - r)
    row_den = np.abs(r).max(axis=1)
    row_num = d.max(axis=1)
    row = np.where(row_den > 0, row_num / np.where(row_den > 0, row_den, 1), row_num)
    den = np.abs(r).sum()
    mean = d.sum() / den if den > 0 else d.sum()
    return float(row.max()), float(mean)


def assert_y_close(y_gpu, y_ref, what=""):
    mx, mean = normwise(y_gpu, y_ref)
    assert mx <= Y_MAX_REL and mean <= Y_MEAN_REL, f"{what}: normwise max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def assert_h_close(h_gpu, h_ref, what=""):
    mx, mean = normwise(h_gpu, h_ref)
    assert mx <= H_MAX_REL and mean <= H_MEAN_REL, f"{what}: normwise max {mx:.3e} mean {mean:.3e}"
    return mx, mean
