"""Seeded synthetic inputs for the decode-stage SwiGLU MLP.

This module only draws numbers: it holds none of the MLP's arithmetic, imports
neither the HIP library nor the oracle, and is the one piece of code that both
sides of a parity check share.  bf16 tensors are returned as numpy uint16 bit
patterns (the form both the C-ABI and the oracle take).

Recipe (every workload is synthetic and shape-only; model names stand for
layer shapes, no trained weights are used):
  * values are drawn with ``torch.Generator().manual_seed(seed)`` on the CPU as
    fp32 ``randn`` times a standard deviation, then rounded to bf16 (ties to
    even) by torch's dtype conversion;
  * x ~ N(0, 1); Llama-shaped layers use weight std 0.02; the tiny layer uses
    std 1/sqrt(d_in) (variance 1/d_in) for every weight.
  * seeds: tiny layer x=0, W_gate=1, W_up=2, W_down=3; Llama-3-8B layer weights
    1001..1003, x 1100+B; 8B 32-layer stack weights 3000+4l+{1,2,3}, x0 3000;
    Llama-3-70B layer weights 4001..4003, x 4100+B; shape sweep entry s weights
    5000+100s+{1,2,3}, x 5000+100s+10+B.
  * RMS-normalization gains: 1 + N(0, 0.1^2) per column (``norm_gain``).
  * FP8 weights (``fp8_weights``): N(0, std^2) rows scaled by max|row| / 448
    into OCP E4M3 codes, x ~ N(0, 1); seeds seed+{1,2,3} for gate, up, down.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

# (d_model, d_ff) of the layer shapes the workloads name.
LLAMA3_8B = (4096, 14336)
LLAMA3_70B = (8192, 28672)
TINY = (256, 688)
SWEEP_SHAPES = [(2048, 5632), (3072, 8192), (4096, 14336), (5120, 13824), (8192, 28672)]
SWEEP_BATCHES = [1, 2, 4, 8, 16, 32, 64]


def to_bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Round an fp32 CPU tensor to bf16 (torch's RNE) and return the uint16 bits."""
    return t.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_float32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def randn_bf16(shape, std: float, seed: int) -> np.ndarray:
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return to_bf16_bits(t)


def rand_int_bf16(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """Uniform integers in [lo, hi] as bf16 (exact for |v| <= 256)."""
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randint(lo, hi + 1, tuple(shape), generator=g).to(torch.float32)
    return to_bf16_bits(t)


def randn_f32(shape, std: float, seed: int) -> np.ndarray:
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.numpy()


@dataclass
class Layer:
    """One MLP layer's inputs as bf16 bit patterns."""
    x: np.ndarray        # [B, d_model]
    w_gate: np.ndarray   # [d_ff, d_model]
    w_up: np.ndarray     # [d_ff, d_model]
    w_down: np.ndarray   # [d_model, d_ff]

    @property
    def B(self) -> int:
        return self.x.shape[0]

    @property
    def d_model(self) -> int:
        return self.x.shape[1]

    @property
    def d_ff(self) -> int:
        return self.w_gate.shape[0]


def weights(d_model: int, d_ff: int, seeds, std: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Gate/up/down weights; std None means 1/sqrt(d_in) per matrix."""
    sg = std if std is not None else 1.0 / math.sqrt(d_model)
    sd = std if std is not None else 1.0 / math.sqrt(d_ff)
    return {
        "w_gate": randn_bf16((d_ff, d_model), sg, seeds[0]),
        "w_up": randn_bf16((d_ff, d_model), sg, seeds[1]),
        "w_down": randn_bf16((d_model, d_ff), sd, seeds[2]),
    }


def tiny_layer() -> Layer:
    d_model, d_ff = TINY
    w = weights(d_model, d_ff, (1, 2, 3), std=None)
    return Layer(x=randn_bf16((1, d_model), 1.0, 0), **w)


def llama8b_layer(B: int) -> Layer:
    d_model, d_ff = LLAMA3_8B
    w = weights(d_model, d_ff, (1001, 1002, 1003), std=0.02)
    return Layer(x=randn_bf16((B, d_model), 1.0, 1100 + B), **w)


def llama70b_layer(B: int) -> Layer:
    d_model, d_ff = LLAMA3_70B
    w = weights(d_model, d_ff, (4001, 4002, 4003), std=0.02)
    return Layer(x=randn_bf16((B, d_model), 1.0, 4100 + B), **w)


def stack_layer_weights(layer: int) -> Dict[str, np.ndarray]:
    d_model, d_ff = LLAMA3_8B
    base = 3000 + 4 * layer
    return weights(d_model, d_ff, (base + 1, base + 2, base + 3), std=0.02)


def stack_x0(B: int = 1) -> np.ndarray:
    return randn_bf16((B, LLAMA3_8B[0]), 1.0, 3000)


def sweep_layer(s: int, B: int, d_model: Optional[int] = None, d_ff: Optional[int] = None) -> Layer:
    dm, df = SWEEP_SHAPES[s]
    dm = d_model or dm
    df = d_ff or df
    base = 5000 + 100 * s
    w = weights(dm, df, (base + 1, base + 2, base + 3), std=0.02)
    return Layer(x=randn_bf16((B, dm), 1.0, base + 10 + B), **w)


def random_layer(B: int, d_model: int, d_ff: int, seed: int, std: Optional[float] = None) -> Layer:
    """A generic seeded layer (std None: 1/sqrt(d_in))."""
    w = weights(d_model, d_ff, (seed + 1, seed + 2, seed + 3), std=std)
    return Layer(x=randn_bf16((B, d_model), 1.0, seed), **w)


def integer_layer(B: int, d_model: int, d_ff: int, seed: int, lo: int = -2, hi: int = 2) -> Layer:
    """Small-integer x and weights: every product and partial sum is exact in fp32."""
    return Layer(
        x=rand_int_bf16((B, d_model), lo, hi, seed),
        w_gate=rand_int_bf16((d_ff, d_model), lo, hi, seed + 1),
        w_up=rand_int_bf16((d_ff, d_model), lo, hi, seed + 2),
        w_down=rand_int_bf16((d_model, d_ff), lo, hi, seed + 3),
    )


def norm_gain(d_model: int, seed: int, std: float = 0.1) -> np.ndarray:
    """RMS-normalization gain [d_model] as bf16 bits: 1 + N(0, std^2) (a trained
    gain's spread around its initial value of one)."""
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randn(d_model, generator=g, dtype=torch.float32).mul_(std).add_(1.0)
    return to_bf16_bits(t)


def fp8_weights(rows: int, cols: int, std: float, seed: int):
    """Weight-only FP8 weights: (codes, scales).  Draws W ~ N(0, std^2) as
    fp32, takes one scale per row, s = max|W[row]| / 448 (1 for an all-zero
    row), and stores W / s as OCP FP8 E4M3 codes (torch's float8_e4m3fn
    conversion, round to nearest even): codes uint8 [rows, cols], scales
    float32 [rows].  The weight the codes stand for is s[row] * e4m3(code)."""
    g = torch.Generator().manual_seed(int(seed))
    w = torch.randn(rows, cols, generator=g, dtype=torch.float32).mul_(std)
    amax = w.abs().amax(dim=1)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (w / s[:, None]).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy().copy(), s.numpy().copy()


def fp8_layer(B: int, d_model: int, d_ff: int, seed: int, std: float = 0.02) -> Dict[str, np.ndarray]:
    """x (bf16 bits) and FP8 gate/up/down weights with their row scales."""
    qg, sg = fp8_weights(d_ff, d_model, std, seed + 1)
    qu, su = fp8_weights(d_ff, d_model, std, seed + 2)
    qd, sd = fp8_weights(d_model, d_ff, std, seed + 3)
    return {"x": randn_bf16((B, d_model), 1.0, seed), "q_gate": qg, "s_gate": sg, "q_up": qu, "s_up": su,
            "q_down": qd, "s_down": sd}


def integer_h(B: int, d_ff: int, seed: int, bound: int = 256) -> np.ndarray:
    """fp32 integer-valued h in [-bound, bound] (exactly representable)."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.randint(-bound, bound + 1, (B, d_ff), generator=g).to(torch.float32).numpy()


def h_like(B: int, d_ff: int, seed: int, std: float = 1.0) -> np.ndarray:
    """fp32 h drawn from N(0, std^2) (the spread of SiLU(g)*u at unit-scale g, u)."""
    return randn_f32((B, d_ff), std, seed)


def randn_bf16_device(shape, std: float, seed: int, device="cuda"):
    """bf16 N(0, std^2) drawn on the GPU with a seeded device generator (for
    multi-GB weight sets: the chained 32-layer stack and the benchmark's
    rotating weight copies).  Returns a torch bf16 tensor on `device`."""
    g = torch.Generator(device=device).manual_seed(int(seed))
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def stack_layer_weights_device(layer: int, device="cuda"):
    """W_gate, W_up, W_down of layer `layer` of the 8B 32-layer stack, on the GPU."""
    d_model, d_ff = LLAMA3_8B
    base = 3000 + 4 * layer
    return (randn_bf16_device((d_ff, d_model), 0.02, base + 1, device),
            randn_bf16_device((d_ff, d_model), 0.02, base + 2, device),
            randn_bf16_device((d_model, d_ff), 0.02, base + 3, device))
