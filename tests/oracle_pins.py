"""Pins that tie the fp64 oracle to something other than itself.

Each ``check_*`` takes a loaded oracle and raises AssertionError when the
oracle disagrees with the mathematics: closed forms evaluated another way
(mpmath's tanh form of SiLU, the Lambert-W minimum), exact rational brute
force, library routines in another precision (numpy extended precision),
and invariants the definition implies.  The test suite runs every check on
the real oracle, and again on copies with planted mistakes, each of which
must fail at least one check.
"""
from __future__ import annotations

import math
from fractions import Fraction

import mpmath
import numpy as np
import scipy.special
import torch

from swiglu_mlp_amd import inputs

mpmath.mp.dps = 40


# ---------------------------------------------------------------- helpers --

def mp_silu(z) -> mpmath.mpf:
    """SiLU through the identity z*sigma(z) = (z/2)(1 + tanh(z/2)), at 40 digits."""
    z = mpmath.mpf(z)
    return z / 2 * (1 + mpmath.tanh(z / 2))


def widen(bits) -> np.ndarray:
    return inputs.bits_to_float32(bits).astype(np.float64)


def exact_mlp(x_bits, wg_bits, wu_bits, wd_bits):
    """Brute force: g, u as exact rationals; h and y at 40 digits via mpmath."""
    x, wg, wu, wd = (widen(a) for a in (x_bits, wg_bits, wu_bits, wd_bits))
    B, K = x.shape
    N = wg.shape[0]
    M = wd.shape[0]
    fx = [[Fraction(float(v)) for v in row] for row in x]
    g = [[sum((fx[b][k] * Fraction(float(wg[n, k])) for k in range(K)), Fraction(0))
          for n in range(N)] for b in range(B)]
    u = [[sum((fx[b][k] * Fraction(float(wu[n, k])) for k in range(K)), Fraction(0))
          for n in range(N)] for b in range(B)]
    h = [[mp_silu(mpmath.mpf(g[b][n].numerator) / g[b][n].denominator)
          * (mpmath.mpf(u[b][n].numerator) / u[b][n].denominator)
          for n in range(N)] for b in range(B)]
    y = [[mpmath.fsum(h[b][n] * mpmath.mpf(float(wd[m, n])) for n in range(N))
          for m in range(M)] for b in range(B)]
    return g, u, h, y


def normwise(actual, expect) -> float:
    a = np.asarray(actual, dtype=np.float64)
    e = np.asarray(expect, dtype=np.float64)
    den = np.abs(e).sum()
    num = np.abs(a - e).sum()
    return float(num / den) if den > 0 else float(num)


def bf16_of(values) -> np.ndarray:
    return inputs.to_bf16_bits(torch.tensor(np.asarray(values, dtype=np.float32)))


# ----------------------------------------------------------------- SiLU ----

def check_silu_tanh_form(orc):
    """SiLU against mpmath's tanh form on [-40, 40], within 4 ulp-ish (2e-15 rel)."""
    for z in np.concatenate([np.linspace(-40, 40, 161), [1e-300, -1e-300, 0.5, -0.5, 1e-8]]):
        ref = mp_silu(float(z))
        got = orc.silu(float(z))
        assert abs(mpmath.mpf(got) - ref) <= 2e-15 * abs(ref) + 1e-300, (z, got, ref)


def check_silu_lambert_minimum(orc):
    """SiLU has its global minimum -W(1/e) at z* = -1 - W(1/e) (W = Lambert W)."""
    w = float(scipy.special.lambertw(1.0 / math.e).real)
    zs = -1.0 - w
    assert abs(orc.silu(zs) - (-w)) <= 1e-15, (orc.silu(zs), -w)
    for d in (1e-3, 1e-2, 0.1, 1.0):
        assert orc.silu(zs - d) > orc.silu(zs) and orc.silu(zs + d) > orc.silu(zs)


def check_silu_identities(orc):
    """SiLU(z) - SiLU(-z) = z; SiLU(z) = z * expit(z) (scipy's logistic)."""
    for z in np.linspace(-30, 30, 121):
        z = float(z)
        assert abs((orc.silu(z) - orc.silu(-z)) - z) <= 4e-15 * max(1.0, abs(z))
        ref = z * float(scipy.special.expit(z))
        assert abs(orc.silu(z) - ref) <= 4e-16 * max(1.0, abs(z)) + 1e-300


def check_silu_limits(orc):
    """Limits and special values: 0 at 0, -0 far left, z far right, NaN propagates."""
    assert orc.silu(0.0) == 0.0
    v = orc.silu(-800.0)
    assert v == 0.0 and math.copysign(1.0, v) < 0
    assert orc.silu(800.0) == 800.0
    assert 0 > orc.silu(-20.0) > -5e-8
    assert math.isnan(orc.silu(float("nan")))


# ------------------------------------------------------------- bf16 RNE ---

def check_bf16_rne(orc):
    """Round-to-nearest-even into bf16, straight from fp64."""
    cases = {
        1.0: 0x3F80, -1.0: 0xBF80, 0.0: 0x0000, 2.0: 0x4000,
        1.0 + 2 ** -8: 0x3F80,                 # tie -> even
        1.0 + 3 * 2 ** -8: 0x3F82,             # tie -> even (up)
        1.0 + 2 ** -8 + 2 ** -40: 0x3F81,      # just above the tie: a float detour would tie
        1.1321045812384946: 0x3F91,
        1.2836359521984556: 0x3FA4,
        2 ** -133: 0x0001,                     # smallest subnormal
        2 ** -134: 0x0000,                     # tie with zero -> even (zero)
        3.0 * 2 ** -134: 0x0002,               # 1.5 quanta -> 2 (even)
        3.4e38: 0x7F80,                        # rounds past the largest finite value
        3.3895313892515355e38: 0x7F7F,         # largest finite bf16
        -math.inf: 0xFF80,
    }
    for d, bits in cases.items():
        assert orc.bf16_rne(d) == bits, (d, hex(orc.bf16_rne(d)), hex(bits))
    assert math.copysign(1.0, orc.bf16_to_double(orc.bf16_rne(-0.0))) < 0
    assert orc.bf16_rne(float("nan")) == 0x7FC0
    # every binary32 value: the same as torch's fp32 -> bf16 conversion
    gen = torch.Generator().manual_seed(7)
    f = torch.randn(20000, generator=gen) * torch.exp(torch.randn(20000, generator=gen) * 20)
    want = f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_rne_array(f.double().numpy())
    assert np.array_equal(got, want)


# ---------------------------------------------------- whole-MLP pins -------

def worked_example():
    """x=[1,-2]; gate rows [1,0],[0,1],[1,1]; up rows [2,0],[0,1],[1,-1];
    down rows [1,1,1],[0,1,-1]; zero-padded to d_model = d_ff = 8."""
    x = np.zeros((1, 8)); x[0, :2] = [1, -2]
    wg = np.zeros((8, 8)); wg[0, :2] = [1, 0]; wg[1, :2] = [0, 1]; wg[2, :2] = [1, 1]
    wu = np.zeros((8, 8)); wu[0, :2] = [2, 0]; wu[1, :2] = [0, 1]; wu[2, :2] = [1, -1]
    wd = np.zeros((8, 8)); wd[0, :3] = [1, 1, 1]; wd[1, :3] = [0, 1, -1]
    return bf16_of(x), bf16_of(wg), bf16_of(wu), bf16_of(wd)


def worked_example_expected():
    """Closed form: g = [1,-2,-1], u = [2,-2,3], h = SiLU(g)*u, y = Wd h."""
    g = [1, -2, -1]
    u = [2, -2, 3]
    h = [mp_silu(gi) * ui for gi, ui in zip(g, u)]
    y = [h[0] + h[1] + h[2], h[1] - h[2]]
    return g, u, h, y


def check_worked_example(orc):
    x, wg, wu, wd = worked_example()
    g, u, h = orc.gate_up(x, wg, wu)
    eg, eu, eh, ey = worked_example_expected()
    assert np.array_equal(g[0, :3], eg) and np.array_equal(u[0, :3], eu)
    assert np.all(g[0, 3:] == 0) and np.all(h[0, 3:] == 0)
    for a, e in zip(h[0, :3], eh):
        assert abs(mpmath.mpf(a) - e) <= 1e-15 * abs(e)
    y, _ = orc.mlp(x, wg, wu, wd)
    for a, e in zip(y[0, :2], ey):
        assert abs(mpmath.mpf(a) - e) <= 1e-15 * abs(e)
    assert np.all(y[0, 2:] == 0)
    # y in bf16 (RNE): 1.1321045812... -> 0x3F91, 1.2836359521... -> 0x3FA4
    assert list(orc.bf16_rne_array(y[0, :2])) == [0x3F91, 0x3FA4]


def check_bruteforce_tiny(orc):
    """Tiny shapes (non-square, several seeds, integer and normal values) against
    exact rationals + 40-digit SiLU: normwise error <= 1e-14 on g, u, h and y."""
    shapes = [(1, 3, 5), (2, 5, 3), (3, 8, 8), (2, 7, 4), (3, 4, 7)]
    for i, (B, K, N) in enumerate(shapes):
        for kind in ("int", "normal"):
            if kind == "int":
                L = inputs.integer_layer(B, K, N, seed=100 + i, lo=-3, hi=3)
            else:
                L = inputs.random_layer(B, K, N, seed=200 + i, std=0.7)
            eg, eu, eh, ey = exact_mlp(L.x, L.w_gate, L.w_up, L.w_down)
            g, u, h = orc.gate_up(L.x, L.w_gate, L.w_up)
            y, h2 = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
            fl = lambda m: np.array([[float(v) for v in row] for row in m])
            assert normwise(g, fl(eg)) <= 1e-14, ("g", B, K, N, kind)
            assert normwise(u, fl(eu)) <= 1e-14, ("u", B, K, N, kind)
            assert normwise(h, fl(eh)) <= 1e-14, ("h", B, K, N, kind)
            assert normwise(y, fl(ey)) <= 1e-14, ("y", B, K, N, kind)
            assert np.array_equal(h, h2)


def check_extended_precision(orc):
    """Moderate shapes against numpy's 80-bit extended-precision matmul."""
    L = inputs.random_layer(3, 96, 160, seed=300, std=None)
    x, wg, wu, wd = (widen(a).astype(np.longdouble) for a in (L.x, L.w_gate, L.w_up, L.w_down))
    g = x @ wg.T
    u = x @ wu.T
    h = g / (1 + np.exp(-g)) * u
    y = h @ wd.T
    og, ou, oh = orc.gate_up(L.x, L.w_gate, L.w_up)
    oy, _ = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    assert normwise(og, g.astype(np.float64)) <= 1e-15
    assert normwise(ou, u.astype(np.float64)) <= 1e-15
    assert normwise(oy, y.astype(np.float64)) <= 1e-14
    # the down projection on its own, on an arbitrary fp32 h
    hf = inputs.h_like(3, 160, seed=301)
    oyd = orc.down(hf, L.w_down)
    yd = hf.astype(np.longdouble) @ wd.T
    assert normwise(oyd, yd.astype(np.float64)) <= 1e-15


def check_zero_invariants(orc):
    """x = 0, W_gate = 0, W_up = 0 or W_down = 0 each give y == 0 exactly."""
    L = inputs.random_layer(3, 64, 96, seed=400, std=None)
    zero_x = np.zeros_like(L.x)
    for args in ((zero_x, L.w_gate, L.w_up, L.w_down),
                 (L.x, np.zeros_like(L.w_gate), L.w_up, L.w_down),
                 (L.x, L.w_gate, np.zeros_like(L.w_up), L.w_down),
                 (L.x, L.w_gate, L.w_up, np.zeros_like(L.w_down))):
        y, _ = orc.mlp(*args)
        assert np.all(y == 0.0)
    y, h = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    assert np.any(y != 0.0) and np.any(h != 0.0)


def check_linearity_in_wdown(orc):
    """y(2 Wd) = 2 y(Wd) and y(-Wd) = -y(Wd) exactly; disjoint supports add."""
    L = inputs.random_layer(2, 48, 80, seed=500, std=None)
    wd = widen(L.w_down).astype(np.float32)
    y, _ = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    y2, _ = orc.mlp(L.x, L.w_gate, L.w_up, bf16_of(2 * wd))
    yn, _ = orc.mlp(L.x, L.w_gate, L.w_up, bf16_of(-wd))
    assert np.array_equal(y2, 2 * y) and np.array_equal(yn, -y)
    mask = (np.arange(wd.size).reshape(wd.shape) * 7919) % 3 == 0
    ya, _ = orc.mlp(L.x, L.w_gate, L.w_up, bf16_of(np.where(mask, wd, 0)))
    yb, _ = orc.mlp(L.x, L.w_gate, L.w_up, bf16_of(np.where(mask, 0, wd)))
    assert normwise(ya + yb, y) <= 1e-14


def check_batch_and_permutation(orc):
    """Each batch row is its own problem; permuting the d_ff neurons consistently
    (rows of W_gate and W_up, columns of W_down) leaves y unchanged."""
    L = inputs.random_layer(5, 40, 72, seed=600, std=None)
    y, _ = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    for b in range(L.B):
        yb, _ = orc.mlp(L.x[b:b + 1], L.w_gate, L.w_up, L.w_down)
        assert np.array_equal(yb[0], y[b])
    perm = np.random.default_rng(601).permutation(L.d_ff)
    yp, hp = orc.mlp(L.x, L.w_gate[perm], L.w_up[perm], np.ascontiguousarray(L.w_down[:, perm]))
    assert normwise(yp, y) <= 1e-14
    _, h = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down)
    assert np.array_equal(hp, h[:, perm])


def check_threads_deterministic(orc):
    L = inputs.random_layer(4, 64, 128, seed=700, std=None)
    y1, h1 = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down, nthreads=1)
    y7, h7 = orc.mlp(L.x, L.w_gate, L.w_up, L.w_down, nthreads=7)
    assert np.array_equal(y1, y7) and np.array_equal(h1, h7)


def check_rms_rescale(orc):
    """Between-layer rescale: each output row has mean square 1 (to bf16 rounding),
    and scaling y by a power of two leaves the result unchanged."""
    y = inputs.randn_bf16((3, 256), 3.0, seed=800)
    x = orc.rms_rescale(y, eps=0.0)
    xf = widen(x)
    assert np.allclose((xf ** 2).mean(axis=1), 1.0, rtol=1e-2)
    y4 = bf16_of(4 * widen(y))
    assert np.array_equal(orc.rms_rescale(y4, eps=0.0), x)
    # a row that is a power-of-two multiple of a ones vector maps to exactly ones
    ones = bf16_of(np.full((1, 64), 8.0))
    assert np.all(widen(orc.rms_rescale(ones, eps=0.0)) == 1.0)
    # eps > 0 against 60-digit arithmetic and an independent ties-to-even
    # rounding, on rows whose mean square is of the order of eps (so eps
    # placed outside the square root, or dropped, moves every value)
    mpmath.mp.dps = 60
    try:
        small = inputs.randn_bf16((2, 48), 0.01, seed=801)
        sf = widen(small)
        for eps in (1e-4, 1e-6, 0.5):
            got = orc.rms_rescale(small, eps=eps)
            for b in range(2):
                ms = mpmath.fsum(mpmath.mpf(float(v)) ** 2 for v in sf[b]) / 48
                inv = 1 / mpmath.sqrt(ms + mpmath.mpf(eps))
                for k in range(48):
                    want = _mp_rne_bf16_bits(mpmath.mpf(float(sf[b, k])) * inv)
                    assert int(got[b, k]) == want, (eps, b, k)
    finally:
        mpmath.mp.dps = 40


def _mp_rne_bf16_bits(v):
    """Round an mpmath real to bf16 bits, ties to even, for normal-range values
    (an implementation independent of the oracle's)."""
    import mpmath
    if v == 0:
        return 0x8000 if mpmath.sign(v) < 0 else 0
    m, e = mpmath.frexp(v)            # v = m * 2^e, 0.5 <= |m| < 1
    q = mpmath.ldexp(1, int(e) - 8)   # one unit in the 8th significant bit
    r = mpmath.nint(v / q) * q        # nint: nearest integer, ties to even
    return int(np.float32(float(r)).view(np.uint32) >> 16)


def check_rmsnorm_bruteforce(orc):
    """Tiny rows against 60-digit arithmetic and an independent bf16 rounding."""
    import mpmath
    mpmath.mp.dps = 60
    x = inputs.randn_bf16((3, 7), 1.5, seed=810)
    g = inputs.randn_bf16((7,), 1.0, seed=811)
    for eps in (0.0, 1e-5, 0.25):
        xn = orc.rmsnorm(x, g, eps=eps)
        xf, gf = widen(x), widen(g)
        for b in range(3):
            ss = mpmath.fsum(mpmath.mpf(float(v)) ** 2 for v in xf[b])
            inv = 1 / mpmath.sqrt(ss / 7 + mpmath.mpf(eps))
            for k in range(7):
                want = _mp_rne_bf16_bits(mpmath.mpf(float(xf[b, k])) * inv * mpmath.mpf(float(gf[k])))
                assert int(xn[b, k]) == want, (eps, b, k)


def check_rmsnorm_invariants(orc):
    """Exact invariants: power-of-two scaling of x (eps = 0) changes nothing;
    doubling the gain doubles the output; a constant row maps to the gain
    itself; rows are independent; eps dominates a tiny row."""
    x = inputs.randn_bf16((4, 96), 2.0, seed=820)
    g = inputs.randn_bf16((96,), 1.0, seed=821)
    base = orc.rmsnorm(x, g, eps=0.0)
    assert np.array_equal(orc.rmsnorm(bf16_of(8 * widen(x)), g, eps=0.0), base)
    assert np.array_equal(orc.rmsnorm(x, bf16_of(2 * widen(g)), eps=0.0), bf16_of(2 * widen(base)))
    const = bf16_of(np.full((2, 96), 8.0))
    assert np.array_equal(orc.rmsnorm(const, g, eps=0.0), np.stack([g, g]))
    for b in range(4):
        assert np.array_equal(orc.rmsnorm(x[b:b + 1], g, eps=1e-5)[0], orc.rmsnorm(x, g, eps=1e-5)[b])
    tiny = bf16_of(np.full((1, 96), 2.0 ** -12))
    ones = bf16_of(np.ones(96))
    want = bf16_of(np.full((1, 96), 2.0 ** -12 / np.sqrt(2.0 ** -24 + 1.0)))
    assert np.array_equal(orc.rmsnorm(tiny, ones, eps=1.0), want)
    # unit gain: mean square 1 up to the bf16 rounding
    assert np.allclose((widen(orc.rmsnorm(x, ones, eps=0.0)) ** 2).mean(axis=1), 1.0, rtol=1e-2)


# ------------------------------------------------------- FP8 weights ----

def check_e4m3_decode(orc):
    """Every E4M3 code against torch's float8_e4m3fn (an independent decoder)
    and the format's fixed points: 448 the largest finite value, 2^-6 the
    smallest normal, 2^-9 the smallest subnormal, S.1111.111 NaN, signed zero."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3_to_double(int(c)) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert orc.e4m3_to_double(0x7E) == 448.0 and orc.e4m3_to_double(0xFE) == -448.0
    assert orc.e4m3_to_double(0x08) == 2.0 ** -6 and orc.e4m3_to_double(0x01) == 2.0 ** -9
    assert orc.e4m3_to_double(0x38) == 1.0 and orc.e4m3_to_double(0x3F) == 1.875
    assert np.isnan(orc.e4m3_to_double(0x7F)) and np.isnan(orc.e4m3_to_double(0xFF))
    assert math.copysign(1.0, orc.e4m3_to_double(0x80)) == -1.0


def _fp8_exact_bf16_layer(B, K, N, seed):
    """FP8 codes with power-of-two row scales 2^-(row % 5): every weight
    s * e4m3(q) then has at most 4 significant bits, so it is also exactly a
    bf16 value."""
    rng = np.random.default_rng(seed)

    def codes(r, c):
        q = rng.integers(0, 256, size=(r, c), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x38  # no NaN codes
        return q

    def scales(r):
        return np.array([2.0 ** -(i % 5) for i in range(r)], dtype=np.float32)

    def as_bf16(q, s):
        vals = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64) * torch.from_numpy(
            s.astype(np.float64))[:, None]
        return inputs.to_bf16_bits(vals.to(torch.float32))

    x = inputs.randn_bf16((B, K), 1.0, seed)
    qg, qu, qd = codes(N, K), codes(N, K), codes(K, N)
    sg, su, sd = scales(N), scales(N)[::-1].copy(), scales(K)
    return x, (qg, sg, qu, su, qd, sd), (as_bf16(qg, sg), as_bf16(qu, su), as_bf16(qd, sd))


def check_fp8_reduces_to_bf16(orc):
    """Quantized weights whose dequantized values are exactly bf16: the FP8
    MLP must equal the (pinned) bf16 MLP over those values bit for bit in
    fp64, on h and y."""
    for i, (B, K, N) in enumerate([(1, 16, 24), (3, 40, 8), (2, 8, 56)]):
        x, (qg, sg, qu, su, qd, sd), (wg, wu, wd) = _fp8_exact_bf16_layer(B, K, N, seed=300 + i)
        y8, h8 = orc.mlp_fp8(x, qg, sg, qu, su, qd, sd)
        y, h = orc.mlp(x, wg, wu, wd)
        assert np.array_equal(h8, h), ("h", B, K, N)
        assert np.array_equal(y8, y), ("y", B, K, N)
        assert np.array_equal(orc.gate_up_fp8(x, qg, sg, qu, su), h)
        assert np.array_equal(orc.down_fp8(h, qd, sd), y)


def check_fp8_bruteforce(orc):
    """General fp32 row scales against exact rationals + 40-digit SiLU:
    normwise error <= 1e-14 on h and y."""
    for i, (B, K, N) in enumerate([(1, 8, 5), (2, 5, 7), (3, 16, 4)]):
        L = inputs.fp8_layer(B, K, N, seed=400 + i, std=0.5)

        def deq(q, s):
            return torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy() * \
                s.astype(np.float64)[:, None]

        wg, wu, wd = deq(L["q_gate"], L["s_gate"]), deq(L["q_up"], L["s_up"]), deq(L["q_down"], L["s_down"])
        xs = widen(L["x"])
        fx = [[Fraction(float(v)) for v in row] for row in xs]
        g = [[sum((fx[b][k] * Fraction(float(wg[n, k])) for k in range(K)), Fraction(0)) for n in range(N)]
             for b in range(B)]
        u = [[sum((fx[b][k] * Fraction(float(wu[n, k])) for k in range(K)), Fraction(0)) for n in range(N)]
             for b in range(B)]
        eh = [[mp_silu(mpmath.mpf(g[b][n].numerator) / g[b][n].denominator)
               * (mpmath.mpf(u[b][n].numerator) / u[b][n].denominator) for n in range(N)] for b in range(B)]
        ey = [[mpmath.fsum(eh[b][n] * mpmath.mpf(float(wd[m, n])) for n in range(N)) for m in range(K)]
              for b in range(B)]
        y, h = orc.mlp_fp8(L["x"], L["q_gate"], L["s_gate"], L["q_up"], L["s_up"], L["q_down"], L["s_down"])
        fl = lambda m: np.array([[float(v) for v in row] for row in m])
        assert normwise(h, fl(eh)) <= 1e-14, ("h", B, K, N)
        assert normwise(y, fl(ey)) <= 1e-14, ("y", B, K, N)


def check_fp8_scale_linearity(orc):
    """Doubling every up scale doubles h and y; doubling every down scale
    doubles y (powers of two: exact in fp64)."""
    L = inputs.fp8_layer(2, 24, 40, seed=450, std=0.3)
    a = [L[k] for k in ("q_gate", "s_gate", "q_up", "s_up", "q_down", "s_down")]
    y, h = orc.mlp_fp8(L["x"], *a)
    a_up = list(a); a_up[3] = a[3] * 2
    y2, h2 = orc.mlp_fp8(L["x"], *a_up)
    assert np.array_equal(h2, 2 * h) and np.array_equal(y2, 2 * y)
    a_dn = list(a); a_dn[5] = a[5] * 2
    y3, h3 = orc.mlp_fp8(L["x"], *a_dn)
    assert np.array_equal(h3, h) and np.array_equal(y3, 2 * y)


ALL_CHECKS = [
    check_silu_tanh_form, check_silu_lambert_minimum, check_silu_identities,
    check_silu_limits, check_bf16_rne, check_worked_example, check_bruteforce_tiny,
    check_extended_precision, check_zero_invariants, check_linearity_in_wdown,
    check_batch_and_permutation, check_threads_deterministic, check_rms_rescale,
    check_rmsnorm_bruteforce, check_rmsnorm_invariants, check_e4m3_decode, check_fp8_reduces_to_bf16,
    check_fp8_bruteforce, check_fp8_scale_linearity,
]
