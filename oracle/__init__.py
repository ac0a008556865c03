"""fp64 CPU oracle for the decode-stage SwiGLU MLP (ctypes binding).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package.  It imports
nothing from the HIP library and the HIP library imports nothing from it.

The arithmetic lives in ``swiglu_oracle.c`` (plain C, fp64, summation in
ascending index order); this module only builds it with gcc, marshals numpy
arrays and returns numpy arrays.  bf16 tensors travel as their uint16 bit
patterns.  What each function computes, and the passages it follows, is
documented in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "swiglu_oracle.c")
# DFK_ORACLE_LIBRARY may name another build of the same source (the
# sanitizer test runs the pins against an ASan/UBSan build).
LIBRARY = os.environ.get("DFK_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")

# No -ffast-math and no FMA contraction: every product and sum is one IEEE
# fp64 operation, in source order.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-pthread"]


def build(source: str = SOURCE, output: str = LIBRARY, extra=()) -> str:
    """Compile the oracle with gcc; returns the library path."""
    cmd = ["gcc", *CFLAGS, *extra, source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)


def _p16(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_u16p)


def _p64(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_f64p)


def _codes(a, name: str) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8 or a.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint8 array of FP8 codes")
    return a


def _scales(a, n: int) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    if a.shape != (n,):
        raise ValueError(f"expected {n} row scales, got {a.shape}")
    return a


def _bits(a, name: str) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name}: expected bf16 bit patterns as uint16, got {a.dtype}")
    return a


class Oracle:
    """One loaded copy of the oracle library (tests may load a rebuilt copy)."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library {path} is not built")
        lib = ctypes.CDLL(path)
        self._lib = lib
        self.path = path
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_rne_array.restype = None
        lib.oracle_bf16_rne_array.argtypes = [_f64p, ctypes.c_long, _u16p]
        lib.oracle_gate_up.restype = ctypes.c_int
        lib.oracle_gate_up.argtypes = [_u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, _f64p, _f64p, _f64p, ctypes.c_int]
        lib.oracle_down.restype = ctypes.c_int
        lib.oracle_down.argtypes = [_f64p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    _f64p, ctypes.c_int]
        lib.oracle_mlp.restype = ctypes.c_int
        lib.oracle_mlp.argtypes = [_u16p, _u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, _f64p, _f64p, ctypes.c_int]
        lib.oracle_rms_rescale.restype = ctypes.c_int
        lib.oracle_rms_rescale.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                           _u16p]
        lib.oracle_e4m3_to_double.restype = ctypes.c_double
        lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        _u8p, _f32p = ctypes.c_void_p, ctypes.c_void_p
        lib.oracle_gate_up_fp8.restype = ctypes.c_int
        lib.oracle_gate_up_fp8.argtypes = [_u16p, _u8p, _f32p, _u8p, _f32p, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, _f64p, ctypes.c_int]
        lib.oracle_down_fp8.restype = ctypes.c_int
        lib.oracle_down_fp8.argtypes = [_f64p, _u8p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _f64p,
                                        ctypes.c_int]
        lib.oracle_mlp_fp8.restype = ctypes.c_int
        lib.oracle_mlp_fp8.argtypes = [_u16p, _u8p, _f32p, _u8p, _f32p, _u8p, _f32p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, _f64p, _f64p, ctypes.c_int]
        lib.oracle_rmsnorm.restype = ctypes.c_int
        lib.oracle_rmsnorm.argtypes = [_u16p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_double, _u16p]

    # -- scalars -----------------------------------------------------------
    def silu(self, z: float) -> float:
        return self._lib.oracle_silu(float(z))

    def bf16_rne(self, d: float) -> int:
        return int(self._lib.oracle_bf16_rne(float(d)))

    def bf16_to_double(self, bits: int) -> float:
        return self._lib.oracle_bf16_to_double(int(bits))

    def bf16_rne_array(self, a) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self._lib.oracle_bf16_rne_array(_p64(a), a.size, _p16(out))
        return out

    # -- the MLP ------------------------------------------------------------
    def gate_up(self, x, w_gate, w_up, nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Returns fp64 (g, u, h), each [B, d_ff]."""
        x, wg, wu = _bits(x, "x"), _bits(w_gate, "w_gate"), _bits(w_up, "w_up")
        B, d_model = x.shape
        d_ff = wg.shape[0]
        if wg.shape != (d_ff, d_model) or wu.shape != (d_ff, d_model):
            raise ValueError("gate/up weights must be [d_ff, d_model]")
        g = np.empty((B, d_ff)); u = np.empty((B, d_ff)); h = np.empty((B, d_ff))
        rc = self._lib.oracle_gate_up(_p16(x), _p16(wg), _p16(wu), B, d_model, d_ff,
                                      _p64(g), _p64(u), _p64(h), nthreads)
        if rc != 0:
            raise RuntimeError(f"oracle_gate_up failed ({rc})")
        return g, u, h

    def down(self, h, w_down, nthreads: int = 0) -> np.ndarray:
        """h: [B, d_ff] (any float dtype; widened exactly to fp64). Returns fp64 y [B, d_model]."""
        h = np.ascontiguousarray(h, dtype=np.float64)
        wd = _bits(w_down, "w_down")
        B, d_ff = h.shape
        d_model = wd.shape[0]
        if wd.shape != (d_model, d_ff):
            raise ValueError("down weight must be [d_model, d_ff]")
        y = np.empty((B, d_model))
        rc = self._lib.oracle_down(_p64(h), _p16(wd), B, d_model, d_ff, _p64(y), nthreads)
        if rc != 0:
            raise RuntimeError(f"oracle_down failed ({rc})")
        return y

    def mlp(self, x, w_gate, w_up, w_down, nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """Returns fp64 (y [B, d_model], h [B, d_ff])."""
        x, wg, wu, wd = (_bits(x, "x"), _bits(w_gate, "w_gate"), _bits(w_up, "w_up"),
                         _bits(w_down, "w_down"))
        B, d_model = x.shape
        d_ff = wg.shape[0]
        if (wg.shape != (d_ff, d_model) or wu.shape != (d_ff, d_model)
                or wd.shape != (d_model, d_ff)):
            raise ValueError("weight shapes do not match x")
        y = np.empty((B, d_model)); h = np.empty((B, d_ff))
        rc = self._lib.oracle_mlp(_p16(x), _p16(wg), _p16(wu), _p16(wd), B, d_model, d_ff,
                                  _p64(y), _p64(h), nthreads)
        if rc != 0:
            raise RuntimeError(f"oracle_mlp failed ({rc})")
        return y, h

    # -- weight-only FP8 weights ---------------------------------------------
    def e4m3_to_double(self, code: int) -> float:
        return self._lib.oracle_e4m3_to_double(int(code))

    def gate_up_fp8(self, x, q_gate, s_gate, q_up, s_up, nthreads: int = 0) -> np.ndarray:
        """h fp64 [B, d_ff] over W = s[row] * e4m3(q)."""
        x = _bits(x, "x")
        B, d_model = x.shape
        qg, qu = _codes(q_gate, "q_gate"), _codes(q_up, "q_up")
        sg, su = _scales(s_gate, qg.shape[0]), _scales(s_up, qg.shape[0])
        d_ff = qg.shape[0]
        if qg.shape != (d_ff, d_model) or qu.shape != (d_ff, d_model):
            raise ValueError("weight shapes do not match x")
        h = np.empty((B, d_ff))
        rc = self._lib.oracle_gate_up_fp8(_p16(x), qg.ctypes.data, sg.ctypes.data, qu.ctypes.data,
                                          su.ctypes.data, B, d_model, d_ff, _p64(h), nthreads)
        if rc != 0:
            raise RuntimeError(f"oracle_gate_up_fp8 failed ({rc})")
        return h

    def down_fp8(self, h, q_down, s_down, nthreads: int = 0) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.float64)
        B, d_ff = h.shape
        qd = _codes(q_down, "q_down")
        d_model = qd.shape[0]
        if qd.shape != (d_model, d_ff):
            raise ValueError("q_down shape does not match h")
        sd = _scales(s_down, d_model)
        y = np.empty((B, d_model))
        rc = self._lib.oracle_down_fp8(_p64(h), qd.ctypes.data, sd.ctypes.data, B, d_model, d_ff, _p64(y),
                                       nthreads)
        if rc != 0:
            raise RuntimeError(f"oracle_down_fp8 failed ({rc})")
        return y

    def mlp_fp8(self, x, q_gate, s_gate, q_up, s_up, q_down, s_down, nthreads: int = 0):
        """(y, h) fp64 over the dequantized FP8 weights."""
        x = _bits(x, "x")
        B, d_model = x.shape
        qg, qu, qd = _codes(q_gate, "q_gate"), _codes(q_up, "q_up"), _codes(q_down, "q_down")
        d_ff = qg.shape[0]
        if qg.shape != (d_ff, d_model) or qu.shape != (d_ff, d_model) or qd.shape != (d_model, d_ff):
            raise ValueError("weight shapes do not match x")
        sg, su, sd = _scales(s_gate, d_ff), _scales(s_up, d_ff), _scales(s_down, d_model)
        y = np.empty((B, d_model)); h = np.empty((B, d_ff))
        rc = self._lib.oracle_mlp_fp8(_p16(x), qg.ctypes.data, sg.ctypes.data, qu.ctypes.data, su.ctypes.data,
                                      qd.ctypes.data, sd.ctypes.data, B, d_model, d_ff, _p64(y), _p64(h),
                                      nthreads)
        if rc != 0:
            raise RuntimeError(f"oracle_mlp_fp8 failed ({rc})")
        return y, h

    def rmsnorm(self, x, gain, eps: float = 1e-5) -> np.ndarray:
        """RMS normalization ahead of the gate-up projections; returns bf16 bits [B, d_model]."""
        x, g = _bits(x, "x"), _bits(gain, "gain")
        B, d_model = x.shape
        g = g.reshape(-1)
        if g.shape != (d_model,):
            raise ValueError("gain must be [d_model]")
        out = np.empty_like(x)
        rc = self._lib.oracle_rmsnorm(_p16(x), _p16(np.ascontiguousarray(g)), B, d_model, float(eps), _p16(out))
        if rc != 0:
            raise RuntimeError(f"oracle_rmsnorm failed ({rc})")
        return out

    def rms_rescale(self, y_bits, eps: float = 1e-6) -> np.ndarray:
        """Between-layer rescale of the chained workload; returns bf16 bits."""
        y = _bits(y_bits, "y")
        B, d_model = y.shape
        out = np.empty_like(y)
        rc = self._lib.oracle_rms_rescale(_p16(y), B, d_model, float(eps), _p16(out))
        if rc != 0:
            raise RuntimeError(f"oracle_rms_rescale failed ({rc})")
        return out


_default: Optional[Oracle] = None


def get(build_if_missing: bool = True) -> Oracle:
    """The oracle built from this package's source (built on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) and build_if_missing:
            build()
        _default = Oracle(LIBRARY)
    return _default
