"""Fused decode-stage SwiGLU MLP for MI355X (gfx950): Python binding of libdfk.so.

Argument marshalling only: every step of the MLP runs in the HIP kernels of
``libdfk.so``; this module checks tensor dtypes/devices/shapes, passes device
pointers and the current HIP stream through the C ABI (``include/dfk.h``), and
turns a non-OK status into ``DfkError``.  There is no fallback path: if the
library is missing, every call raises.

The functions keep the C names:
    dfk_gate_up_silu_mul(x, W_gate, W_up, h=None, layout=AUTO, stream=None) -> h
    dfk_down_proj(h, W_down, out=None, layout=AUTO, stream=None) -> out
    dfk_swiglu_mlp(x, W_gate, W_up, W_down, out=None, layout=AUTO, stream=None) -> out
    dfk_schedule_select(B, d_model, d_ff) -> (gate_up_layout, down_layout)
Tensors: x [B, d_model] bf16, W_gate/W_up [d_ff, d_model] bf16, W_down
[d_model, d_ff] bf16, h [B, d_ff] fp32, out [B, d_model] bf16, all contiguous
on one GPU.
"""
from __future__ import annotations

import ctypes
import enum
import os
from typing import Optional, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# DFK_LIBRARY may name another build of the same library (e.g. one compiled
# with different tile parameters for a sweep).
LIBRARY = os.environ.get("DFK_LIBRARY") or os.path.join(PKG_DIR, "libdfk.so")
TUNING_TABLE = os.path.join(PKG_DIR, "tuning", "gfx950.json")


class Layout(enum.IntEnum):
    AUTO = 0
    ROW = 1
    COL = 2
    ROW_VALU = 3
    COL_VALU = 4
    ROW_MFMA = 5
    COL_MFMA = 6
    ROW_PERSISTENT = 7


class Packing(enum.IntEnum):
    BLOCKED = 0
    INTERLEAVED = 1


class Status(enum.IntEnum):
    OK = 0
    INVALID_ARG = 1
    UNSUPPORTED = 2
    MISALIGNED = 3
    HIP = 4
    OOM = 5


EXPORTED = (
    "dfk_gate_up_silu_mul", "dfk_down_proj", "dfk_swiglu_mlp", "dfk_schedule_select",
    "dfk_status_string", "dfk_layout_name", "dfk_version", "dfk_load_tuning_table",
    "dfk_tuning_table_source", "dfk_release_workspace", "dfk_rmsnorm",
    "dfk_rmsnorm_gate_up_silu_mul", "dfk_rmsnorm_swiglu_mlp", "dfk_gate_up_silu_mul_packed",
    "dfk_swiglu_mlp_packed", "dfk_gate_up_silu_mul_fp8", "dfk_down_proj_fp8", "dfk_swiglu_mlp_fp8",
    "dfk_swiglu_mlp_noalloc", "dfk_stream_read",
)


class DfkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = Status(status) if status in Status._value2member_map_ else status
        super().__init__(f"{where}: {status_string(status)}")


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(
            f"{LIBRARY} is not built; run `python -m swiglu_mlp_amd.build` "
            "(the HIP library is required: there is no fallback path)")
    L = ctypes.CDLL(LIBRARY)
    vp, i, u16p, f32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    L.dfk_gate_up_silu_mul.argtypes = [u16p, u16p, u16p, f32p, i, i, i, i, vp]
    L.dfk_gate_up_silu_mul.restype = i
    L.dfk_down_proj.argtypes = [f32p, u16p, u16p, i, i, i, i, vp]
    L.dfk_down_proj.restype = i
    L.dfk_swiglu_mlp.argtypes = [u16p, u16p, u16p, u16p, u16p, i, i, i, i, vp]
    L.dfk_swiglu_mlp.restype = i
    L.dfk_swiglu_mlp_noalloc.argtypes = [u16p, u16p, u16p, u16p, u16p, i, i, i, i, vp]
    L.dfk_swiglu_mlp_noalloc.restype = i
    L.dfk_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    L.dfk_stream_read.restype = i
    L.dfk_schedule_select.argtypes = [i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    L.dfk_schedule_select.restype = i
    L.dfk_status_string.argtypes = [i]
    L.dfk_status_string.restype = ctypes.c_char_p
    L.dfk_layout_name.argtypes = [i]
    L.dfk_layout_name.restype = ctypes.c_char_p
    L.dfk_version.argtypes = []
    L.dfk_version.restype = ctypes.c_char_p
    L.dfk_load_tuning_table.argtypes = [ctypes.c_char_p]
    L.dfk_load_tuning_table.restype = i
    L.dfk_tuning_table_source.argtypes = []
    L.dfk_tuning_table_source.restype = ctypes.c_char_p
    L.dfk_release_workspace.argtypes = []
    L.dfk_release_workspace.restype = i
    d = ctypes.c_double
    L.dfk_rmsnorm.argtypes = [u16p, u16p, d, u16p, i, i, vp]
    L.dfk_rmsnorm.restype = i
    L.dfk_rmsnorm_gate_up_silu_mul.argtypes = [u16p, u16p, d, u16p, u16p, f32p, i, i, i, i, vp]
    L.dfk_rmsnorm_gate_up_silu_mul.restype = i
    L.dfk_rmsnorm_swiglu_mlp.argtypes = [u16p, u16p, d, u16p, u16p, u16p, u16p, i, i, i, i, vp]
    L.dfk_rmsnorm_swiglu_mlp.restype = i
    L.dfk_gate_up_silu_mul_packed.argtypes = [u16p, u16p, f32p, i, i, i, i, i, vp]
    L.dfk_gate_up_silu_mul_packed.restype = i
    L.dfk_swiglu_mlp_packed.argtypes = [u16p, u16p, u16p, u16p, i, i, i, i, i, vp]
    L.dfk_swiglu_mlp_packed.restype = i
    L.dfk_gate_up_silu_mul_fp8.argtypes = [u16p, vp, vp, vp, vp, f32p, i, i, i, i, vp]
    L.dfk_gate_up_silu_mul_fp8.restype = i
    L.dfk_down_proj_fp8.argtypes = [f32p, vp, vp, u16p, i, i, i, i, vp]
    L.dfk_down_proj_fp8.restype = i
    L.dfk_swiglu_mlp_fp8.argtypes = [u16p, vp, vp, vp, vp, vp, vp, u16p, i, i, i, i, vp]
    L.dfk_swiglu_mlp_fp8.restype = i
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().dfk_status_string(int(status)).decode()


def layout_name(layout: int) -> str:
    return lib().dfk_layout_name(int(layout)).decode()


def version() -> str:
    return lib().dfk_version().decode()


def _check(status: int, where: str) -> None:
    if status != Status.OK:
        raise DfkError(status, where)


def _stream_handle(stream, device) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _expect(t, name: str, dtype, shape) -> None:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def dfk_gate_up_silu_mul(x, W_gate, W_up, h=None, layout: int = Layout.AUTO, stream=None):
    """h = SiLU(x W_gate^T) * (x W_up^T) in fp32, one fused kernel."""
    import torch
    B, d_model = x.shape
    d_ff = W_gate.shape[0]
    _expect(x, "x", torch.bfloat16, (B, d_model))
    _expect(W_gate, "W_gate", torch.bfloat16, (d_ff, d_model))
    _expect(W_up, "W_up", torch.bfloat16, (d_ff, d_model))
    if h is None:
        h = torch.empty((B, d_ff), dtype=torch.float32, device=x.device)
    _expect(h, "h", torch.float32, (B, d_ff))
    st = lib().dfk_gate_up_silu_mul(x.data_ptr(), W_gate.data_ptr(), W_up.data_ptr(), h.data_ptr(),
                                    B, d_model, d_ff, int(layout), _stream_handle(stream, x.device))
    _check(st, "dfk_gate_up_silu_mul")
    return h


def dfk_down_proj(h, W_down, out=None, layout: int = Layout.AUTO, stream=None):
    """out = bf16_RNE(h W_down^T), a separate kernel."""
    import torch
    B, d_ff = h.shape
    d_model = W_down.shape[0]
    _expect(h, "h", torch.float32, (B, d_ff))
    _expect(W_down, "W_down", torch.bfloat16, (d_model, d_ff))
    if out is None:
        out = torch.empty((B, d_model), dtype=torch.bfloat16, device=h.device)
    _expect(out, "out", torch.bfloat16, (B, d_model))
    st = lib().dfk_down_proj(h.data_ptr(), W_down.data_ptr(), out.data_ptr(), B, d_model, d_ff,
                             int(layout), _stream_handle(stream, h.device))
    _check(st, "dfk_down_proj")
    return out


def dfk_swiglu_mlp(x, W_gate, W_up, W_down, out=None, layout: int = Layout.AUTO, stream=None):
    """The whole MLP: fused gate-up kernel, then the down-projection kernel."""
    import torch
    B, d_model = x.shape
    d_ff = W_gate.shape[0]
    _expect(x, "x", torch.bfloat16, (B, d_model))
    _expect(W_gate, "W_gate", torch.bfloat16, (d_ff, d_model))
    _expect(W_up, "W_up", torch.bfloat16, (d_ff, d_model))
    _expect(W_down, "W_down", torch.bfloat16, (d_model, d_ff))
    if out is None:
        out = torch.empty((B, d_model), dtype=torch.bfloat16, device=x.device)
    _expect(out, "out", torch.bfloat16, (B, d_model))
    st = lib().dfk_swiglu_mlp(x.data_ptr(), W_gate.data_ptr(), W_up.data_ptr(), W_down.data_ptr(),
                              out.data_ptr(), B, d_model, d_ff, int(layout),
                              _stream_handle(stream, x.device))
    _check(st, "dfk_swiglu_mlp")
    return out


def dfk_swiglu_mlp_noalloc(x, W_gate, W_up, W_down, out, layout: int = Layout.AUTO, stream=None):
    """dfk_swiglu_mlp with h and the split sums in the library's static device
    scratch: the library allocates nothing (the caller passes `out`)."""
    import torch
    B, d_model = x.shape
    d_ff = W_gate.shape[0]
    _expect(x, "x", torch.bfloat16, (B, d_model))
    _expect(W_gate, "W_gate", torch.bfloat16, (d_ff, d_model))
    _expect(W_up, "W_up", torch.bfloat16, (d_ff, d_model))
    _expect(W_down, "W_down", torch.bfloat16, (d_model, d_ff))
    _expect(out, "out", torch.bfloat16, (B, d_model))
    st = lib().dfk_swiglu_mlp_noalloc(x.data_ptr(), W_gate.data_ptr(), W_up.data_ptr(), W_down.data_ptr(),
                                      out.data_ptr(), B, d_model, d_ff, int(layout),
                                      _stream_handle(stream, x.device))
    _check(st, "dfk_swiglu_mlp_noalloc")
    return out


def dfk_stream_read(buf, sink, nbytes: Optional[int] = None, stream=None) -> None:
    """Measurement helper: one plain streaming read of `nbytes` (default: all)
    of the device tensor `buf`; `sink` is a device tensor of >= 64 int32."""
    import torch
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    if not isinstance(sink, torch.Tensor) or sink.device.type != "cuda" or sink.numel() * sink.element_size() < 256:
        raise ValueError("sink must be a GPU tensor of at least 256 bytes")
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if n > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    _check(lib().dfk_stream_read(buf.data_ptr(), n, sink.data_ptr(), _stream_handle(stream, buf.device)),
           "dfk_stream_read")


def dfk_gate_up_silu_mul_packed(x, W_gu, packing: int, h=None, layout: int = Layout.AUTO, stream=None):
    """dfk_gate_up_silu_mul with W_gate and W_up packed in W_gu [2 d_ff, d_model]."""
    import torch
    B, d_model = x.shape
    d_ff = W_gu.shape[0] // 2
    _expect(x, "x", torch.bfloat16, (B, d_model))
    _expect(W_gu, "W_gu", torch.bfloat16, (2 * d_ff, d_model))
    if h is None:
        h = torch.empty((B, d_ff), dtype=torch.float32, device=x.device)
    _expect(h, "h", torch.float32, (B, d_ff))
    st = lib().dfk_gate_up_silu_mul_packed(x.data_ptr(), W_gu.data_ptr(), h.data_ptr(), B, d_model, d_ff,
                                           int(packing), int(layout), _stream_handle(stream, x.device))
    _check(st, "dfk_gate_up_silu_mul_packed")
    return h


def dfk_swiglu_mlp_packed(x, W_gu, W_down, packing: int, out=None, layout: int = Layout.AUTO, stream=None):
    """dfk_swiglu_mlp with W_gate and W_up packed in W_gu [2 d_ff, d_model]."""
    import torch
    B, d_model = x.shape
    d_ff = W_gu.shape[0] // 2
    _expect(x, "x", torch.bfloat16, (B, d_model))
    _expect(W_gu, "W_gu", torch.bfloat16, (2 * d_ff, d_model))
    _expect(W_down, "W_down", torch.bfloat16, (d_model, d_ff))
    if out is None:
        out = torch.empty((B, d_model), dtype=torch.bfloat16, device=x.device)
    _expect(out, "out", torch.bfloat16, (B, d_model))
    st = lib().dfk_swiglu_mlp_packed(x.data_ptr(), W_gu.data_ptr(), W_down.data_ptr(), out.data_ptr(), B,
                                     d_model, d_ff, int(packing), int(layout), _stream_handle(stream, x.device))
    _check(st, "dfk_swiglu_mlp_packed")
    return out


def _expect_fp8(q, s, name: str, rows: int, cols: int) -> None:
    import torch
    _expect_codes(q, name, (rows, cols))
    _expect(s, name.replace("q", "s", 1), torch.float32, (rows,))


def _expect_codes(q, name: str, shape) -> None:
    import torch
    if not isinstance(q, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if q.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn), got {q.dtype}")
    if q.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {q.device}")
    if tuple(q.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(q.shape)}")
    if not q.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def dfk_gate_up_silu_mul_fp8(x, q_gate, s_gate, q_up, s_up, h=None, layout: int = Layout.AUTO, stream=None):
    """h = SiLU(x W_gate^T) * (x W_up^T) with W = s[row] * e4m3(q), one fused kernel."""
    import torch
    B, d_model = x.shape
    d_ff = q_gate.shape[0]
    _expect(x, "x", torch.bfloat16, (B, d_model))
    _expect_fp8(q_gate, s_gate, "q_gate", d_ff, d_model)
    _expect_fp8(q_up, s_up, "q_up", d_ff, d_model)
    if h is None:
        h = torch.empty((B, d_ff), dtype=torch.float32, device=x.device)
    _expect(h, "h", torch.float32, (B, d_ff))
    st = lib().dfk_gate_up_silu_mul_fp8(x.data_ptr(), q_gate.data_ptr(), s_gate.data_ptr(), q_up.data_ptr(),
                                        s_up.data_ptr(), h.data_ptr(), B, d_model, d_ff, int(layout),
                                        _stream_handle(stream, x.device))
    _check(st, "dfk_gate_up_silu_mul_fp8")
    return h


def dfk_down_proj_fp8(h, q_down, s_down, out=None, layout: int = Layout.AUTO, stream=None):
    """out = bf16_RNE(h W_down^T) with W_down = s[row] * e4m3(q)."""
    import torch
    B, d_ff = h.shape
    d_model = q_down.shape[0]
    _expect(h, "h", torch.float32, (B, d_ff))
    _expect_fp8(q_down, s_down, "q_down", d_model, d_ff)
    if out is None:
        out = torch.empty((B, d_model), dtype=torch.bfloat16, device=h.device)
    _expect(out, "out", torch.bfloat16, (B, d_model))
    st = lib().dfk_down_proj_fp8(h.data_ptr(), q_down.data_ptr(), s_down.data_ptr(), out.data_ptr(), B, d_model,
                                 d_ff, int(layout), _stream_handle(stream, h.device))
    _check(st, "dfk_down_proj_fp8")
    return out


def dfk_swiglu_mlp_fp8(x, q_gate, s_gate, q_up, s_up, q_down, s_down, out=None, layout: int = Layout.AUTO,
                       stream=None):
    """The whole MLP over FP8 weights (two kernels)."""
    import torch
    B, d_model = x.shape
    d_ff = q_gate.shape[0]
    _expect(x, "x", torch.bfloat16, (B, d_model))
    _expect_fp8(q_gate, s_gate, "q_gate", d_ff, d_model)
    _expect_fp8(q_up, s_up, "q_up", d_ff, d_model)
    _expect_fp8(q_down, s_down, "q_down", d_model, d_ff)
    if out is None:
        out = torch.empty((B, d_model), dtype=torch.bfloat16, device=x.device)
    _expect(out, "out", torch.bfloat16, (B, d_model))
    st = lib().dfk_swiglu_mlp_fp8(x.data_ptr(), q_gate.data_ptr(), s_gate.data_ptr(), q_up.data_ptr(),
                                  s_up.data_ptr(), q_down.data_ptr(), s_down.data_ptr(), out.data_ptr(), B,
                                  d_model, d_ff, int(layout), _stream_handle(stream, x.device))
    _check(st, "dfk_swiglu_mlp_fp8")
    return out


def pack_gate_up(W_gate, W_up, packing: int):
    """Pack two [d_ff, d_model] tensors into one [2 d_ff, d_model] (a copy)."""
    import torch
    if int(packing) == Packing.BLOCKED:
        return torch.cat([W_gate, W_up], dim=0).contiguous()
    if int(packing) == Packing.INTERLEAVED:
        return torch.stack([W_gate, W_up], dim=1).reshape(-1, W_gate.shape[1]).contiguous()
    raise ValueError(f"unknown packing {packing}")


def dfk_rmsnorm(x, gain, eps: float = 1e-5, out=None, stream=None):
    """out = bf16_RNE((x * inv) * gain), inv = 1/sqrt(mean(x^2) + eps) per row."""
    import torch
    B, d_model = x.shape
    _expect(x, "x", torch.bfloat16, (B, d_model))
    _expect(gain, "gain", torch.bfloat16, (d_model,))
    if out is None:
        out = torch.empty((B, d_model), dtype=torch.bfloat16, device=x.device)
    _expect(out, "out", torch.bfloat16, (B, d_model))
    st = lib().dfk_rmsnorm(x.data_ptr(), gain.data_ptr(), float(eps), out.data_ptr(), B, d_model,
                           _stream_handle(stream, x.device))
    _check(st, "dfk_rmsnorm")
    return out


def dfk_rmsnorm_gate_up_silu_mul(x, gain, eps: float, W_gate, W_up, h=None, layout: int = Layout.AUTO,
                                 stream=None):
    """h = SiLU(xn W_gate^T) * (xn W_up^T), xn the RMS normalization of x."""
    import torch
    B, d_model = x.shape
    d_ff = W_gate.shape[0]
    _expect(x, "x", torch.bfloat16, (B, d_model))
    _expect(gain, "gain", torch.bfloat16, (d_model,))
    _expect(W_gate, "W_gate", torch.bfloat16, (d_ff, d_model))
    _expect(W_up, "W_up", torch.bfloat16, (d_ff, d_model))
    if h is None:
        h = torch.empty((B, d_ff), dtype=torch.float32, device=x.device)
    _expect(h, "h", torch.float32, (B, d_ff))
    st = lib().dfk_rmsnorm_gate_up_silu_mul(x.data_ptr(), gain.data_ptr(), float(eps), W_gate.data_ptr(),
                                            W_up.data_ptr(), h.data_ptr(), B, d_model, d_ff, int(layout),
                                            _stream_handle(stream, x.device))
    _check(st, "dfk_rmsnorm_gate_up_silu_mul")
    return h


def dfk_rmsnorm_swiglu_mlp(x, gain, eps: float, W_gate, W_up, W_down, out=None, layout: int = Layout.AUTO,
                           stream=None):
    """The whole MLP on the RMS-normalized input."""
    import torch
    B, d_model = x.shape
    d_ff = W_gate.shape[0]
    _expect(x, "x", torch.bfloat16, (B, d_model))
    _expect(gain, "gain", torch.bfloat16, (d_model,))
    _expect(W_gate, "W_gate", torch.bfloat16, (d_ff, d_model))
    _expect(W_up, "W_up", torch.bfloat16, (d_ff, d_model))
    _expect(W_down, "W_down", torch.bfloat16, (d_model, d_ff))
    if out is None:
        out = torch.empty((B, d_model), dtype=torch.bfloat16, device=x.device)
    _expect(out, "out", torch.bfloat16, (B, d_model))
    st = lib().dfk_rmsnorm_swiglu_mlp(x.data_ptr(), gain.data_ptr(), float(eps), W_gate.data_ptr(),
                                      W_up.data_ptr(), W_down.data_ptr(), out.data_ptr(), B, d_model, d_ff,
                                      int(layout), _stream_handle(stream, x.device))
    _check(st, "dfk_rmsnorm_swiglu_mlp")
    return out


def dfk_schedule_select(B: int, d_model: int, d_ff: int) -> Tuple[Layout, Layout]:
    """The scheduler's (gate_up, down) variants for a shape (host only)."""
    g, d = ctypes.c_int(0), ctypes.c_int(0)
    st = lib().dfk_schedule_select(int(B), int(d_model), int(d_ff), ctypes.byref(g), ctypes.byref(d))
    _check(st, "dfk_schedule_select")
    return Layout(g.value), Layout(d.value)


def dfk_load_tuning_table(path: Optional[str] = None) -> None:
    st = lib().dfk_load_tuning_table(path.encode() if path is not None else None)
    _check(st, "dfk_load_tuning_table")


def dfk_tuning_table_source() -> str:
    return lib().dfk_tuning_table_source().decode()


def dfk_release_workspace() -> None:
    _check(lib().dfk_release_workspace(), "dfk_release_workspace")
