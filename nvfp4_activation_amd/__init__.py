"""Fused block-Hadamard rotation + NVFP4 activation quantization on MI355X.

Thin ctypes binding over ``libnvfp4rq.so`` (HIP, gfx950), whose C ABI is
declared in ``include/nvfp4rq.h``.  This module only marshals arguments: it
allocates outputs with PyTorch on the input's device, takes the current HIP
stream from PyTorch, and calls the library.  Every step of the method runs in
the library's kernels; there is no fallback path, and importing this module
fails if the library is not built.

Method: page "A Fused Hadamard + NVFP4 Quantization Kernel in Triton",
sections 1-3 (two-level NVFP4 scaling of 16-element blocks after a 16-point
Hadamard rotation).
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

__all__ = [
    "LIB_PATH", "Nvfp4Error", "rotquant", "rotamax", "quant_from_amax", "dequant",
    "status_string", "lib", "mx_rotquant", "mx_dequant",
    "rotate16", "rotate_matrix", "rotquant_timed", "rotquant_swizzled", "dequant_swizzled",
    "swizzled_scale_bytes", "stream_calibrate", "stream_calibrate_single",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4rq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int

_SIGS = {
    "nvfp4_rotquant": [_p, _i64, _i64, _int, _p, _p, _p, _p, _p],
    "nvfp4_rotquant_f32": [_p, _i64, _i64, _int, _p, _p, _p, _p, _p],
    "nvfp4_rotamax": [_p, _i64, _i64, _int, _p, _p],
    "nvfp4_rotamax_f32": [_p, _i64, _i64, _int, _p, _p],
    "nvfp4_quant_from_amax": [_p, _i64, _i64, _int, _p, _p, _p, _p, _p],
    "nvfp4_quant_from_amax_f32": [_p, _i64, _i64, _int, _p, _p, _p, _p, _p],
    "nvfp4_dequant": [_p, _p, _p, _i64, _i64, _int, _p, _p],
    "nvfp4_rotate16": [_p, _i64, _i64, _p, _p],
    "nvfp4_rotate_matrix": [_p, _i64, _i64, _p, _p, _p],
    "nvfp4_rotquant_swizzled": [_p, _i64, _i64, _int, _p, _p, _p, _p, _p],
    "nvfp4_rotquant_timed": [_p, _i64, _i64, _int, _p, _p, _p, _p, _p, _p, _int, _p],
    "nvfp4_rotquant_f32_timed": [_p, _i64, _i64, _int, _p, _p, _p, _p, _p, _p, _int, _p],
    "nvfp4_rotquant_swizzled_f32": [_p, _i64, _i64, _int, _p, _p, _p, _p, _p],
    "nvfp4_dequant_swizzled": [_p, _p, _p, _i64, _i64, _int, _p, _p],
    "nvfp4_rotate16_f32": [_p, _i64, _i64, _p, _p],
    "nvfp4_rotate_matrix_f32": [_p, _i64, _i64, _p, _p, _p],
    "mxfp4_rotquant": [_p, _i64, _i64, _int, _p, _p, _p],
    "mxfp4_rotquant_f32": [_p, _i64, _i64, _int, _p, _p, _p],
    "mxfp4_dequant": [_p, _p, _i64, _i64, _int, _p, _p],
    "nvfp4_stream_calibrate": [_p, _i64, _i64, _p, _p, _p],
    "nvfp4_stream_calibrate_f32": [_p, _i64, _i64, _p, _p, _p],
    "nvfp4_stream_calibrate_single": [_p, _i64, _i64, _p, _p, _p],
    "nvfp4_stream_calibrate_single_f32": [_p, _i64, _i64, _p, _p, _p],
}
for _name, _args in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _int
lib.nvfp4_swizzled_scale_bytes.argtypes = [_i64, _i64]
lib.nvfp4_swizzled_scale_bytes.restype = _i64
lib.nvfp4_status_string.argtypes = [_int]
lib.nvfp4_status_string.restype = ctypes.c_char_p


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def status_string(status: int) -> str:
    return lib.nvfp4_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Nvfp4Error(fn, status)


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    return t.data_ptr() or None


def _stream(device: torch.device, stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _on_device(fn):
    """Run the call with its first tensor's GPU as the current device, so that
    the library sizes its launches for that device and launches there (the
    stream passed down belongs to the same device).  Host tensors go through
    unchanged, to be refused by the call's own checks."""
    @functools.wraps(fn)
    def call(t, *args, **kwargs):
        if isinstance(t, torch.Tensor) and t.is_cuda:
            with torch.cuda.device(t.device):
                return fn(t, *args, **kwargs)
        return fn(t, *args, **kwargs)
    return call


def _variant(x: torch.Tensor, base: str) -> str:
    if x.dtype == torch.bfloat16:
        return base
    if x.dtype == torch.float32:
        return base + "_f32"
    raise TypeError(f"input must be bfloat16 or float32, got {x.dtype}")


def _check_input(x: torch.Tensor, multiple: int = 16) -> tuple[int, int]:
    if x.dim() != 2:
        raise ValueError("input must be 2-D [rows, cols]")
    if x.shape[1] % multiple:
        raise ValueError(f"cols must be a multiple of {multiple}, got {x.shape[1]}")
    if not x.is_cuda:
        raise ValueError("input must be a device tensor")
    if not x.is_contiguous():
        raise ValueError("input must be contiguous (row-major)")
    return x.shape[0], x.shape[1]


def _buf(t, numel: int, dtype: torch.dtype, device: torch.device, name: str) -> torch.Tensor:
    """A caller-supplied buffer: the library receives only its address, so the
    dtype, device, layout and size are checked here, before any launch."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the input on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")
    return t


def _check_out4(x, rows, cols, q, s, g, a, s_numel):
    _buf(q, rows * cols // 2, torch.uint8, x.device, "q")
    _buf(s, s_numel, torch.uint8, x.device, "s")
    _buf(g, 1, torch.float32, x.device, "g")
    _buf(a, 1, torch.float32, x.device, "amax")


def _decode_inputs(q, s, g, s_numel):
    if not q.is_cuda:
        raise ValueError("q must be a device tensor")
    _buf(q, q.numel(), torch.uint8, q.device, "q")
    _buf(s, s_numel, torch.uint8, q.device, "s")
    if g is not None:
        _buf(g, 1, torch.float32, q.device, "g")


@_on_device
def rotamax(x: torch.Tensor, rotate: bool = True, amax: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    """Pass 1: the rotated global amax, as a float32 device tensor [1]."""
    rows, cols = _check_input(x)
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=x.device)
    _buf(amax, 1, torch.float32, x.device, "amax")
    fn = _variant(x, "nvfp4_rotamax")
    _check(fn, getattr(lib, fn)(_ptr(x), rows, cols, int(bool(rotate)), _ptr(amax),
                                _stream(x.device, stream)))
    return amax


@_on_device
def quant_from_amax(x: torch.Tensor, amax: torch.Tensor, rotate: bool = True,
                    out: tuple | None = None, stream=None):
    """Pass 2: global scale from a device amax, then rotate+quantize.
    Returns (q uint8 [rows, cols/2], s uint8 [rows, cols/16], g float32 [1])."""
    rows, cols = _check_input(x)
    if out is None:
        q = torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device)
        s = torch.empty(rows, cols // 16, dtype=torch.uint8, device=x.device)
        g = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        q, s, g = out
    _buf(amax, 1, torch.float32, x.device, "amax")
    _buf(q, rows * cols // 2, torch.uint8, x.device, "q")
    _buf(s, rows * cols // 16, torch.uint8, x.device, "s")
    _buf(g, 1, torch.float32, x.device, "g")
    fn = _variant(x, "nvfp4_quant_from_amax")
    _check(fn, getattr(lib, fn)(_ptr(x), rows, cols, int(bool(rotate)), _ptr(amax), _ptr(q),
                                _ptr(s), _ptr(g), _stream(x.device, stream)))
    return q, s, g


@_on_device
def rotquant(x: torch.Tensor, rotate: bool = True, out: tuple | None = None, stream=None):
    """Both passes.  x: bfloat16 or float32 [rows, cols], cols % 16 == 0.
    Returns (q uint8 [rows, cols/2], s uint8 [rows, cols/16] E4M3FN bytes,
    g float32 [1] global scale, amax float32 [1])."""
    rows, cols = _check_input(x)
    if out is None:
        q = torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device)
        s = torch.empty(rows, cols // 16, dtype=torch.uint8, device=x.device)
        g = torch.empty(1, dtype=torch.float32, device=x.device)
        a = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        q, s, g, a = out
    _check_out4(x, rows, cols, q, s, g, a, rows * cols // 16)
    fn = _variant(x, "nvfp4_rotquant")
    _check(fn, getattr(lib, fn)(_ptr(x), rows, cols, int(bool(rotate)), _ptr(q), _ptr(s),
                                _ptr(g), _ptr(a), _stream(x.device, stream)))
    return q, s, g, a


@_on_device
def rotquant_timed(x: torch.Tensor, events: list, rotate: bool = True, out: tuple | None = None,
                   stream=None):
    """rotquant with each launched kernel timed in place: events is a list of
    torch.cuda.Event(enable_timing=True), each recorded once already; kernel k
    records events[2k] and events[2k+1].  Returns (q, s, g, amax, number of
    kernels launched)."""
    rows, cols = _check_input(x)
    if out is None:
        q = torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device)
        s = torch.empty(rows, cols // 16, dtype=torch.uint8, device=x.device)
        g = torch.empty(1, dtype=torch.float32, device=x.device)
        a = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        q, s, g, a = out
    _check_out4(x, rows, cols, q, s, g, a, rows * cols // 16)
    if len(events) < 2 or len(events) % 2:
        raise ValueError("events must hold start/stop pairs")
    handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    nk = ctypes.c_int(0)
    fn = "nvfp4_rotquant_timed" if x.dtype == torch.bfloat16 else _variant(x, "nvfp4_rotquant") + "_timed"
    _check(fn, getattr(lib, fn)(
        _ptr(x), rows, cols, int(bool(rotate)), _ptr(q), _ptr(s), _ptr(g), _ptr(a),
        _stream(x.device, stream), handles, len(events) // 2, ctypes.byref(nk)))
    return q, s, g, a, nk.value


@_on_device
def dequant(q: torch.Tensor, s: torch.Tensor, g: torch.Tensor, rotate: bool = True,
            out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode codes and scales back to float32 [rows, cols] (inverse rotation
    included when rotate)."""
    if s.dim() != 2 or q.dim() != 2:
        raise ValueError("q and s must be 2-D")
    rows, cols = s.shape[0], s.shape[1] * 16
    if q.shape != (rows, cols // 2):
        raise ValueError("q and s shapes disagree")
    _decode_inputs(q, s, g, s.numel())
    if out is None:
        out = torch.empty(rows, cols, dtype=torch.float32, device=q.device)
    _buf(out, rows * cols, torch.float32, q.device, "out")
    _check("nvfp4_dequant", lib.nvfp4_dequant(_ptr(q), _ptr(s), _ptr(g), rows, cols,
                                              int(bool(rotate)), _ptr(out),
                                              _stream(q.device, stream)))
    return out


def swizzled_scale_bytes(rows: int, cols: int) -> int:
    n = int(lib.nvfp4_swizzled_scale_bytes(rows, cols))
    if n < 0:
        raise ValueError(f"no swizzled scale layout for shape ({rows}, {cols})")
    return n


@_on_device
def rotquant_swizzled(x: torch.Tensor, rotate: bool = True, out: tuple | None = None, stream=None):
    """rotquant with the block scales in the 128 x 4-tile swizzled layout.
    Returns (q uint8 [rows, cols/2], s uint8 [swizzled_scale_bytes], g, amax)."""
    rows, cols = _check_input(x)
    if out is None:
        q = torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device)
        s = torch.empty(swizzled_scale_bytes(rows, cols), dtype=torch.uint8, device=x.device)
        g = torch.empty(1, dtype=torch.float32, device=x.device)
        a = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        q, s, g, a = out
    _check_out4(x, rows, cols, q, s, g, a, swizzled_scale_bytes(rows, cols))
    fn = _variant(x, "nvfp4_rotquant_swizzled")
    _check(fn, getattr(lib, fn)(_ptr(x), rows, cols, int(bool(rotate)), _ptr(q), _ptr(s),
                                _ptr(g), _ptr(a), _stream(x.device, stream)))
    return q, s, g, a


@_on_device
def dequant_swizzled(q: torch.Tensor, s: torch.Tensor, g: torch.Tensor, rotate: bool = True,
                     out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    if q.dim() != 2:
        raise ValueError("q must be 2-D [rows, cols/2]")
    rows, cols = q.shape[0], q.shape[1] * 2
    _decode_inputs(q, s, g, swizzled_scale_bytes(rows, cols))
    if out is None:
        out = torch.empty(rows, cols, dtype=torch.float32, device=q.device)
    _buf(out, rows * cols, torch.float32, q.device, "out")
    _check("nvfp4_dequant_swizzled", lib.nvfp4_dequant_swizzled(
        _ptr(q), _ptr(s), _ptr(g), rows, cols, int(bool(rotate)), _ptr(out),
        _stream(q.device, stream)))
    return out


@_on_device
def rotate16(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The block rotation alone: float32 [rows, cols] = x H16 per 16-element block."""
    rows, cols = _check_input(x)
    if out is None:
        out = torch.empty(rows, cols, dtype=torch.float32, device=x.device)
    _buf(out, rows * cols, torch.float32, x.device, "out")
    fn = _variant(x, "nvfp4_rotate16")
    _check(fn, getattr(lib, fn)(_ptr(x), rows, cols, _ptr(out), _stream(x.device, stream)))
    return out


@_on_device
def rotate_matrix(x: torch.Tensor, r: torch.Tensor, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """General block rotation: float32 [rows, cols] = x R per 16-element block.
    r: float32 [16, 16] on x's device, row k multiplying input k."""
    rows, cols = _check_input(x)
    _buf(r, 256, torch.float32, x.device, "r")
    if out is None:
        out = torch.empty(rows, cols, dtype=torch.float32, device=x.device)
    _buf(out, rows * cols, torch.float32, x.device, "out")
    fn = _variant(x, "nvfp4_rotate_matrix")
    _check(fn, getattr(lib, fn)(_ptr(x), rows, cols, _ptr(r), _ptr(out),
                                _stream(x.device, stream)))
    return out


@_on_device
def mx_rotquant(x: torch.Tensor, rotate: bool = True, out: tuple | None = None, stream=None):
    """MXFP4 single pass.  x: bfloat16 or float32 [rows, cols], cols % 32 == 0.
    Returns (q uint8 [rows, cols/2], s uint8 [rows, cols/32] E8M0 bytes)."""
    rows, cols = _check_input(x, 32)
    if out is None:
        q = torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device)
        s = torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device)
    else:
        q, s = out
    _buf(q, rows * cols // 2, torch.uint8, x.device, "q")
    _buf(s, rows * cols // 32, torch.uint8, x.device, "s")
    fn = _variant(x, "mxfp4_rotquant")
    _check(fn, getattr(lib, fn)(_ptr(x), rows, cols, int(bool(rotate)), _ptr(q), _ptr(s),
                                _stream(x.device, stream)))
    return q, s


@_on_device
def mx_dequant(q: torch.Tensor, s: torch.Tensor, rotate: bool = True,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    if s.dim() != 2 or q.dim() != 2:
        raise ValueError("q and s must be 2-D")
    rows, cols = s.shape[0], s.shape[1] * 32
    if q.shape != (rows, cols // 2):
        raise ValueError("q and s shapes disagree")
    _decode_inputs(q, s, None, s.numel())
    if out is None:
        out = torch.empty(rows, cols, dtype=torch.float32, device=q.device)
    _buf(out, rows * cols, torch.float32, q.device, "out")
    _check("mxfp4_dequant", lib.mxfp4_dequant(_ptr(q), _ptr(s), rows, cols, int(bool(rotate)),
                                              _ptr(out), _stream(q.device, stream)))
    return out


@_on_device
def stream_calibrate(x: torch.Tensor, out: tuple | None = None, stream=None):
    """Measurement support: the fused call's launch sequence with no-arithmetic
    twins of its two kernels (same grids, access patterns and bytes).  Returns
    (q, s) holding meaningless bytes."""
    return _calibrate("nvfp4_stream_calibrate", x, out, stream)


@_on_device
def stream_calibrate_single(x: torch.Tensor, out: tuple | None = None, stream=None):
    """Measurement support: the no-arithmetic twin launched as one pass with a
    workgroup per chunk (the given-scale pass's launch shape).  Returns (q, s)
    holding meaningless bytes."""
    return _calibrate("nvfp4_stream_calibrate_single", x, out, stream)


def _calibrate(name: str, x: torch.Tensor, out, stream):
    rows, cols = _check_input(x)
    if out is None:
        q = torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device)
        s = torch.empty(rows, cols // 16, dtype=torch.uint8, device=x.device)
    else:
        q, s = out
    _buf(q, rows * cols // 2, torch.uint8, x.device, "q")
    _buf(s, rows * cols // 16, torch.uint8, x.device, "s")
    fn = _variant(x, name)
    _check(fn, getattr(lib, fn)(_ptr(x), rows, cols, _ptr(q), _ptr(s), _stream(x.device, stream)))
    return q, s
