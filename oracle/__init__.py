"""CPU oracle for fused block-Hadamard rotation + NVFP4 activation quantization.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library and
its Python binding never import, load or call it.

This is a thin ctypes layer over ``libnvfp4oracle.so`` (built from
``nvfp4_oracle.c`` next to this file), which holds the arithmetic: plain scalar
binary32 C following the page "A Fused Hadamard + NVFP4 Quantization Kernel in
Triton", sections 1-3.  See the header of ``nvfp4_oracle.c`` for the readings
taken where the page leaves a step open.

Inputs: bf16 tensors as ``numpy.uint16`` bit patterns, fp32 as
``numpy.float32``; shape [rows, cols] with cols % 16 == 0.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4oracle.so")
_lib = None

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p
_int = ctypes.c_int
_f32 = ctypes.c_float
_u32 = ctypes.c_uint32


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.oracle_rotate16.argtypes = [_ptr, _ptr]
    lib.oracle_e2m1_code.argtypes = [_f32]
    lib.oracle_e2m1_code.restype = ctypes.c_uint8
    lib.oracle_e4m3_byte.argtypes = [_f32]
    lib.oracle_e4m3_byte.restype = ctypes.c_uint8
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = _f32
    lib.oracle_global_scale.argtypes = [_f32]
    lib.oracle_global_scale.restype = _f32
    lib.oracle_amax.argtypes = [_ptr, _int, _i64, _i64, _int, _int]
    lib.oracle_amax.restype = _f32
    lib.oracle_quantize.argtypes = [_ptr, _int, _i64, _i64, _int, _ptr, _ptr, _ptr, _ptr, _int]
    lib.oracle_quantize.restype = _int
    lib.oracle_quantize_given_scale.argtypes = [_ptr, _int, _i64, _i64, _int, _f32, _ptr,
                                                _ptr, _int]
    lib.oracle_quantize_given_scale.restype = _int
    lib.oracle_dequant_f64.argtypes = [_ptr, _ptr, _f32, _i64, _i64, _int, _ptr, _int]
    lib.oracle_roundtrip_error.argtypes = [_ptr, _int, _i64, _i64, _int, _ptr, _ptr, _f32,
                                           _ptr, _int]
    lib.oracle_roundtrip_error.restype = ctypes.c_double
    lib.oracle_e2m1_code_array.argtypes = [_ptr, _i64, _ptr, _int]
    lib.oracle_e4m3_byte_array.argtypes = [_ptr, _i64, _ptr, _int]
    lib.oracle_e2m1_code_bits.argtypes = [_u32, _u32, _ptr, _int]
    lib.oracle_e8m0_byte.argtypes = [_f32]
    lib.oracle_e8m0_byte.restype = ctypes.c_uint8
    lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_value.restype = _f32
    lib.oracle_mx_quantize.argtypes = [_ptr, _int, _i64, _i64, _int, _ptr, _ptr, _int]
    lib.oracle_mx_quantize.restype = _int
    lib.oracle_mx_roundtrip_error.argtypes = [_ptr, _int, _i64, _i64, _int, _ptr, _ptr, _int]
    lib.oracle_mx_roundtrip_error.restype = ctypes.c_double
    lib.oracle_swizzled_scale_bytes.argtypes = [_i64, _i64]
    lib.oracle_swizzled_scale_bytes.restype = _i64
    lib.oracle_swizzle_scales.argtypes = [_ptr, _i64, _i64, _ptr]
    lib.oracle_rotate_tensor.argtypes = [_ptr, _int, _i64, _i64, _ptr, _int]
    lib.oracle_rotate_tensor.restype = _int
    lib.oracle_rotate_matrix.argtypes = [_ptr, _int, _i64, _i64, _ptr, _ptr, _int]
    lib.oracle_rotate_matrix.restype = _int
    lib.oracle_mx_dequant_f64.argtypes = [_ptr, _ptr, _i64, _i64, _int, _ptr, _int]
    lib.oracle_e4m3_byte_bits.argtypes = [_u32, _u32, _ptr, _int]
    _lib = lib
    return lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _is_f32(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return 1
    if x.dtype == np.uint16:
        return 0
    raise TypeError(f"oracle input must be uint16 (bf16 bits) or float32, got {x.dtype}")


# ---------------------------------------------------------------- element helpers

def rotate16(x: np.ndarray) -> np.ndarray:
    """Block rotation of one 16-vector (binary32 butterfly, strides 1,2,4,8, x0.25)."""
    xi = np.ascontiguousarray(x, dtype=np.float32).reshape(16)
    y = np.empty(16, dtype=np.float32)
    _load().oracle_rotate16(_p(xi), _p(y))
    return y


def rotate_tensor(x: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """rotate16 applied to every 16-element block of x [rows, cols]; float32."""
    rows, cols = x.shape
    y = np.empty((rows, cols), dtype=np.float32)
    if _load().oracle_rotate_tensor(_p(x), _is_f32(x), rows, cols, _p(y), nthreads):
        raise ValueError("cols must be a multiple of 16")
    return y


def rotate_matrix(x: np.ndarray, r: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """y = x_b r for every 16-element block x_b of x [rows, cols] (r: 16 x 16,
    rows are inputs), binary32 with the fused multiply-add order of
    oracle_rotate_matrix; float32."""
    rows, cols = x.shape
    rr = np.ascontiguousarray(r, dtype=np.float32)
    if rr.shape != (16, 16):
        raise ValueError("r must be 16 x 16")
    y = np.empty((rows, cols), dtype=np.float32)
    if _load().oracle_rotate_matrix(_p(x), _is_f32(x), rows, cols, _p(rr), _p(y), nthreads):
        raise ValueError("cols must be a multiple of 16")
    return y


def e2m1_code(v: float) -> int:
    return int(_load().oracle_e2m1_code(float(np.float32(v))))


def e4m3_byte(v: float) -> int:
    return int(_load().oracle_e4m3_byte(float(np.float32(v))))


def e4m3_value(b: int) -> float:
    return float(_load().oracle_e4m3_value(int(b)))


def global_scale(amax: float) -> float:
    return float(np.float32(_load().oracle_global_scale(float(np.float32(amax)))))


def e2m1_codes(v: np.ndarray, nthreads: int = 0) -> np.ndarray:
    vv = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(vv.shape, dtype=np.uint8)
    _load().oracle_e2m1_code_array(_p(vv), vv.size, _p(out), nthreads)
    return out


def e4m3_bytes(v: np.ndarray, nthreads: int = 0) -> np.ndarray:
    vv = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(vv.shape, dtype=np.uint8)
    _load().oracle_e4m3_byte_array(_p(vv), vv.size, _p(out), nthreads)
    return out


def e2m1_codes_bits(lo: int, hi: int, nthreads: int = 0) -> np.ndarray:
    out = np.empty(hi - lo + 1, dtype=np.uint8)
    _load().oracle_e2m1_code_bits(lo, hi, _p(out), nthreads)
    return out


def e4m3_bytes_bits(lo: int, hi: int, nthreads: int = 0) -> np.ndarray:
    out = np.empty(hi - lo + 1, dtype=np.uint8)
    _load().oracle_e4m3_byte_bits(lo, hi, _p(out), nthreads)
    return out


# ---------------------------------------------------------------- tensor level

def amax(x: np.ndarray, rotate: bool, nthreads: int = 0) -> float:
    rows, cols = x.shape
    return float(_load().oracle_amax(_p(x), _is_f32(x), rows, cols, int(rotate), nthreads))


def quantize(x: np.ndarray, rotate: bool, nthreads: int = 0):
    """Returns (q uint8 [rows, cols/2], s uint8 [rows, cols/16], g float32, amax float32)."""
    rows, cols = x.shape
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty((rows, cols // 16), dtype=np.uint8)
    g = ctypes.c_float(0.0)
    a = ctypes.c_float(0.0)
    rc = _load().oracle_quantize(_p(x), _is_f32(x), rows, cols, int(rotate), _p(q), _p(s),
                                 ctypes.addressof(g), ctypes.addressof(a), nthreads)
    if rc:
        raise ValueError("oracle_quantize rejected its arguments")
    return q, s, np.float32(g.value), np.float32(a.value)


def quantize_given_scale(x: np.ndarray, rotate: bool, g: float, nthreads: int = 0):
    rows, cols = x.shape
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty((rows, cols // 16), dtype=np.uint8)
    rc = _load().oracle_quantize_given_scale(_p(x), _is_f32(x), rows, cols, int(rotate),
                                             float(np.float32(g)), _p(q), _p(s), nthreads)
    if rc:
        raise ValueError("oracle_quantize_given_scale rejected its arguments")
    return q, s


def dequant_f64(q: np.ndarray, s: np.ndarray, g: float, rotate: bool,
                nthreads: int = 0) -> np.ndarray:
    rows = s.shape[0]
    cols = s.shape[1] * 16
    out = np.empty((rows, cols), dtype=np.float64)
    _load().oracle_dequant_f64(_p(np.ascontiguousarray(q)), _p(np.ascontiguousarray(s)),
                               float(np.float32(g)), rows, cols, int(rotate), _p(out), nthreads)
    return out


def roundtrip_error(x: np.ndarray, rotate: bool, q: np.ndarray, s: np.ndarray, g: float,
                    col_mask: np.ndarray | None = None, nthreads: int = 0) -> float:
    rows, cols = x.shape
    cm = None
    if col_mask is not None:
        cm = np.ascontiguousarray(col_mask, dtype=np.uint8)
        assert cm.size == cols
    return float(_load().oracle_roundtrip_error(
        _p(x), _is_f32(x), rows, cols, int(rotate), _p(np.ascontiguousarray(q)),
        _p(np.ascontiguousarray(s)), float(np.float32(g)),
        None if cm is None else _p(cm), nthreads))


# ---------------------------------------------------------------- MXFP4 variant

def e8m0_byte(t: float) -> int:
    """Byte of the smallest power of two >= t (exponent clamped to [-127, 127])."""
    return int(_load().oracle_e8m0_byte(float(np.float32(t))))


def e8m0_value(b: int) -> float:
    return float(_load().oracle_e8m0_value(int(b)))


def mx_quantize(x: np.ndarray, rotate: bool, nthreads: int = 0):
    """MXFP4: returns (q uint8 [rows, cols/2], s uint8 [rows, cols/32] E8M0 bytes)."""
    rows, cols = x.shape
    if cols % 32:
        raise ValueError("cols must be a multiple of 32")
    q = np.empty((rows, cols // 2), dtype=np.uint8)
    s = np.empty((rows, cols // 32), dtype=np.uint8)
    rc = _load().oracle_mx_quantize(_p(x), _is_f32(x), rows, cols, int(rotate), _p(q), _p(s),
                                    nthreads)
    if rc:
        raise ValueError("oracle_mx_quantize rejected its arguments")
    return q, s


def mx_roundtrip_error(x: np.ndarray, rotate: bool, q: np.ndarray, s: np.ndarray,
                       nthreads: int = 0) -> float:
    rows, cols = x.shape
    return float(_load().oracle_mx_roundtrip_error(
        _p(x), _is_f32(x), rows, cols, int(rotate), _p(np.ascontiguousarray(q)),
        _p(np.ascontiguousarray(s)), nthreads))


def mx_dequant_f64(q: np.ndarray, s: np.ndarray, rotate: bool, nthreads: int = 0) -> np.ndarray:
    rows = s.shape[0]
    cols = s.shape[1] * 32
    out = np.empty((rows, cols), dtype=np.float64)
    _load().oracle_mx_dequant_f64(_p(np.ascontiguousarray(q)), _p(np.ascontiguousarray(s)),
                                  rows, cols, int(rotate), _p(out), nthreads)
    return out


# ---------------------------------------------------------------- swizzled scales

def swizzled_scale_bytes(rows: int, cb: int) -> int:
    return int(_load().oracle_swizzled_scale_bytes(rows, cb))


def swizzle_scales(s: np.ndarray) -> np.ndarray:
    """Row-major block scales [rows, cols/16] -> the padded 128 x 4-tile layout
    (1-D uint8, zero padding)."""
    ss = np.ascontiguousarray(s, dtype=np.uint8)
    rows, cb = ss.shape
    out = np.empty(swizzled_scale_bytes(rows, cb), dtype=np.uint8)
    _load().oracle_swizzle_scales(_p(ss), rows, cb, _p(out))
    return out
