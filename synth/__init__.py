"""Seeded synthetic activation tensors (shared by the tests and the benchmark).

Only random numbers and their placement live here: no step of the quantizer.
The C library ``libnvfp4synth.so`` (built from ``synth.c`` next to this file)
does the drawing; this module allocates numpy arrays and names the workloads.

bf16 tensors are returned as ``numpy.uint16`` arrays of bf16 bit patterns,
fp32 tensors as ``numpy.float32``.  Every value is a pure function of
(seed, stream, index), so the same call gives the same bytes on every machine
with the same C math library, whatever the thread count.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4synth.so")
_lib = None

_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_ptr = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.synth_normal_bf16.argtypes = [_u64, _u64, _i64, ctypes.c_double, _ptr]
    lib.synth_normal_f32.argtypes = [_u64, _u64, _i64, ctypes.c_double, _ptr]
    lib.synth_normal_f64.argtypes = [_u64, _u64, _u64, _i64, _ptr]
    lib.synth_uniform_f64.argtypes = [_u64, _u64, _u64, _i64, _ptr]
    lib.synth_round_bf16.argtypes = [_ptr, _i64, _ptr]
    lib.synth_gauss_outliers.argtypes = [_u64, _i64, _i64, _i64, ctypes.c_double,
                                         ctypes.c_double, _ptr, _ptr]
    lib.synth_t3_lognormal.argtypes = [_u64, _i64, _i64, _ptr]
    lib.synth_silu_ties.argtypes = [_u64, _i64, _i64, ctypes.c_int, _ptr, _ptr, _ptr, _ptr]
    lib.synth_kv_heads.argtypes = [_u64, _i64, _i64, _i64, _ptr, _ptr]
    for name in ("synth_gauss_outliers", "synth_t3_lognormal", "synth_silu_ties",
                 "synth_kv_heads"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what}: generator rejected its arguments (rc={rc})")


# ---------------------------------------------------------------- primitives

def normal_bf16(n: int, seed: int = 0, stream: int = 0, scale: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_bf16(seed, stream, n, scale, _p(out))
    return out


def normal_f32(n: int, seed: int = 0, stream: int = 0, scale: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(seed, stream, n, scale, _p(out))
    return out


def normal_f64(n: int, seed: int = 0, stream: int = 0, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal_f64(seed, stream, start, n, _p(out))
    return out


def uniform_f64(n: int, seed: int = 0, stream: int = 0, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform_f64(seed, stream, start, n, _p(out))
    return out


def round_bf16(values: np.ndarray) -> np.ndarray:
    """fp64 values -> bf16 bit patterns, one round-to-nearest-even step."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().synth_round_bf16(_p(v), v.size, _p(out))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (a bit shift; no rounding)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- recipes

def gauss_outliers(rows: int, cols: int, n_out: int, lo: float, hi: float, seed: int = 0):
    out = np.empty((rows, cols), dtype=np.uint16)
    picked = np.empty(max(n_out, 1), dtype=np.int64)
    _check(_load().synth_gauss_outliers(seed, rows, cols, n_out, lo, hi, _p(out), _p(picked)),
           "gauss_outliers")
    return out, picked[:n_out].copy()


def t3_lognormal(rows: int, cols: int, seed: int = 0) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    _check(_load().synth_t3_lognormal(seed, rows, cols, _p(out)), "t3_lognormal")
    return out


def silu_ties(rows: int, cols: int, rotate: bool, seed: int = 0):
    out = np.empty((rows, cols), dtype=np.uint16)
    nb = rows * (cols // 16)
    flags = np.empty(max(nb, 1), dtype=np.uint8)
    anchor = ctypes.c_int64(-1)
    nties = ctypes.c_int64(0)
    _check(_load().synth_silu_ties(seed, rows, cols, int(bool(rotate)), _p(out),
                                   ctypes.addressof(anchor), ctypes.addressof(nties),
                                   _p(flags)), "silu_ties")
    return out, int(anchor.value), flags[:nb]


def kv_heads(tokens: int, heads: int, dim: int, seed: int = 0):
    out = np.empty((tokens, heads * dim), dtype=np.float32)
    nb = tokens * heads * dim // 16
    kind = np.empty(max(nb, 1), dtype=np.uint8)
    _check(_load().synth_kv_heads(seed, tokens, heads, dim, _p(out), _p(kind)), "kv_heads")
    return out, kind[:nb]


# ---------------------------------------------------------------- named workloads

def random_orthogonal16(seed: int = 0) -> np.ndarray:
    """A random orthogonal 16 x 16 matrix, binary32: Q of the QR factorisation
    of a seeded standard-normal matrix, each column's sign chosen so that the
    triangular factor has a positive diagonal (the Haar-distributed draw).
    The matrix is an input of the general block rotation; numpy's QR is the
    library routine that draws it."""
    g = normal_f64(256, seed=seed, stream=11).reshape(16, 16)
    q, r = np.linalg.qr(g)
    return (q * np.sign(np.diag(r))).astype(np.float32)


@dataclass
class Workload:
    """One synthetic activation tensor plus the facts its recipe plants."""
    name: str
    x: np.ndarray                # uint16 (bf16 bits) or float32, shape [rows, cols]
    dtype: str                   # "bf16" or "f32"
    rotate: bool
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.x.shape[0]

    @property
    def cols(self) -> int:
        return self.x.shape[1]

    def sha256(self) -> str:
        return hashlib.sha256(self.x.tobytes()).hexdigest()


# The five activation workloads: name -> (rows, cols, dtype, rotate settings).
WORKLOADS = {
    "gauss_outliers_128x1024": (128, 1024, "bf16", (True,)),
    "gauss_1pct_cols_4096x4096": (4096, 4096, "bf16", (True, False)),
    "t3_lognormal_16384x8192": (16384, 8192, "bf16", (True,)),
    "silu_ties_32768x14336": (32768, 14336, "bf16", (False, True)),
    "kv_heads_65536x8x128_f32": (65536, 1024, "f32", (True,)),
}


def make(name: str, rotate: bool | None = None, seed: int = 0, rows: int | None = None) -> Workload:
    """Build a named workload.  `rows` shrinks the row count (same recipe and
    columns) for tests that need a smaller slice of the same distribution."""
    full_rows, cols, dtype, rots = WORKLOADS[name]
    if rotate is None:
        rotate = rots[0]
    r = full_rows if rows is None else rows
    if name.startswith("gauss_outliers"):
        x, picked = gauss_outliers(r, cols, 4, 50.0, 50.0, seed)
        return Workload(name, x, dtype, rotate, {"outlier_cols": picked.tolist()})
    if name.startswith("gauss_1pct_cols"):
        n_out = int(round(0.01 * cols))
        x, picked = gauss_outliers(r, cols, n_out, 10.0, 100.0, seed)
        return Workload(name, x, dtype, rotate, {"outlier_cols": picked.tolist()})
    if name.startswith("t3_lognormal"):
        return Workload(name, t3_lognormal(r, cols, seed), dtype, rotate, {})
    if name.startswith("silu_ties"):
        x, anchor, flags = silu_ties(r, cols, rotate, seed)
        return Workload(name, x, dtype, rotate, {"anchor_block": anchor, "tie_flags": flags})
    if name.startswith("kv_heads"):
        x, kind = kv_heads(r, 8, 128, seed)
        return Workload(name, x, dtype, rotate, {"block_kind": kind})
    raise KeyError(name)
