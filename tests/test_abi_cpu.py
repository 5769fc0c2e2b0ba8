"""The C ABI on the CPU: the library loads, exports every declared entry point,
and rejects bad arguments before any HIP call (validation is host-only, so
these calls never touch a device and run without a GPU)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "nvfp4rq.h")
LIB = os.path.join(ROOT, "nvfp4_activation_amd", "libnvfp4rq.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_ARG, ERR_HIP = range(6)


def declared_functions() -> list[str]:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:nvfp4|mxfp4)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    lib = ctypes.CDLL(LIB)
    p, i64, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    for name in ("nvfp4_rotquant", "nvfp4_rotquant_f32", "nvfp4_quant_from_amax",
                 "nvfp4_quant_from_amax_f32"):
        getattr(lib, name).argtypes = [p, i64, i64, i, p, p, p, p, p]
    for name in ("nvfp4_rotamax", "nvfp4_rotamax_f32"):
        getattr(lib, name).argtypes = [p, i64, i64, i, p, p]
    lib.nvfp4_dequant.argtypes = [p, p, p, i64, i64, i, p, p]
    for name in ("mxfp4_rotquant", "mxfp4_rotquant_f32"):
        getattr(lib, name).argtypes = [p, i64, i64, i, p, p, p]
    lib.mxfp4_dequant.argtypes = [p, p, i64, i64, i, p, p]
    for name in ("nvfp4_rotate16", "nvfp4_rotate16_f32"):
        getattr(lib, name).argtypes = [p, i64, i64, p, p]
    for name in ("nvfp4_rotate_matrix", "nvfp4_rotate_matrix_f32"):
        getattr(lib, name).argtypes = [p, i64, i64, p, p, p]
    for name in ("nvfp4_rotquant_swizzled", "nvfp4_rotquant_swizzled_f32"):
        getattr(lib, name).argtypes = [p, i64, i64, i, p, p, p, p, p]
    lib.nvfp4_dequant_swizzled.argtypes = [p, p, p, i64, i64, i, p, p]
    for name in ("nvfp4_rotquant_timed", "nvfp4_rotquant_f32_timed"):
        getattr(lib, name).argtypes = [p, i64, i64, i, p, p, p, p, p, p, i, p]
    lib.nvfp4_swizzled_scale_bytes.argtypes = [i64, i64]
    lib.nvfp4_swizzled_scale_bytes.restype = i64
    for name in ("nvfp4_stream_calibrate", "nvfp4_stream_calibrate_f32", "nvfp4_stream_calibrate_single",
                 "nvfp4_stream_calibrate_single_f32"):
        getattr(lib, name).argtypes = [p, i64, i64, p, p, p]
    lib.nvfp4_status_string.argtypes = [i]
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    return lib


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("nvfp4_rotquant", "nvfp4_rotquant_f32", "nvfp4_dequant",
                 "nvfp4_status_string", "nvfp4_rotamax", "nvfp4_quant_from_amax",
                 "mxfp4_rotquant", "mxfp4_rotquant_f32", "mxfp4_dequant",
                 "nvfp4_rotate16", "nvfp4_rotate16_f32", "nvfp4_rotquant_swizzled",
                 "nvfp4_rotquant_swizzled_f32", "nvfp4_dequant_swizzled",
                 "nvfp4_swizzled_scale_bytes", "nvfp4_rotquant_timed",
                 "nvfp4_rotquant_f32_timed", "nvfp4_stream_calibrate",
                 "nvfp4_stream_calibrate_f32", "nvfp4_stream_calibrate_single",
                 "nvfp4_stream_calibrate_single_f32", "nvfp4_rotate_matrix", "nvfp4_rotate_matrix_f32"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    seen = set()
    for st in range(6):
        s = lib.nvfp4_status_string(st).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.nvfp4_status_string(99).decode() == "unknown status"


# Fake, never-dereferenced device addresses: validation only looks at them.
X, Q, S, G, A = 0x10000, 0x20000, 0x30000, 0x40000, 0x40010


def rq(lib, x=X, rows=4, cols=64, rotate=1, q=Q, s=S, g=G, a=A, name="nvfp4_rotquant"):
    if "from_amax" in name:   # (x, rows, cols, rotate, amax_in, q, s, gscale, stream)
        return getattr(lib, name)(x, rows, cols, rotate, a, q, s, g, None)
    return getattr(lib, name)(x, rows, cols, rotate, q, s, g, a, None)


@pytest.mark.parametrize("name", ["nvfp4_rotquant", "nvfp4_rotquant_f32",
                                  "nvfp4_quant_from_amax", "nvfp4_quant_from_amax_f32"])
def test_quant_validation(lib, name):
    f = lambda **kw: rq(lib, name=name, **kw)  # noqa: E731
    assert f(x=None) == ERR_NULL
    assert f(q=None) == ERR_NULL
    assert f(s=None) == ERR_NULL
    assert f(g=None) == ERR_NULL
    assert f(a=None) == ERR_NULL
    assert f(cols=24) == ERR_SHAPE
    assert f(cols=-16) == ERR_SHAPE
    assert f(rows=-1) == ERR_SHAPE
    assert f(rows=1 << 40, cols=1 << 40) == ERR_SHAPE
    assert f(rotate=2) == ERR_ARG
    assert f(rotate=-1) == ERR_ARG
    assert f(x=X + 8) == ERR_ALIGN
    assert f(q=Q + 8) == ERR_ALIGN
    assert f(s=S + 2) == ERR_ALIGN
    assert f(g=G + 2) == ERR_ALIGN
    assert f(a=A + 1) == ERR_ALIGN
    # outputs overlapping the input or each other
    assert f(q=X) == ERR_ARG
    assert f(s=Q + 16) == ERR_ARG
    assert f(g=S) == ERR_ARG
    assert f(a=G) == ERR_ARG


def test_empty_tensor_needs_only_the_scalars(lib):
    # rows * cols == 0 with NULL tensors still validates the scalar pointers
    assert rq(lib, x=None, q=None, s=None, rows=0, g=None) == ERR_NULL
    assert rq(lib, x=None, q=None, s=None, rows=0, a=None) == ERR_NULL


def test_rotamax_validation(lib):
    f = lib.nvfp4_rotamax
    assert f(None, 4, 64, 1, A, None) == ERR_NULL
    assert f(X, 4, 64, 1, None, None) == ERR_NULL
    assert f(X, 4, 40, 1, A, None) == ERR_SHAPE
    assert f(X, 4, 64, 3, A, None) == ERR_ARG
    assert f(X + 4, 4, 64, 1, A, None) == ERR_ALIGN
    assert f(X, 4, 64, 1, A + 2, None) == ERR_ALIGN
    assert f(X, 4, 64, 1, X + 64, None) == ERR_ARG


def test_stream_calibrate_validation(lib):
    for name in ("nvfp4_stream_calibrate", "nvfp4_stream_calibrate_f32", "nvfp4_stream_calibrate_single",
                 "nvfp4_stream_calibrate_single_f32"):
        f = getattr(lib, name)
        assert f(None, 4, 64, Q, S, None) == ERR_NULL
        assert f(X, 4, 64, None, S, None) == ERR_NULL
        assert f(X, 4, 64, Q, None, None) == ERR_NULL
        assert f(X, 4, 40, Q, S, None) == ERR_SHAPE
        assert f(X, -1, 64, Q, S, None) == ERR_SHAPE
        assert f(X + 8, 4, 64, Q, S, None) == ERR_ALIGN
        assert f(X, 4, 64, Q + 8, S, None) == ERR_ALIGN
        assert f(X, 4, 64, X, S, None) == ERR_ARG
        assert f(X, 4, 64, Q, Q + 16, None) == ERR_ARG
        assert f(None, 0, 64, None, None, None) == OK


def test_dequant_validation(lib):
    f = lib.nvfp4_dequant
    Y = 0x80000
    assert f(None, S, G, 4, 64, 1, Y, None) == ERR_NULL
    assert f(Q, None, G, 4, 64, 1, Y, None) == ERR_NULL
    assert f(Q, S, None, 4, 64, 1, Y, None) == ERR_NULL
    assert f(Q, S, G, 4, 64, 1, None, None) == ERR_NULL
    assert f(Q, S, G, 4, 48 + 8, 1, Y, None) == ERR_SHAPE
    assert f(Q, S, G, 4, 64, 7, Y, None) == ERR_ARG
    assert f(Q + 4, S, G, 4, 64, 1, Y, None) == ERR_ALIGN
    assert f(Q, S, G, 4, 64, 1, Y + 8, None) == ERR_ALIGN
    assert f(Q, S, G, 4, 64, 1, Q, None) == ERR_ARG


@pytest.mark.parametrize("name", ["mxfp4_rotquant", "mxfp4_rotquant_f32"])
def test_mx_quant_validation(lib, name):
    f = lambda x=X, rows=4, cols=64, rotate=1, q=Q, s=S: getattr(lib, name)(  # noqa: E731
        x, rows, cols, rotate, q, s, None)
    assert f(x=None) == ERR_NULL
    assert f(q=None) == ERR_NULL
    assert f(s=None) == ERR_NULL
    assert f(cols=48) == ERR_SHAPE          # a multiple of 16, not of 32
    assert f(cols=-32) == ERR_SHAPE
    assert f(rows=-1) == ERR_SHAPE
    assert f(rows=1 << 40, cols=1 << 40) == ERR_SHAPE
    assert f(rotate=2) == ERR_ARG
    assert f(x=X + 8) == ERR_ALIGN
    assert f(q=Q + 8) == ERR_ALIGN
    assert f(q=X) == ERR_ARG
    assert f(s=Q + 16) == ERR_ARG
    assert f(x=None, q=None, s=None, rows=0) == OK     # empty: nothing to do


def test_mx_dequant_validation(lib):
    f = lib.mxfp4_dequant
    Y = 0x80000
    assert f(None, S, 4, 64, 1, Y, None) == ERR_NULL
    assert f(Q, None, 4, 64, 1, Y, None) == ERR_NULL
    assert f(Q, S, 4, 64, 1, None, None) == ERR_NULL
    assert f(Q, S, 4, 48, 1, Y, None) == ERR_SHAPE
    assert f(Q, S, 4, 64, 5, Y, None) == ERR_ARG
    assert f(Q + 4, S, 4, 64, 1, Y, None) == ERR_ALIGN
    assert f(Q, S, 4, 64, 1, Y + 8, None) == ERR_ALIGN
    assert f(Q, S, 4, 64, 1, Q, None) == ERR_ARG


@pytest.mark.parametrize("name", ["nvfp4_rotate16", "nvfp4_rotate16_f32"])
def test_rotate_validation(lib, name):
    f = getattr(lib, name)
    Y = 0x80000
    assert f(None, 4, 64, Y, None) == ERR_NULL
    assert f(X, 4, 64, None, None) == ERR_NULL
    assert f(X, 4, 40, Y, None) == ERR_SHAPE
    assert f(X + 8, 4, 64, Y, None) == ERR_ALIGN
    assert f(X, 4, 64, Y + 4, None) == ERR_ALIGN
    assert f(X, 4, 64, X + 64, None) == ERR_ARG
    assert f(None, 0, 64, None, None) == OK


@pytest.mark.parametrize("name", ["nvfp4_rotate_matrix", "nvfp4_rotate_matrix_f32"])
def test_rotate_matrix_validation(lib, name):
    f = getattr(lib, name)
    Y, R = 0x80000, 0x200000
    assert f(None, 4, 64, R, Y, None) == ERR_NULL
    assert f(X, 4, 64, None, Y, None) == ERR_NULL
    assert f(X, 4, 64, R, None, None) == ERR_NULL
    assert f(X, 4, 40, R, Y, None) == ERR_SHAPE
    assert f(X + 8, 4, 64, R, Y, None) == ERR_ALIGN
    assert f(X, 4, 64, R + 4, Y, None) == ERR_ALIGN
    assert f(X, 4, 64, R, Y + 4, None) == ERR_ALIGN
    assert f(X, 4, 64, R, X + 64, None) == ERR_ARG          # output over the input
    assert f(X, 4, 64, Y + 256, Y, None) == ERR_ARG         # output over the matrix
    assert f(None, 0, 64, R, None, None) == OK
    assert f(None, 0, 64, None, None, None) == ERR_NULL


def test_swizzled_scale_bytes(lib):
    f = lib.nvfp4_swizzled_scale_bytes
    assert f(128, 64) == 512
    assert f(129, 64) == 1024
    assert f(128, 80) == 1024
    assert f(16384, 8192) == 16384 * 512
    assert f(0, 64) == 0
    assert f(1, 16) == 512
    assert f(4, 40) == -1
    assert f(-1, 64) == -1
    assert f(1 << 20, 1 << 20) == -1          # more than 2^32 - 1 blocks


@pytest.mark.parametrize("name", ["nvfp4_rotquant_swizzled", "nvfp4_rotquant_swizzled_f32"])
def test_swizzled_quant_validation(lib, name):
    f = lambda **kw: rq(lib, name=name, **kw)  # noqa: E731
    assert f(x=None) == ERR_NULL
    assert f(s=None) == ERR_NULL
    assert f(cols=24) == ERR_SHAPE
    assert f(rotate=2) == ERR_ARG
    assert f(q=Q + 8) == ERR_ALIGN
    assert f(s=S + 2) == ERR_ALIGN
    assert f(s=X + 64) == ERR_ARG            # inside the input
    assert f(q=S - 64) == ERR_ARG            # codes run into the 512-byte scale tile
    assert f(rows=1 << 20, cols=1 << 20) == ERR_SHAPE


def test_swizzled_dequant_validation(lib):
    f = lib.nvfp4_dequant_swizzled
    Y = 0x80000
    assert f(None, S, G, 4, 64, 1, Y, None) == ERR_NULL
    assert f(Q, S, G, 4, 40, 1, Y, None) == ERR_SHAPE
    assert f(Q, S, G, 4, 64, 3, Y, None) == ERR_ARG
    assert f(Q, S, G, 4, 64, 1, S - 64, None) == ERR_ARG


@pytest.mark.parametrize("name", ["nvfp4_rotquant_timed", "nvfp4_rotquant_f32_timed"])
def test_timed_validation(lib, name):
    """events and nkernels are host memory (an array of event handles and an
    int); validation runs before any event is touched."""
    f = getattr(lib, name)
    ev = (ctypes.c_void_p * 4)()
    nk = ctypes.c_int(-1)
    EV, NK = ctypes.addressof(ev), ctypes.addressof(nk)
    assert f(X, 4, 64, 1, Q, S, G, A, None, None, 2, NK) == ERR_NULL
    assert f(X, 4, 64, 1, Q, S, G, A, None, EV, 0, NK) == ERR_NULL
    assert f(X, 4, 64, 1, Q, S, G, A, None, EV, 2, None) == ERR_NULL
    assert f(X, 4, 40, 1, Q, S, G, A, None, EV, 2, NK) == ERR_SHAPE
    assert nk.value == 0                     # nothing launched
    assert f(X, 4, 64, 1, X, S, G, A, None, EV, 2, NK) == ERR_ARG


def test_header_is_a_c_interface(tmp_path):
    """A C11 program (gcc, no C++) includes the header, links the library and
    calls the one entry point that needs no device: the header is a C
    interface usable without PyTorch or a C++ compiler."""
    import subprocess
    src = tmp_path / "use.c"
    src.write_text('#include <stdio.h>\n#include "nvfp4rq.h"\n'
                   'int main(void) {\n'
                   '  printf("%s|%s\\n", nvfp4_status_string(NVFP4_OK),\n'
                   '         nvfp4_status_string(NVFP4_ERR_SHAPE));\n'
                   '  return 0;\n}\n')
    exe = tmp_path / "use"
    libdir = os.path.dirname(LIB)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    f"-L{libdir}", "-lnvfp4rq", f"-Wl,-rpath,{libdir}"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.strip()
    ok, shape = out.split("|")
    assert ok and shape and ok != shape


def test_binding_buffer_checks_on_host():
    """The binding's buffer check is host logic: exercise it with host tensors."""
    import torch
    import nvfp4_activation_amd as nv
    cpu = torch.device("cpu")
    ok = torch.empty(8, dtype=torch.uint8)
    assert nv._buf(ok, 8, torch.uint8, cpu, "q") is ok
    assert nv._buf(torch.empty(9, dtype=torch.uint8), 8, torch.uint8, cpu, "q") is not None
    with pytest.raises(ValueError, match="7 elements, 8 needed"):
        nv._buf(torch.empty(7, dtype=torch.uint8), 8, torch.uint8, cpu, "q")
    with pytest.raises(TypeError, match="uint8"):
        nv._buf(torch.empty(8, dtype=torch.int8), 8, torch.uint8, cpu, "q")
    with pytest.raises(ValueError, match="contiguous"):
        nv._buf(torch.empty(16, dtype=torch.uint8)[::2], 8, torch.uint8, cpu, "q")
    with pytest.raises(ValueError, match="is on"):
        nv._buf(ok, 8, torch.uint8, torch.device("cuda", 0), "q")
    with pytest.raises(TypeError, match="tensor"):
        nv._buf(None, 8, torch.uint8, cpu, "q")


def test_binding_rejects_ragged_columns_on_host():
    """The binding names the column rule itself (before any device check)."""
    import torch
    import nvfp4_activation_amd as nv
    with pytest.raises(ValueError, match="multiple of 16"):
        nv.rotquant(torch.empty(4, 24, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="multiple of 32"):
        nv.mx_rotquant(torch.empty(4, 48, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="device tensor"):
        nv.rotquant(torch.empty(4, 32, dtype=torch.bfloat16))
