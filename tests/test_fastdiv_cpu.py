"""CPU proof that the kernels' division shortcut is exact where it is used.

The rotate+quantize kernel replaces each binary32 division y / d of the
definition (page "A Fused Hadamard + NVFP4 Quantization Kernel in Triton",
section 2: the block value (amax / 6) / g and the element quotient) by a
reciprocal computed once with a true division and a fused-multiply-add
correction (Markstein).  These enumerations show it returns the correctly
rounded quotient at every input that can change an E2M1 code or an E4M3
scale (see tests/helpers/fastdiv.c for the argument).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

from conftest import TESTS


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    out = tmp_path_factory.mktemp("fastdiv") / "libfastdiv.so"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", os.path.join(TESTS, "helpers", "fastdiv.c"), "-o",
                    str(out), "-lm"], check=True)
    lib = ctypes.CDLL(str(out))
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.verify_element.argtypes = [ctypes.c_int, u32p, u32p]
    lib.verify_element.restype = ctypes.c_longlong
    lib.verify_block.argtypes = [ctypes.c_int, u32p, u32p]
    lib.verify_block.restype = ctypes.c_longlong
    lib.verify_div6.argtypes = [ctypes.c_uint32, ctypes.c_uint32, u32p]
    lib.verify_div6.restype = ctypes.c_longlong
    lib.verify_random_codes.argtypes = [ctypes.c_int64, ctypes.c_uint64,
                                        ctypes.POINTER(ctypes.c_double)]
    lib.verify_random_codes.restype = ctypes.c_longlong
    return lib


def test_element_quotient_at_every_e2m1_boundary(lib):
    a, b = ctypes.c_uint32(), ctypes.c_uint32()
    bad = lib.verify_element(4, ctypes.byref(a), ctypes.byref(b))
    assert bad == 0, f"{bad} mismatches, e.g. d4={a.value:#010x} z={b.value:#010x}"


def test_block_value_at_every_e4m3_boundary(lib):
    a, b = ctypes.c_uint32(), ctypes.c_uint32()
    bad = lib.verify_block(4, ctypes.byref(a), ctypes.byref(b))
    assert bad == 0, f"{bad} mismatches, e.g. g={a.value:#010x} a={b.value:#010x}"


def test_divide_by_six_every_float(lib):
    """Exact for every binary32 from 2^-124 up.  Below that the remainder
    underflows; such a block value is below 2^-70 once divided by a global
    scale >= 2^-52 (the kernels' fast-path range), so its E4M3 scale is 0
    whichever way the quotient rounds."""
    a = ctypes.c_uint32()
    bad = lib.verify_div6(0x01800000, 0x7F7FFFFF, ctypes.byref(a))
    assert bad == 0, f"{bad} mismatches, e.g. bits {a.value:#010x}"
    bad_low = lib.verify_div6(1, 0x017FFFFF, ctypes.byref(a))
    assert bad_low > 0   # the underflow region is real; the range above is what is proved


def test_random_element_codes(lib):
    mx = ctypes.c_double()
    bad = lib.verify_random_codes(200_000_000, 12345, ctypes.byref(mx))
    assert bad == 0, f"{bad} code mismatches (max ulp difference {mx.value})"
