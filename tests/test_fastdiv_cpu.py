"""CPU proof that the kernels' division shortcuts are exact where they are used.

The rotate+quantize kernel replaces each binary32 division y / d of the
definition (page "A Fused Hadamard + NVFP4 Quantization Kernel in Triton",
section 2: the block value (amax / 6) / g and the element quotient) by
multiplications with reciprocals computed once with true divisions:

- the block value: a fused-multiply-add correction (Markstein), which returns
  the correctly rounded quotient at every input that can change an E4M3 scale;
- the element quotient: a two-word reciprocal (two fused multiply-adds per
  element), whose E2M1 code equals that of the correctly rounded quotient at
  every input where the two could differ;
- the global scale (amax / 6) / 448 and the reciprocal table's low words: the
  same correction, equal to the divisions at every input the kernels give it.

See tests/helpers/fastdiv.c for the arguments.
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
    lib.verify_div_const.argtypes = [ctypes.c_float, ctypes.c_uint32, ctypes.c_uint32, u32p]
    lib.verify_div_const.restype = ctypes.c_longlong
    lib.verify_element2.argtypes = [ctypes.c_int, u32p, u32p]
    lib.verify_element2.restype = ctypes.c_longlong
    lib.max_tail_error.argtypes = []
    lib.max_tail_error.restype = ctypes.c_double
    lib.verify_random_codes2.argtypes = [ctypes.c_int64, ctypes.c_uint64]
    lib.verify_random_codes2.restype = ctypes.c_longlong
    lib.verify_random_codes.argtypes = [ctypes.c_int64, ctypes.c_uint64,
                                        ctypes.POINTER(ctypes.c_double)]
    lib.verify_random_codes.restype = ctypes.c_longlong
    lib.verify_recip_tail.argtypes = [ctypes.c_int, ctypes.c_int, u32p]
    lib.verify_recip_tail.restype = ctypes.c_longlong
    lib.verify_global_scale.argtypes = [ctypes.c_uint32, ctypes.c_uint32, u32p]
    lib.verify_global_scale.restype = ctypes.c_longlong
    return lib


def test_element_quotient_at_every_e2m1_boundary(lib):
    a, b = ctypes.c_uint32(), ctypes.c_uint32()
    bad = lib.verify_element(4, ctypes.byref(a), ctypes.byref(b))
    assert bad == 0, f"{bad} mismatches, e.g. d4={a.value:#010x} z={b.value:#010x}"


def test_block_value_at_every_e4m3_boundary(lib):
    a, b = ctypes.c_uint32(), ctypes.c_uint32()
    bad = lib.verify_block(4, ctypes.byref(a), ctypes.byref(b))
    assert bad == 0, f"{bad} mismatches, e.g. g={a.value:#010x} a={b.value:#010x}"


@pytest.mark.parametrize("c,lo", [(6.0, 0x01800000), (24.0, 0x02800000)])
def test_divide_by_constant_every_float(lib, c, lo):
    """a / 6 exact for every binary32 from 2^-124 up, a / 24 from 2^-122 up
    (the rotated block's amax enters unscaled, z / 24 = y / 6).  Below that
    the remainder underflows; such a block value is below 2^-70 once divided
    by a global scale >= 2^-52 (the kernels' fast-path range), so its E4M3
    scale is 0 whichever way the quotient rounds."""
    a = ctypes.c_uint32()
    bad = lib.verify_div_const(c, lo, 0x7F7FFFFF, ctypes.byref(a))
    assert bad == 0, f"{bad} mismatches, e.g. bits {a.value:#010x}"
    bad_low = lib.verify_div_const(c, 1, lo - 1, ctypes.byref(a))
    assert bad_low > 0   # the underflow region is real; the range above is what is proved


def test_random_element_codes(lib):
    mx = ctypes.c_double()
    bad = lib.verify_random_codes(200_000_000, 12345, ctypes.byref(mx))
    assert bad == 0, f"{bad} code mismatches (max ulp difference {mx.value})"


def test_two_word_reciprocal_tail(lib):
    """rh + rl approximates 1/D within 2^-47 relative for every significand,
    the bound the window argument for the two-operation quotient rests on."""
    assert lib.max_tail_error() < 2.0


def test_element_codes_two_operation_quotient(lib):
    """Every input within 16 ulps of every E2M1 decision boundary, both signs,
    for all 2^23 divisor significands: the two-operation quotient gives the
    code of the correctly rounded one."""
    a, b = ctypes.c_uint32(), ctypes.c_uint32()
    bad = lib.verify_element2(16, ctypes.byref(a), ctypes.byref(b))
    assert bad == 0, f"{bad} mismatches, e.g. D={a.value:#010x} z={b.value:#010x}"


def test_random_element_codes_two_operation_quotient(lib):
    assert lib.verify_random_codes2(200_000_000, 777) == 0


def test_corrected_reciprocal_tail_every_divisor(lib):
    """The table's low word RN((1 - rh D) / D) from the corrected product
    equals the division for every binary32 D in [2^-60, 2^16), every divisor
    the tables can hold (all exponents enumerated, not only one binade)."""
    a = ctypes.c_uint32()
    bad = lib.verify_recip_tail(-60, 16, ctypes.byref(a))
    assert bad == 0, f"{bad} mismatches, e.g. D={a.value:#010x}"


def test_divide_by_448_on_the_fast_range(lib):
    """y / 448 through the corrected product for every y in [2^-41, 2^13),
    which holds every RN(amax / 6) of the fast path."""
    a = ctypes.c_uint32()
    bad = lib.verify_div_const(448.0, 0x2B000000, 0x45FFFFFF, ctypes.byref(a))
    assert bad == 0, f"{bad} mismatches, e.g. bits {a.value:#010x}"


def test_global_scale_every_fast_amax(lib):
    """(amax / 6) / 448 as two corrected products equals the two divisions
    for every binary32 amax in [2^-38, 2^15), the fast path's range."""
    a = ctypes.c_uint32()
    bad = lib.verify_global_scale(0x2C800000, 0x46FFFFFF, ctypes.byref(a))
    assert bad == 0, f"{bad} mismatches, e.g. amax bits {a.value:#010x}"
