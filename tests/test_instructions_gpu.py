"""Exhaustive checks of the gfx950 conversion instructions the kernels use,
through the library's own device helpers, against the CPU oracle.

- E2M1: v_cvt_scalef32_pk_fp4_f32 (scale 1.0) behind e2m1_pack8, every
  non-NaN binary32 except -0.0, against the page's midpoint compares (page "A
  Fused Hadamard + NVFP4 Quantization Kernel in Triton", section 2).  -0.0 is
  the one input where the instruction (sign bit from IEEE) and the page (code
  8 only when v < 0) differ; the kernels never pass it, and the test records
  the difference.
- E4M3: min(v, 448) then v_cvt_pk_fp8_f32 behind e4m3_byte, every binary32
  in [0, +inf], against the oracle's round-to-nearest-even with the 448 clamp
  (section 2, _round_e4m3; section 3).
- Decode: v_cvt_scalef32_pk_f32_fp4 (scale 1.0) behind e2m1_pair, every byte
  at every byte position, against the grid table of section 1, bit for bit.
- The quantize prologue's corrected products on the device (the CPU proofs
  in tests/helpers/fastdiv.c assume an exactly rounded fused multiply-add):
  the global scale (amax / 6) / 448 against two binary32 divisions, and the
  reciprocal table's words rh = RN(1/D), rl = RN((1 - rh D) / D) against
  binary32 divisions, over whole binades and a strided sample of the range.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from conftest import ROOT

pytestmark = pytest.mark.gpu

PROBE = os.path.join(ROOT, "tests", "helpers", "libinstrprobe.so")


@pytest.fixture(scope="module")
def probe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib = ctypes.CDLL(PROBE)
    for name in ("probe_e2m1", "probe_e4m3"):
        getattr(lib, name).argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                       ctypes.c_void_p]
        getattr(lib, name).restype = ctypes.c_int
    for name in ("probe_gscale", "probe_recip2"):
        getattr(lib, name).argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                       ctypes.c_void_p]
        getattr(lib, name).restype = ctypes.c_int
    lib.probe_pack.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_values.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _sweep(probe_fn, ref_fn, lo: int, hi: int, exclude) -> None:
    chunk = 1 << 27
    buf = torch.empty(chunk, dtype=torch.uint8, device="cuda:0")
    for base in range(lo, hi + 1, chunk):
        n = min(chunk, hi + 1 - base)
        assert probe_fn(base, n, buf.data_ptr(), _stream()) == 0
        torch.cuda.synchronize()
        got = buf[:n].cpu().numpy()
        ref = ref_fn(base, base + n - 1)
        bad = np.nonzero(got != ref)[0]
        if bad.size:
            bits = (base + bad).astype(np.uint64)
            keep = ~exclude(bits)
            bad, bits = bad[keep], bits[keep]
        assert bad.size == 0, (f"{bad.size} mismatches from bits {base:#010x}, first "
                               f"{int(bits[0]):#010x}: gpu {got[bad[0]]} oracle {ref[bad[0]]}")


def test_e2m1_conversion_every_float(probe):
    def exclude(bits):
        mag = bits & 0x7FFFFFFF
        return (mag > 0x7F800000) | (bits == 0x80000000)     # NaNs, -0.0
    _sweep(probe.probe_e2m1, oracle.e2m1_codes_bits, 0, 0xFFFFFFFF, exclude)


def test_e2m1_conversion_negative_zero_is_the_exception(probe):
    buf = torch.empty(1, dtype=torch.uint8, device="cuda:0")
    assert probe.probe_e2m1(0x80000000, 1, buf.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    assert buf.item() == 8 and oracle.e2m1_code(-0.0) == 0


def test_e4m3_conversion_every_nonnegative_float(probe):
    _sweep(probe.probe_e4m3, oracle.e4m3_bytes_bits, 0, 0x7F800000,
           lambda bits: np.zeros(bits.shape, dtype=bool))


def test_nibble_order_and_value_tables(probe):
    v = torch.tensor([0.5, 1, 1.5, 2, 3, 4, 6, -0.5, 0, -1, -1.5, -2, -3, -4, -6, 0.25],
                     dtype=torch.float32, device="cuda:0")
    out = torch.zeros(2, dtype=torch.int32, device="cuda:0")
    probe.probe_pack(v.data_ptr(), out.data_ptr(), _stream())
    torch.cuda.synchronize()
    w = out.cpu().numpy().view(np.uint32)
    codes = [(int(w[i // 8]) >> (4 * (i % 8))) & 15 for i in range(16)]
    assert codes == [oracle.e2m1_code(float(t)) for t in v.cpu().numpy()]
    e4 = torch.zeros(256, dtype=torch.float32, device="cuda:0")
    e2 = torch.zeros(2048, dtype=torch.float32, device="cuda:0")
    probe.probe_values(e4.data_ptr(), e2.data_ptr(), _stream())
    torch.cuda.synchronize()
    e4 = e4.cpu().numpy()
    for b in range(127):
        assert e4[b] == oracle.e4m3_value(b), b
    # E2M1 decode (v_cvt_scalef32_pk_f32_fp4, scale 1.0): every byte at every
    # byte position, low nibble first, compared as bits so that code 8 must
    # give -0.0 (the page's dequantize flips the sign of a zero magnitude)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    table = np.concatenate([grid, -grid]).astype(np.float32)
    byte = np.arange(256)
    want = np.stack([table[byte & 15], table[byte >> 4]], axis=1).reshape(-1)
    got = e2.cpu().numpy().reshape(4, 512)
    for pos in range(4):
        assert np.array_equal(got[pos].view(np.uint32), want.view(np.uint32)), pos


def _strided(lo: int, hi: int, stride: int):
    """(base, stride, count) covering bit patterns lo, lo + stride, ... <= hi."""
    return lo, stride, (hi - lo) // stride + 1


def _floats(base: int, stride: int, n: int) -> np.ndarray:
    bits = np.uint64(base) + np.arange(n, dtype=np.uint64) * np.uint64(stride)
    assert int(bits[-1]) < 1 << 32
    return bits.astype(np.uint32).view(np.float32)


# whole binades at both ends and in the middle, plus a stride-97 sample of the range
GSCALE_CASES = [_strided(0x2C800000, 0x2CFFFFFF, 1), _strided(0x3F000000, 0x3F7FFFFF, 1),
                _strided(0x46800000, 0x46FFFFFF, 1), _strided(0x2C800000, 0x46FFFFFF, 97)]
RECIP_CASES = [_strided(0x21800000, 0x21FFFFFF, 1), _strided(0x3F800000, 0x3FFFFFFF, 1),
               _strided(0x47000000, 0x477FFFFF, 1), _strided(0x21800000, 0x477FFFFF, 97)]


@pytest.mark.parametrize("base,stride,n", GSCALE_CASES)
def test_global_scale_corrected_products(probe, base, stride, n):
    """amax in the fast path's range [2^-38, 2^15): the device's two corrected
    products give the bits of fl(fl(amax / 6) / 448)."""
    out = torch.empty(n, dtype=torch.int32, device="cuda:0")
    assert probe.probe_gscale(base, stride, n, out.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    a = _floats(base, stride, n)
    want = (a / np.float32(6.0)) / np.float32(448.0)
    assert want.dtype == np.float32
    got = out.cpu().numpy().view(np.uint32)
    bad = np.nonzero(got != want.view(np.uint32))[0]
    assert bad.size == 0, f"{bad.size} mismatches, first amax bits {a[bad[0]].view(np.uint32):#010x}"


@pytest.mark.parametrize("base,stride,n", RECIP_CASES)
def test_reciprocal_table_words(probe, base, stride, n):
    """D in [2^-60, 2^16), every divisor the tables can hold: the device's
    rh is RN(1/D) and its rl, from the corrected product, is RN(e / D) with
    e = 1 - rh D (exact in binary32)."""
    out = torch.empty(2 * n, dtype=torch.int32, device="cuda:0")
    assert probe.probe_recip2(base, stride, n, out.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    d = _floats(base, stride, n)
    rh = np.float32(1.0) / d
    e64 = 1.0 - rh.astype(np.float64) * d.astype(np.float64)   # exact: 48-bit product near 1
    e = e64.astype(np.float32)
    assert np.array_equal(e.astype(np.float64), e64)            # the residual fits binary32
    rl = e / d
    got = out.cpu().numpy().view(np.uint32).reshape(n, 2)
    for col, want, name in ((0, rh, "rh"), (1, rl, "rl")):
        bad = np.nonzero(got[:, col] != want.view(np.uint32))[0]
        assert bad.size == 0, f"{name}: {bad.size} mismatches, first D bits {d[bad[0]].view(np.uint32):#010x}"
