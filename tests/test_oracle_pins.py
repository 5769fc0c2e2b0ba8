"""Pins of the CPU oracle against what the pages and the mathematics fix.

Page: "A Fused Hadamard + NVFP4 Quantization Kernel in Triton" (kanthi.in).
Every test here runs on the CPU.  None of them compares the oracle with
itself: each one checks it against a printed value, a closed form, an
invariant, a library routine on a special case, an exhaustive nearest-point
search, or an exact-rational re-implementation.
"""
from __future__ import annotations

import ctypes
import math

import numpy as np
import pytest
import torch

import exact_model as em
import oracle
import synth
from conftest import read_golden

F32 = np.float32


def sylvester16() -> np.ndarray:
    """H16 built by Kronecker doubling [[H, H], [H, -H]] four times, then /4
    (section 2, hadamard16)."""
    h = np.ones((1, 1))
    for _ in range(4):
        h = np.block([[h, h], [h, -h]])
    return h / 4.0


# ---------------------------------------------------------------- P1: rotation

def test_rotation_columns_are_sylvester():
    """The butterfly applied to each unit vector gives that column of H16, exactly."""
    H = sylvester16().astype(np.float32)
    for i in range(16):
        e = np.zeros(16, dtype=np.float32)
        e[i] = 1.0
        y = oracle.rotate16(e)
        assert np.array_equal(y, H[:, i]), i


def test_rotation_is_orthonormal_exactly():
    """Section 1: H*H^T = I; exact in binary32 (entries +-1/4, sums of 16)."""
    cols = np.stack([oracle.rotate16(np.eye(16, dtype=np.float32)[i]) for i in range(16)], 1)
    prod = cols.astype(np.float32) @ cols.T.astype(np.float32)
    assert np.array_equal(prod, np.eye(16, dtype=np.float32))


def test_rotation_is_an_involution_on_small_integers():
    """H16 is symmetric and orthonormal, so H(Hx) = x; exact for small integers."""
    rng = np.random.default_rng(1)
    for _ in range(200):
        x = rng.integers(-100, 101, 16).astype(np.float32)
        assert np.array_equal(oracle.rotate16(oracle.rotate16(x)), x)


def test_rotation_within_rounding_bound_of_fp64():
    """|y_bfly - (H x)_fp64| <= gamma_5 * sum|x| / 4 (four rounded additions and
    one rounded scaling along each path), plus Parseval."""
    H = sylvester16()
    rng = np.random.default_rng(2)
    u = 2.0 ** -24
    gamma5 = 5 * u / (1 - 5 * u)
    for _ in range(2000):
        x = (rng.standard_normal(16) * np.exp(rng.normal(0, 3, 16))).astype(np.float32)
        y = oracle.rotate16(x).astype(np.float64)
        yref = H @ x.astype(np.float64)
        bound = gamma5 * np.abs(x.astype(np.float64)).sum() / 4.0 + 1e-300
        assert np.all(np.abs(y - yref) <= bound)
        assert abs(np.linalg.norm(y) - np.linalg.norm(x.astype(np.float64))) <= \
            1e-5 * np.linalg.norm(x.astype(np.float64))


def test_rotation_stage_order_is_ascending():
    """Reading: strides 1, 2, 4, 8 in that order.  The exact-rational model
    follows that order; a vector where the order changes the binary32 result
    shows the pin is sensitive to it."""
    x = np.array([1.0, 2.0 ** -24, 2.0 ** -24, 0, 2.0 ** -24, 0, 0, 0,
                  0, 0, 0, 0, 0, 0, 0, 2.0 ** -25], dtype=np.float32)
    model = [em.frac_to_f32(v) for v in em.rotate16([em.f32_to_frac(v) for v in x])]
    assert np.array_equal(oracle.rotate16(x), np.array(model, dtype=np.float32))
    # the same stages in descending order give different bits for this vector
    z = [em.f32_to_frac(v) for v in x]
    h = 8
    while h >= 1:
        for i in range(16):
            if i & h == 0:
                a, b = z[i], z[i + h]
                z[i], z[i + h] = em.rn32(a + b), em.rn32(a - b)
        h //= 2
    desc = np.array([em.frac_to_f32(em.rn32(v / 4)) for v in z], dtype=np.float32)
    assert not np.array_equal(desc, oracle.rotate16(x))


# ---------------------------------------------------------------- P2: E2M1

def test_e2m1_table_from_the_page():
    for value, code in read_golden("e2m1_table.txt"):
        v = float(value)
        if value == "-0.0":
            v = -0.0
        assert oracle.e2m1_code(v) == int(code), value


def test_e2m1_neighbours_of_every_midpoint():
    """One ulp either side of each midpoint falls on the nearer grid point."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for k, m in enumerate(mids):
        below = np.nextafter(F32(m), F32(0))
        above = np.nextafter(F32(m), F32(np.inf))
        assert oracle.e2m1_code(below) == k, m
        assert oracle.e2m1_code(above) == k + 1, m
        assert oracle.e2m1_code(-below) == k + 8, m
        assert oracle.e2m1_code(-above) == k + 9, m


def test_e2m1_exhaustive_against_nearest_point(sweeps_lib):
    """All 2^32 - 2^24 non-NaN binary32 inputs against a nearest-grid search."""
    first = ctypes.c_uint32(0)
    bad = sweeps_lib.sweep_e2m1_all(ctypes.byref(first))
    assert bad == 0, f"{bad} mismatches, first at bits {first.value:#010x}"


# ---------------------------------------------------------------- P3: E4M3

def test_e4m3_worked_values_from_the_page():
    for inp, rne, faulty in read_golden("e4m3_worked_values.txt"):
        b = oracle.e4m3_byte(float(inp))
        assert oracle.e4m3_value(b) == float(rne), inp
        if float(faulty) != float(rne):
            assert oracle.e4m3_value(b) != float(faulty)


def test_e4m3_anchor_bytes():
    for value, byte in read_golden("e4m3_anchors.txt"):
        assert oracle.e4m3_byte(float(value)) == int(byte, 16), value
        assert oracle.e4m3_value(int(byte, 16)) == float(value), value


def test_e4m3_saturates_at_448():
    for v in (448.0, 449.0, 463.9, 464.0, 465.0, 480.0, 1e6, 3.0e38, float("inf")):
        assert oracle.e4m3_byte(v) == 0x7E, v


def test_e4m3_ties_go_to_even():
    # 1.0625 sits halfway between 1.0 (mantissa 0) and 1.125 (mantissa 1)
    assert oracle.e4m3_value(oracle.e4m3_byte(1.0625)) == 1.0
    # 1.1875 halfway between 1.125 (odd) and 1.25 (even)
    assert oracle.e4m3_value(oracle.e4m3_byte(1.1875)) == 1.25
    # 2^-10 halfway between 0 and 2^-9: goes to 0; 3*2^-10 goes to 2^-8
    assert oracle.e4m3_byte(2.0 ** -10) == 0
    assert oracle.e4m3_value(oracle.e4m3_byte(3 * 2.0 ** -10)) == 2.0 ** -8


def test_e4m3_exhaustive_against_nearest_point(sweeps_lib):
    """Every binary32 in [0, 2^10] (and up to +inf) against a bisection
    nearest-value search over the 127 E4M3 values."""
    first = ctypes.c_uint32(0)
    bad = sweeps_lib.sweep_e4m3_range(0, 0x7F800000, ctypes.byref(first))
    assert bad == 0, f"{bad} mismatches, first at bits {first.value:#010x}"


def test_e4m3_strided_against_linear_search(sweeps_lib):
    first = ctypes.c_uint32(0)
    bad = sweeps_lib.sweep_e4m3_linear(0, 0x44800000, 97, ctypes.byref(first))
    assert bad == 0, f"{bad} mismatches, first at bits {first.value:#010x}"


def test_e4m3_exhaustive_against_torch_cast():
    """PyTorch's float8_e4m3fn cast (round to nearest even; the reference cast
    of section 3) on every binary32 in [0, 464); above that torch gives NaN and
    the definition clamps at 448."""
    hi = int(np.float32(464.0).view(np.uint32))
    step = 1 << 25
    for lo in range(0, hi, step):
        n = min(step, hi - lo)
        bits = np.arange(lo, lo + n, dtype=np.uint32)
        vals = bits.view(np.float32)
        ours = oracle.e4m3_bytes(vals)
        ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        mism = np.nonzero(ours != ref)[0]
        assert mism.size == 0, f"first mismatch at bits {bits[mism[0]]:#010x}"


# ---------------------------------------------------------------- P4-P6: scales and sizes

def _bf16(x: np.ndarray) -> np.ndarray:
    return synth.round_bf16(np.asarray(x, dtype=np.float64))


def test_all_zero_tensor():
    x = np.zeros((4, 64), dtype=np.uint16)
    for rotate in (True, False):
        q, s, g, a = oracle.quantize(x, rotate)
        assert g == 1.0 and a == 0.0
        assert not q.any() and not s.any()


def test_largest_block_scale_is_448():
    """The global scale puts the block holding the global amax at 448 (0x7E)."""
    for seed in range(6):
        x = synth.normal_bf16(64 * 256, seed=seed, scale=10.0 ** (seed - 3)).reshape(64, 256)
        for rotate in (True, False):
            q, s, g, a = oracle.quantize(x, rotate)
            assert s.max() == 0x7E
            assert g > 0 and abs(float(g) * 2688.0 - float(a)) <= 4e-7 * float(a)


def test_full_scale_blocks_reach_code_7():
    """Invariant: a block with a normal-range E4M3 scale below 448 has its
    largest element at code 7, since a_b / (s g) lies in (5, 6.4]."""
    w = synth.make("gauss_1pct_cols_4096x4096", rows=64)
    for rotate in (True, False):
        q, s, g, a = oracle.quantize(w.x, rotate)
        codes = np.stack([q & 15, q >> 4], -1).reshape(s.shape[0], -1, 16)
        mag = (codes & 7).max(-1)
        scale_vals = np.vectorize(oracle.e4m3_value)(s)
        normal = (scale_vals >= 2.0 ** -6)
        assert normal.any()
        assert np.all(mag[normal] == 7)


def test_storage_is_4p5_bits_per_value():
    rows = dict(read_golden("format_sizes.txt"))
    x = synth.normal_bf16(256 * 64, seed=3).reshape(256, 64)
    q, s, g, a = oracle.quantize(x, True)
    assert q.size == int(rows["packed_bytes"]) and s.size == int(rows["scale_bytes"])
    assert (q.size + s.size) / x.size == float(rows["bytes_per_value"])


# ---------------------------------------------------------------- P7: exact-rational model

def _tiny_inputs(n_cases: int):
    """Small tensors mixing magnitudes so that butterfly sums round, scales land
    near E4M3 midpoints and quotients near E2M1 midpoints."""
    rng = np.random.default_rng(7)
    for i in range(n_cases):
        rows = int(rng.integers(1, 4))
        cols = 16 * int(rng.integers(1, 4))
        n = rows * cols
        kind = i % 5
        if kind == 0:
            v = rng.standard_normal(n)
        elif kind == 1:
            v = rng.standard_normal(n) * np.exp2(rng.integers(-30, 30, n))
        elif kind == 2:
            v = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], n) * \
                rng.choice([-1.0, 1.0], n)
        elif kind == 3:
            v = rng.integers(-64, 65, n).astype(np.float64) / 8.0
        else:
            v = rng.standard_normal(n)
            v[rng.integers(0, n, max(1, n // 8))] = 0.0
            v[rng.integers(0, n)] *= 1e4
        f32 = (i % 2 == 1)
        if f32:
            x = v.astype(np.float32).reshape(rows, cols)
            xf = x
        else:
            x = _bf16(v).reshape(rows, cols)
            xf = synth.bf16_to_f32(x)
        yield x, xf, bool(rng.integers(0, 2))


def test_oracle_matches_exact_rational_model():
    n = 0
    for x, xf, rotate in _tiny_inputs(1500):
        q, s, g, a = oracle.quantize(x, rotate)
        mq, ms, mg, ma = em.quantize(xf, rotate)
        assert np.array_equal(q, mq), (x, rotate)
        assert np.array_equal(s, ms), (x, rotate)
        assert em.f32_bits(g) == em.f32_bits(mg) and em.f32_bits(a) == em.f32_bits(ma)
        n += 1
    assert n == 1500


def test_given_scale_matches_exact_model():
    """Quantization with a caller-supplied global scale (an amax from an
    earlier step, section 2's note on reusing an amax): the block value can
    pass 448 and is clamped there; quotients can pass 6 and saturate."""
    rng = np.random.default_rng(17)
    n = 0
    for x, xf, rotate in _tiny_inputs(300):
        true_amax = float(np.abs(xf).max()) or 1.0
        for factor in (1e-6, 0.01, 0.37, 1.0, 3.0):
            amax_given = np.float32(true_amax * factor * rng.uniform(0.5, 2.0))
            g = oracle.global_scale(amax_given)
            q, s = oracle.quantize_given_scale(x, rotate, g)
            mq, ms = em.quantize_given_scale(xf, rotate, em.f32_to_frac(g))
            assert np.array_equal(q, mq) and np.array_equal(s, ms), (x, rotate, g)
            n += 1
    assert n == 1500


def test_given_scale_with_own_amax_is_the_full_method():
    for name in ("gauss_outliers_128x1024", "kv_heads_65536x8x128_f32"):
        w = synth.make(name, rows=64)
        for rotate in (True, False):
            q, s, g, a = oracle.quantize(w.x, rotate)
            q2, s2 = oracle.quantize_given_scale(w.x, rotate, oracle.global_scale(a))
            assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_given_scale_saturates_blocks_at_448():
    """A global scale 100x too small puts most block values above 448: the
    scale byte is 0x7E and the largest codes saturate at 7."""
    x = synth.normal_bf16(32 * 256, seed=9).reshape(32, 256)
    q, s, g, a = oracle.quantize(x, True)
    q2, s2 = oracle.quantize_given_scale(x, True, oracle.global_scale(a / 100))
    assert (s2 == 0x7E).mean() > 0.9
    codes = np.stack([q2 & 15, q2 >> 4], -1)
    assert ((codes & 7) == 7).mean() > 0.2


def test_divisor_one_when_scale_rounds_to_zero():
    """When a block's scale rounds to E4M3 zero the divisor is 1.0 and codes
    come from the raw values (section 2, the where(s_f == 0, 1, s_f) guard)."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 2.0 ** 20          # block 0 sets amax = 2^20, g = 2^20 / 2688
    x[0, 16:] = 0.3              # block 1: (0.3/6)/g < 2^-10, so s rounds to 0
    q, s, g, a = oracle.quantize(x, False)
    assert s[0, 0] == 0x7E and s[0, 1] == 0
    assert np.all((q[0, 8:] & 15) == 1) and np.all((q[0, 8:] >> 4) == 1)
    mq, ms, mg, ma = em.quantize(x, False)
    assert np.array_equal(q, mq) and np.array_equal(s, ms)


def test_sign_of_zero_and_tiny_negatives():
    """Code 8 needs a quotient below zero; -0.0 gives code 0 (section 2: sign
    bit from v < 0)."""
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, 0] = 6.0
    x[0, 1] = -0.0
    x[0, 2] = -1e-30
    x[0, 3] = 1e-30
    q, s, g, a = oracle.quantize(x, False)
    codes = np.stack([q & 15, q >> 4], -1).reshape(-1)
    assert codes[0] == 7 and codes[1] == 0 and codes[2] == 8 and codes[3] == 0


# ---------------------------------------------------------------- P8: printed errors

def _page_tensors():
    torch.manual_seed(0)
    x = torch.randn(256, 64)
    x[:, [3, 17, 40]] *= 20.0
    gauss = torch.randn(256, 64)
    t3 = torch.distributions.StudentT(3.0).sample((256, 64))
    return x.numpy().copy(), gauss.numpy().copy(), t3.numpy().copy()


def test_printed_round_trip_errors():
    """Sections 3 and 5 print eight relative L2 errors to four decimals."""
    expected = {r[0]: (float(r[1]), float(r[2])) for r in read_golden("error_table.txt")}
    x, gauss, t3 = _page_tensors()
    normal_cols = np.ones(64, dtype=np.uint8)
    normal_cols[[3, 17, 40]] = 0
    cases = {"outlier_all": (x, None), "outlier_normal": (x, normal_cols),
             "gaussian": (gauss, None), "student_t3": (t3, None)}
    for name, (t, mask) in cases.items():
        got = []
        for rotate in (False, True):
            q, s, g, a = oracle.quantize(np.ascontiguousarray(t, dtype=np.float32), rotate)
            got.append(oracle.roundtrip_error(t, rotate, q, s, g, mask))
        assert round(got[0], 4) == expected[name][0], (name, got)
        assert round(got[1], 4) == expected[name][1], (name, got)


# ---------------------------------------------------------------- P9: thread-count invariance

def test_thread_count_does_not_change_bytes():
    w = synth.make("t3_lognormal_16384x8192", rows=64)
    r1 = oracle.quantize(w.x, True, nthreads=1)
    r8 = oracle.quantize(w.x, True, nthreads=8)
    for a, b in zip(r1, r8):
        assert np.array_equal(np.asarray(a), np.asarray(b))


# ---------------------------------------------------------------- P10: library special case

def torch_reference(xf: torch.Tensor, rotate: bool):
    """The arithmetic of section 3's reference in PyTorch (CPU, fp32): a dense
    matmul rotation, torch's float8_e4m3fn cast for the scales, IEEE division,
    the seven threshold compares.  With rotate=False nothing is summed, so this
    computes exactly the definition with library routines."""
    y = xf.reshape(-1, 16).float()
    if rotate:
        y = y @ torch.from_numpy(sylvester16().astype(np.float32))
    g = float(y.abs().max() / 6.0 / 448.0) or 1.0
    s = (y.abs().amax(1) / 6.0 / g).to(torch.float8_e4m3fn)
    sf = s.float() * g
    v = y / torch.where(sf == 0, torch.ones_like(sf), sf)[:, None]
    a = v.abs()
    c = ((a > 0.25).int() + (a >= 0.75).int() + (a > 1.25).int() + (a >= 1.75).int()
         + (a > 2.5).int() + (a >= 3.5).int() + (a > 5.0).int())
    c = (c + (v < 0).int() * 8).to(torch.uint8)
    q = c[:, 0::2] | (c[:, 1::2] << 4)
    return q.numpy(), s.view(torch.uint8).numpy(), np.float32(g)


@pytest.mark.parametrize("name,rows", [
    ("gauss_outliers_128x1024", None),
    ("gauss_1pct_cols_4096x4096", 512),
    ("silu_ties_32768x14336", 128),
    ("kv_heads_65536x8x128_f32", 256),
    ("t3_lognormal_16384x8192", 128),
])
def test_rotate_off_equals_torch_reference(name, rows):
    w = synth.make(name, rotate=False, rows=rows)
    xf = synth.bf16_to_f32(w.x) if w.dtype == "bf16" else w.x
    q, s, g, a = oracle.quantize(w.x, False)
    rq, rs, rg = torch_reference(torch.from_numpy(xf.copy()), False)
    assert em.f32_bits(g) == em.f32_bits(rg)
    assert np.array_equal(s.reshape(-1), rs.reshape(-1))
    assert np.array_equal(q.reshape(-1, 8), rq)


def test_rotate_on_close_to_torch_reference():
    """With the rotation, the page's reference sums in the matmul's order, so
    bits may differ where a sum rounds; on bf16 data that is rare."""
    w = synth.make("gauss_1pct_cols_4096x4096", rows=256)
    xf = synth.bf16_to_f32(w.x)
    q, s, g, a = oracle.quantize(w.x, True)
    rq, rs, rg = torch_reference(torch.from_numpy(xf.copy()), True)
    assert np.mean(q.reshape(-1, 8) != rq) < 1e-4
    assert np.mean(s.reshape(-1) != rs.reshape(-1)) < 1e-4


def test_page_demo_tensor_matches_reference_codes():
    """Section 3: codes and scales of the demo tensor match the reference,
    with and without the rotation."""
    x, _, _ = _page_tensors()
    for rotate in (False, True):
        q, s, g, a = oracle.quantize(x, rotate)
        rq, rs, rg = torch_reference(torch.from_numpy(x), rotate)
        assert np.array_equal(q.reshape(-1, 8), rq)
        assert np.array_equal(s.reshape(-1), rs.reshape(-1))


# ---------------------------------------------------------------- P11: the halved-scale trap

def test_no_block_scale_is_halved():
    """Section 4: a lost exponent carry halves a scale; the oracle's scales
    equal torch's cast of the same values and none is half of it."""
    x, _, _ = _page_tensors()
    q, s, g, a = oracle.quantize(x, False)
    _, rs, _ = torch_reference(torch.from_numpy(x), False)
    ours = np.vectorize(oracle.e4m3_value)(s.reshape(-1))
    ref = np.vectorize(oracle.e4m3_value)(rs.reshape(-1))
    assert not np.any((ref > 0) & (ours == ref / 2))
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------- dequant in fp64

def test_dequant_inverts_exactly_representable_blocks():
    """A block whose rotated values sit on the E2M1 grid times a power-of-two
    scale decodes back to the input exactly (fp64 decode, exact H)."""
    t = np.array([6, -4, 3, 2, -1.5, 1, 0.5, 0, -6, 4, -3, 2, 1.5, -1, 0.5, 0],
                 dtype=np.float64)
    H = sylvester16()
    x = (H @ t).astype(np.float32).reshape(1, 16)   # exact: multiples of 1/8
    q, s, g, a = oracle.quantize(x, True)
    back = oracle.dequant_f64(q, s, g, True)
    assert np.array_equal(back.reshape(-1), x.astype(np.float64).reshape(-1))


# ---------------------------------------------------------------- MXFP4 variant

def test_e8m0_closed_forms():
    assert oracle.e8m0_byte(0.0) == 0
    assert oracle.e8m0_byte(1.0) == 127
    assert oracle.e8m0_byte(float(np.nextafter(F32(1.0), F32(2.0)))) == 128
    assert oracle.e8m0_byte(0.75) == 127
    assert oracle.e8m0_byte(2.0 ** -127) == 0
    assert oracle.e8m0_byte(2.0 ** -140) == 0          # clamped at 2^-127
    assert oracle.e8m0_byte(2.0 ** 127) == 254
    assert oracle.e8m0_byte(3.0e38) == 254             # clamped at 2^127
    for b in range(255):
        assert oracle.e8m0_value(b) == 2.0 ** (b - 127)


def test_e8m0_exhaustive_against_bisection(sweeps_lib):
    first = ctypes.c_uint32(0)
    bad = sweeps_lib.sweep_e8m0_all(ctypes.byref(first))
    assert bad == 0, f"{bad} mismatches, first at bits {first.value:#010x}"


def test_mx_matches_exact_rational_model():
    rng = np.random.default_rng(23)
    for i in range(400):
        rows = int(rng.integers(1, 3))
        cols = 32 * int(rng.integers(1, 3))
        v = rng.standard_normal(rows * cols) * np.exp2(rng.integers(-40, 40, rows * cols))
        if i % 4 == 0:
            v[rng.integers(0, v.size, 3)] = 0.0
        if i % 4 == 1:
            v = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], v.size) * \
                np.exp2(float(rng.integers(-3, 4))) * rng.choice([-1.0, 1.0], v.size)
        if i % 2:
            x = v.astype(np.float32).reshape(rows, cols)
            xf = x
        else:
            x = _bf16(v).reshape(rows, cols)
            xf = synth.bf16_to_f32(x)
        for rotate in (False, True):
            q, s = oracle.mx_quantize(x, rotate)
            mq, ms = em.mx_quantize(xf, rotate)
            assert np.array_equal(q, mq) and np.array_equal(s, ms), (i, rotate)


def test_mx_block_maximum_maps_into_3_to_6():
    """With the smallest power of two at or above amax/6, every nonzero block's
    largest |code| is 5, 6 or 7 (its largest value lands in (3, 6])."""
    w = synth.make("t3_lognormal_16384x8192", rows=64)
    for rotate in (True, False):
        q, s = oracle.mx_quantize(w.x, rotate)
        codes = np.stack([q & 15, q >> 4], -1).reshape(-1, 32) & 7
        top = codes.max(1)
        assert np.all((top >= 5) & (top <= 7))


def test_mx_storage_is_4p25_bits_per_value():
    x = synth.normal_bf16(256 * 64, seed=3).reshape(256, 64)
    q, s = oracle.mx_quantize(x, True)
    assert (q.size + s.size) / x.size == 0.53125


def test_mx_underflow_sign_rule():
    """A tiny negative value in a block with a huge one underflows to -0 and
    takes code 0 (sign bit only when the quotient compares below zero)."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 2.0 ** 100
    x[0, 1] = -(2.0 ** -140)
    x[0, 2] = -(2.0 ** -40)
    q, s = oracle.mx_quantize(x, False)
    codes = np.stack([q & 15, q >> 4], -1).reshape(-1)
    assert s[0, 0] == 98 + 127            # 2^100 / 6 rounds up to 2^98
    assert codes[0] == 6 and codes[1] == 0 and codes[2] == 8


def test_mx_dequant_inverts_exactly_representable_blocks():
    """Two 16-element halves whose (rotated) values are E2M1 grid points times
    2^k, with a largest magnitude of 6 * 2^k, so the block scale is exactly
    2^k: encode then decode returns the input exactly, for either rotation
    setting and for scales from 2^-120 to 2^120."""
    t = np.array([6, -4, 3, 2, -1.5, 1, 0.5, 0, -6, 4, -3, 2, 1.5, -1, 0.5, 0,
                  0.5, 6, -0.5, 1, 1.5, -2, 3, -4, 0, 0, 1, -1, 2, -2, 4, -3],
                 dtype=np.float64)
    H = sylvester16()
    for k in (-120, -7, 0, 5, 120):
        for rotate in (False, True):
            y = t * 2.0 ** k
            x = np.concatenate([H @ y[:16], H @ y[16:]]) if rotate else y
            x32 = x.astype(np.float32).reshape(1, 32)
            assert np.array_equal(x32.astype(np.float64).reshape(-1), x)   # exact input
            q, s = oracle.mx_quantize(x32, rotate)
            assert s[0, 0] == k + 127
            back = oracle.mx_dequant_f64(q, s, rotate)
            assert np.array_equal(back.reshape(-1), x), (k, rotate)


# ---------------------------------------------------------------- rotation alone

def test_rotate_tensor_is_blockwise_sylvester_product():
    """Small-integer inputs: every partial sum is exact, so the tensor rotation
    equals X H (fp64, exact H) block by block, in row-major block order."""
    rng = np.random.default_rng(8)
    rows, cols = 7, 80
    x = rng.integers(-1000, 1000, rows * cols).astype(np.float32).reshape(rows, cols)
    H = sylvester16()
    want = (x.astype(np.float64).reshape(-1, 16) @ H).reshape(rows, cols)
    assert np.array_equal(oracle.rotate_tensor(x).astype(np.float64), want)
    xb = _bf16(x.astype(np.float64).reshape(-1)).reshape(rows, cols)
    wb = (synth.bf16_to_f32(xb).astype(np.float64).reshape(-1, 16) @ H).reshape(rows, cols)
    assert np.array_equal(oracle.rotate_tensor(xb).astype(np.float64), wb)


def test_quantizing_the_stored_rotation_equals_the_fused_definition():
    """Rotate to fp32 first, then quantize with rotation off: the same bytes,
    scale and amax as quantizing with rotation on (the unfused arrangement
    computes the same function)."""
    for name in ("gauss_outliers_128x1024", "t3_lognormal_16384x8192"):
        w = synth.make(name, rows=128)
        y = oracle.rotate_tensor(w.x)
        a = oracle.quantize(w.x, True)
        b = oracle.quantize(y, False)
        for u, v in zip(a, b):
            assert np.array_equal(np.asarray(u), np.asarray(v)), name


# ---------------------------------------------------------------- swizzled scales

def _swizzle_by_reshape(s: np.ndarray) -> np.ndarray:
    """The tiled layout as a tensor reshape: pad to [128 RT, 4 CT], view as
    [RT, 4 (i), 32 (j), CT, 4 (k)] with row = 128 rt + 32 i + j, then order the
    axes (rt, ct, j, i, k)."""
    rows, cb = s.shape
    rt, ct = -(-rows // 128), -(-cb // 4)
    pad = np.zeros((rt * 128, ct * 4), dtype=np.uint8)
    pad[:rows, :cb] = s
    return pad.reshape(rt, 4, 32, ct, 4).transpose(0, 3, 2, 1, 4).reshape(-1)


@pytest.mark.parametrize("rows,cb", [(1, 1), (128, 4), (129, 5), (300, 7), (256, 512), (77, 260)])
def test_swizzle_matches_the_tensor_reshape_form(rows, cb):
    rng = np.random.default_rng(rows * 1000 + cb)
    s = rng.integers(1, 255, (rows, cb), dtype=np.uint8)
    out = oracle.swizzle_scales(s)
    assert out.size == oracle.swizzled_scale_bytes(rows, cb) == (-(-rows // 128)) * (-(-cb // 4)) * 512
    assert np.array_equal(out, _swizzle_by_reshape(s))
    # every scale appears exactly once; the rest is zero padding
    assert np.count_nonzero(out) == rows * cb


def test_swizzle_worked_positions():
    """Hand-placed entries: a 256 x 8 scale matrix has 2 x 2 tiles."""
    s = np.zeros((256, 8), dtype=np.uint8)
    s[0, 0], s[33, 5], s[127, 3], s[128, 0], s[255, 7], s[40, 4] = 1, 2, 3, 4, 5, 6
    out = oracle.swizzle_scales(s)
    assert out[0] == 1
    assert out[512 + 16 * 1 + 4 * 1 + 1] == 2        # tile (0,1), j=1, i=1, k=1
    assert out[16 * 31 + 4 * 3 + 3] == 3             # last byte of tile (0,0)
    assert out[2 * 512] == 4                         # tile (1,0) starts the second tile row
    assert out[4 * 512 - 1] == 5                     # last byte of tile (1,1)
    assert out[512 + 16 * 8 + 4 * 1 + 0] == 6        # row 40: j=8, i=1; column 4: k=0


# ---------------------------------------------------------------- general block rotation ("Try this" 3)

def test_rotate_matrix_identity_and_permutation():
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((5, 64)) * 1e3).astype(np.float32)
    assert np.array_equal(oracle.rotate_matrix(x, np.eye(16, dtype=np.float32)), x)
    perm = rng.permutation(16)
    P = np.zeros((16, 16), dtype=np.float32)
    P[perm, np.arange(16)] = 1.0          # y_j = x_perm[j]
    want = x.reshape(-1, 16)[:, perm].reshape(5, 64)
    assert np.array_equal(oracle.rotate_matrix(x, P), want)
    xb = _bf16(x.astype(np.float64).reshape(-1)).reshape(5, 64)
    assert np.array_equal(oracle.rotate_matrix(xb, np.eye(16, dtype=np.float32)), synth.bf16_to_f32(xb))


def test_rotate_matrix_with_the_hadamard_equals_the_butterfly_when_exact():
    """Small integers times +-1/4: every product and partial sum is exact in
    either order, so the dense product equals the butterfly."""
    rng = np.random.default_rng(32)
    x = rng.integers(-1000, 1000, 6 * 48).astype(np.float32).reshape(6, 48)
    H = sylvester16().astype(np.float32)      # entries +-1/4
    assert np.array_equal(oracle.rotate_matrix(x, H), oracle.rotate_tensor(x))


def test_rotate_matrix_follows_the_fused_multiply_add_order():
    """Exact rational model of acc = RN(x0 r0j), acc = RN(xk rkj + acc):
    bit for bit on random blocks and a random orthogonal matrix (a separately
    rounded multiply and add, or another order, differs on such data)."""
    rng = np.random.default_rng(33)
    R = synth.random_orthogonal16(5)
    x = (rng.standard_normal((3, 16 * 8)) * np.exp2(rng.uniform(-20, 20, size=(3, 1)))).astype(np.float32)
    got = oracle.rotate_matrix(x, R).reshape(-1, 16)
    Rf = [[em.f32_to_frac(R[k, j]) for j in range(16)] for k in range(16)]
    for bi, blk in enumerate(x.reshape(-1, 16)):
        xf = [em.f32_to_frac(v) for v in blk]
        for j in range(16):
            acc = em.rn32(xf[0] * Rf[0][j])
            for k in range(1, 16):
                acc = em.rn32(xf[k] * Rf[k][j] + acc)
            assert got[bi, j] == em.frac_to_f32(acc), (bi, j)
    # the separately rounded variant really differs somewhere on this data
    diff = 0
    for bi, blk in enumerate(x.reshape(-1, 16)):
        xf = [em.f32_to_frac(v) for v in blk]
        for j in range(16):
            acc = em.rn32(xf[0] * Rf[0][j])
            for k in range(1, 16):
                acc = em.rn32(em.rn32(xf[k] * Rf[k][j]) + acc)
            diff += got[bi, j] != em.frac_to_f32(acc)
    assert diff > 0


def test_rotate_matrix_error_bound_and_round_trip():
    """Against the fp64 product: |y - x R| <= gamma_16 sum_k |x_k r_kj|; and
    rotating back with R^T returns x up to the same kind of bound (plus R's
    own distance from orthogonality)."""
    rng = np.random.default_rng(34)
    R = synth.random_orthogonal16(6)
    x = (rng.standard_normal((40, 160)) * 3.0).astype(np.float32)
    xb = x.reshape(-1, 16).astype(np.float64)
    R64 = R.astype(np.float64)
    y = oracle.rotate_matrix(x, R).reshape(-1, 16).astype(np.float64)
    u = 2.0 ** -24
    gamma = 16 * u / (1 - 16 * u)
    assert np.all(np.abs(y - xb @ R64) <= gamma * (np.abs(xb) @ np.abs(R64)))
    z = oracle.rotate_matrix(y.astype(np.float32).reshape(40, 160), np.ascontiguousarray(R.T))
    orth = np.abs(R64 @ R64.T - np.eye(16)).max()
    bound = (2 * gamma + 16 * orth) * (np.abs(xb) @ (np.abs(R64) @ np.abs(R64.T))) + 1e-30
    assert np.all(np.abs(z.reshape(-1, 16) - xb) <= bound)
