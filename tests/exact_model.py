"""Exact-rational model of the rotate+quantize definition (test code).

Every quantity is a ``fractions.Fraction``; each binary32 operation of the
definition is computed exactly and then rounded by ``rn32``, a correct
round-to-nearest-even onto the binary32 grid (subnormals included) written
from the format's definition.  The E4M3 and E2M1 steps are nearest-point
searches over their grids (ties to the even byte / even code).  The model
shares nothing with the C oracle: it pins the oracle on small tensors, bit for
bit (page "A Fused Hadamard + NVFP4 Quantization Kernel in Triton",
sections 1-3).

Zero has no sign here; in the method the sign of a zero never changes an
output (a zero quotient has code 0 whatever its sign, and zeros only meet
abs/max elsewhere), so the model needs none.
"""
from __future__ import annotations

import struct
from fractions import Fraction as F

import numpy as np

F0 = F(0)


def f32_to_frac(x) -> F:
    return F(float(np.float32(x)))


def frac_to_f32(x: F) -> np.float32:
    # exact: x is on the binary32 grid
    return np.float32(float(x))


def _floor_log2(a: F) -> int:
    """e with 2^e <= a < 2^(e+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    elif F(2) ** (e + 1) <= a:
        e += 1
    return e


def rn32(x: F) -> F:
    """Round a rational to the nearest binary32 value, ties to even."""
    if x == 0:
        return F0
    neg = x < 0
    a = -x if neg else x
    e = max(_floor_log2(a), -126)
    quantum = F(2) ** (e - 23)
    k = a / quantum
    n = k.numerator // k.denominator
    rem = k - n
    if rem > F(1, 2) or (rem == F(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= F(2) ** 128:
        raise OverflowError("binary32 overflow")
    return -r if neg else r


def rn32_sat(x: F) -> F:
    """rn32, with results beyond the largest binary32 given as +-2^128 (they
    stand for +-inf: every such quotient has the largest E2M1 code)."""
    try:
        return rn32(x)
    except OverflowError:
        return F(2) ** 128 if x > 0 else -(F(2) ** 128)


# ------------------------------------------------------------------ grids

GRID_E2M1 = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


def _e4m3_values():
    vals = []
    for b in range(127):
        e, m = b >> 3, b & 7
        if e == 0:
            vals.append(F(m, 512))
        else:
            vals.append((1 + F(m, 8)) * F(2) ** (e - 7))
    return vals


E4M3_VALUES = _e4m3_values()


def e4m3_nearest(v: F) -> int:
    """Byte of the nearest E4M3 value (ties to the even byte), 448 for v >= 448."""
    if v >= 448:
        return 0x7E
    best, bd = 0, None
    for b, val in enumerate(E4M3_VALUES):
        d = abs(v - val)
        if bd is None or d < bd or (d == bd and b % 2 == 0):
            best, bd = b, d
    return best


def e2m1_nearest(v: F) -> int:
    a = abs(v)
    best, bd = 0, None
    for k, gv in enumerate(GRID_E2M1):
        d = abs(a - gv)
        if bd is None or d < bd or (d == bd and k % 2 == 0):
            best, bd = k, d
    return best + (8 if v < 0 else 0)


# ------------------------------------------------------------------ method

def rotate16(x: list[F]) -> list[F]:
    """Butterfly with strides 1, 2, 4, 8 ((a, b) -> (a+b, a-b)), then x0.25."""
    z = list(x)
    h = 1
    while h < 16:
        for i in range(16):
            if i & h == 0:
                a, b = z[i], z[i + h]
                z[i], z[i + h] = rn32(a + b), rn32(a - b)
        h *= 2
    return [rn32(F(1, 4) * v) for v in z]


def _blocks(x_f32: np.ndarray, rotate: bool):
    flat = x_f32.reshape(-1)
    out = []
    for b in range(flat.size // 16):
        xb = [f32_to_frac(v) for v in flat[16 * b:16 * b + 16]]
        out.append(rotate16(xb) if rotate else xb)
    return out


def global_scale(amax: F) -> F:
    g = rn32(rn32(amax / 6) / 448)
    return F(1) if g == 0 else g


def quantize(x_f32: np.ndarray, rotate: bool):
    """x_f32: float32 [rows, cols] (bf16 inputs are widened exactly first).
    Returns (q uint8 [rows, cols/2], s uint8 [rows, cols/16], g float32, amax float32)."""
    blocks = _blocks(x_f32, rotate)
    amax = max((abs(v) for blk in blocks for v in blk), default=F0)
    g = global_scale(amax)
    q, s = _encode(blocks, g, x_f32.shape)
    return q, s, frac_to_f32(g), frac_to_f32(amax)


def quantize_given_scale(x_f32: np.ndarray, rotate: bool, g: F):
    """Same block arithmetic with a global scale supplied by the caller."""
    return _encode(_blocks(x_f32, rotate), g, x_f32.shape)


def _encode(blocks, g: F, shape):
    rows, cols = shape
    nb = rows * cols // 16
    q = np.zeros(nb * 8, dtype=np.uint8)
    s = np.zeros(nb, dtype=np.uint8)
    for b, y in enumerate(blocks):
        ab = max(abs(v) for v in y)
        v = rn32_sat(rn32(ab / 6) / g)
        sb = e4m3_nearest(v)
        sf = rn32(E4M3_VALUES[sb] * g)
        d = F(1) if sf == 0 else sf
        codes = [e2m1_nearest(rn32_sat(yi / d)) for yi in y]
        for k in range(8):
            q[8 * b + k] = codes[2 * k] | (codes[2 * k + 1] << 4)
        s[b] = sb
    return q.reshape(rows, cols // 2), s.reshape(rows, cols // 16)


def f32_bits(x: np.float32) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


# ------------------------------------------------------------------ MXFP4 variant

def e8m0_smallest_power_at_or_above(t: F) -> int:
    """Byte of the smallest power of two >= t, exponent clamped to [-127, 127];
    0 for t == 0 (search over the 255 representable scales)."""
    if t == 0:
        return 0
    for b in range(255):
        if F(2) ** (b - 127) >= t:
            return b
    return 254


def mx_quantize(x_f32: np.ndarray, rotate: bool):
    rows, cols = x_f32.shape
    flat = x_f32.reshape(-1)
    nb = flat.size // 32
    q = np.zeros(nb * 16, dtype=np.uint8)
    s = np.zeros(nb, dtype=np.uint8)
    for b in range(nb):
        xb = [f32_to_frac(v) for v in flat[32 * b:32 * b + 32]]
        y = (rotate16(xb[:16]) + rotate16(xb[16:])) if rotate else xb
        ab = max(abs(v) for v in y)
        sb = e8m0_smallest_power_at_or_above(rn32(ab / 6))
        scale = F(2) ** (sb - 127)
        codes = [e2m1_nearest(rn32(yi / scale)) for yi in y]
        for k in range(16):
            q[16 * b + k] = codes[2 * k] | (codes[2 * k + 1] << 4)
        s[b] = sb
    return q.reshape(rows, cols // 2), s.reshape(rows, cols // 32)
