"""GPU parity of the MXFP4 variant: the HIP library, called through its C ABI,
against the CPU oracle.

MXFP4 is the contrast format of the page "A Fused Hadamard + NVFP4
Quantization Kernel in Triton" (section 1: 32-element blocks with power-of-two
E8M0 scales; the "Try this" list asks for the rotation's effect under it).
Bar: codes and scale bytes identical byte for byte; the decoded round trip
within 1e-6 relative of the oracle's fp64 decode.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_activation_amd as nv
    return nv


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(x).to("cuda:0")


def compare(tag, x_np, rotate, got, ref=None):
    q, s = [t.cpu().numpy() if torch.is_tensor(t) else t for t in got]
    oq, os_ = oracle.mx_quantize(x_np, rotate) if ref is None else ref
    msgs = []
    if not np.array_equal(s, os_):
        bad = np.argwhere(s != os_)
        msgs.append(f"{len(bad)} scale bytes differ, first {bad[0].tolist()}: "
                    f"{s[tuple(bad[0])]} vs {os_[tuple(bad[0])]}")
    if not np.array_equal(q, oq):
        bad = np.argwhere(q != oq)
        msgs.append(f"{len(bad)} code bytes differ, first {bad[0].tolist()}: "
                    f"{q[tuple(bad[0])]:#04x} vs {oq[tuple(bad[0])]:#04x}")
    assert not msgs, f"{tag}: " + "; ".join(msgs)


def mixed_input(rows, cols, dtype, seed, spread=2.0):
    n = rows * cols
    v = synth.normal_f64(n, seed=seed, stream=1) * np.exp(spread * synth.normal_f64(n, seed=seed,
                                                                                    stream=2))
    if dtype == "bf16":
        return synth.round_bf16(v).reshape(rows, cols)
    return v.astype(np.float32).reshape(rows, cols)


SHAPES = [(1, 32), (3, 96), (127, 32), (5, 1024), (300, 4128), (1000, 1056), (257, 8192),
          (65536, 32), (4099, 64)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rotate", [True, False])
def test_small_shapes(nv, rows, cols, dtype, rotate):
    x = mixed_input(rows, cols, dtype, seed=rows * 31 + cols)
    got = nv.mx_rotquant(to_dev(x), rotate=rotate)
    torch.cuda.synchronize()
    compare(f"{rows}x{cols} {dtype} rotate={rotate}", x, rotate, got)


WORKLOAD_CASES = [(name, rot) for name, (_, _, _, rots) in synth.WORKLOADS.items() for rot in rots]


@pytest.mark.parametrize("name,rotate", WORKLOAD_CASES)
def test_workload_full_size(nv, name, rotate):
    say(f"[mx parity] {name} rotate={rotate}: generating")
    w = synth.make(name, rotate=rotate)
    xd = to_dev(w.x)
    got = [t.cpu() for t in nv.mx_rotquant(xd, rotate=rotate)]
    del xd
    say(f"[mx parity] {name}: oracle")
    compare(f"{name} rotate={rotate}", w.x, rotate, got)
    say(f"[mx parity] {name}: ok")


def test_zero_and_negative_zero(nv):
    for dtype in ("bf16", "f32"):
        x = np.zeros((4, 64), dtype=np.float32)
        x[1] = -0.0
        x[2, :32] = -0.0
        x[2, 32] = 1.0
        x[3, 5] = -(2.0 ** -130)
        if dtype == "bf16":
            x = synth.round_bf16(x.astype(np.float64)).reshape(4, 64)
        for rotate in (True, False):
            q, s = nv.mx_rotquant(to_dev(x), rotate=rotate)
            torch.cuda.synchronize()
            compare(f"zeros {dtype} rotate={rotate}", x, rotate, (q, s))
            assert s.cpu().numpy()[0, 0] == 0 and not q.cpu().numpy()[:2].any()


def test_empty(nv):
    for rows, cols in ((0, 64), (5, 0), (0, 0)):
        x = torch.empty(rows, cols, dtype=torch.bfloat16, device="cuda:0")
        q, s = nv.mx_rotquant(x)
        torch.cuda.synchronize()
        assert q.numel() == 0 and s.numel() == 0


def test_scale_boundaries(nv):
    """Block maxima at 6 * 2^k and one binary32 step either side: the quotient
    fl(amax / 6) lands on, just above or rounds onto a power of two."""
    rows = []
    for k in range(-130, 118, 7):
        for step in (-2, -1, 0, 1, 2):
            m = np.float32(6.0 * 2.0 ** k) if 6.0 * 2.0 ** k >= 2.0 ** -149 else np.float32(2 ** -149)
            for _ in range(abs(step)):
                m = np.nextafter(m, np.float32(np.inf) if step > 0 else np.float32(0))
            r = np.linspace(-1, 1, 32, dtype=np.float64) * float(m)
            r[7] = float(m)
            rows.append(r.astype(np.float32))
    x = np.stack(rows)
    for rotate in (False, True):
        got = nv.mx_rotquant(to_dev(x), rotate=rotate)
        torch.cuda.synchronize()
        compare(f"boundaries rotate={rotate}", x, rotate, got)
    xb = synth.round_bf16(x.astype(np.float64)).reshape(x.shape)
    for rotate in (False, True):
        got = nv.mx_rotquant(to_dev(xb), rotate=rotate)
        torch.cuda.synchronize()
        compare(f"boundaries bf16 rotate={rotate}", xb, rotate, got)


def test_extreme_magnitudes_and_underflow(nv):
    """Values from 2^-149 to 2^123 in one tensor; blocks where a huge value
    sends tiny ones (negative included) below the smallest quotient."""
    rng = np.random.default_rng(11)
    n = 512 * 64
    v = rng.standard_normal(n) * np.exp2(rng.integers(-149, 121, n).astype(np.float64))
    v[::97] = -(2.0 ** -140)
    v[::101] = 2.0 ** 100
    for dtype in ("bf16", "f32"):
        x = (synth.round_bf16(v) if dtype == "bf16" else v.astype(np.float32)).reshape(512, 64)
        for rotate in (True, False):
            got = nv.mx_rotquant(to_dev(x), rotate=rotate)
            torch.cuda.synchronize()
            compare(f"extremes {dtype} rotate={rotate}", x, rotate, got)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_launch_shape_invariance(nv, monkeypatch, dtype):
    x = mixed_input(777, 2080, dtype, seed=99)
    xd = to_dev(x)
    ref = [t.clone() for t in nv.mx_rotquant(xd)]
    torch.cuda.synchronize()
    compare(f"default shape {dtype}", x, True, ref)
    for wgs in (1, 3, 64, 1000, 100000):
        monkeypatch.setenv("NVFP4RQ_QUANT_WGS", str(wgs))
        got = nv.mx_rotquant(xd)
        torch.cuda.synchronize()
        for r, g in zip(ref, got):
            assert torch.equal(r, g), wgs


@pytest.mark.parametrize("name,rotate", WORKLOAD_CASES)
def test_dequant_round_trip(nv, name, rotate):
    w = synth.make(name, rotate=rotate, rows=min(synth.WORKLOADS[name][0], 2048))
    xd = to_dev(w.x)
    q, s = nv.mx_rotquant(xd, rotate=rotate)
    y = nv.mx_dequant(q, s, rotate=rotate)
    torch.cuda.synchronize()
    xf = xd.double()
    e_gpu = ((y.double() - xf).norm() / xf.norm()).item()
    oq, os_ = oracle.mx_quantize(w.x, rotate)
    e_ora = oracle.mx_roundtrip_error(w.x, rotate, oq, os_)
    assert abs(e_gpu - e_ora) <= 1e-6 * e_ora, (e_gpu, e_ora)
    yd = oracle.mx_dequant_f64(oq, os_, rotate)
    err = np.abs(y.cpu().numpy().astype(np.float64) - yd)
    # fp32 decode: each output is a 16-term signed sum, rounded per step
    assert np.all(err <= 1e-6 * np.abs(yd).reshape(-1, 16).max(1).repeat(16).reshape(yd.shape))


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("rotate", [True, False])
def test_dequant_small_shapes(nv, rows, cols, rotate):
    x = mixed_input(rows, cols, "f32", seed=rows * 17 + cols)
    q, s = nv.mx_rotquant(to_dev(x), rotate=rotate)
    y = nv.mx_dequant(q, s, rotate=rotate)
    torch.cuda.synchronize()
    compare(f"{rows}x{cols} rotate={rotate}", x, rotate, (q, s))
    yd = oracle.mx_dequant_f64(q.cpu().numpy(), s.cpu().numpy(), rotate)
    tol = 1e-6 * np.abs(yd).reshape(-1, 16).max(1).repeat(16).reshape(yd.shape)
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - yd) <= tol)
