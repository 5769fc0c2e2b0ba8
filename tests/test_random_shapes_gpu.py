"""Seeded randomized differential test: many shapes (ragged row counts, column
counts from one block to hundreds; every 20th case 897-1024 rows of 241-256
blocks), both input dtypes, both rotation settings,
magnitudes spread over most of the binary32 range, planted zero and -0.0
blocks.  Every quantize entry point must match the oracle byte for byte."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

N_CASES = 160


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_activation_amd as nv
    return nv


def case(i: int):
    rng = np.random.default_rng(1000 + i)
    rows = int(rng.integers(1, 700))
    kb = int(rng.integers(1, 300))
    if i % 20 == 19:
        # 8 row tiles (the last ragged) of 16 column windows: the swizzled
        # pass then gives each XCD runs of 16 windows
        rows = int(rng.integers(897, 1025))
        kb = int(rng.integers(241, 257))
    cols = 16 * kb
    dtype = "bf16" if i % 3 else "f32"
    rotate = bool(i % 2)
    n = rows * cols
    z = synth.normal_f64(n, seed=2000 + i, stream=1)
    # per-row magnitudes 2^(c + U(-w, w)) with the spread w cycling through
    # 0, 4, 20 and 40 (narrow spreads keep the bf16 fast path in play),
    # times a per-element log-normal spread
    span = (0.0, 4.0, 20.0, 40.0)[i % 4]
    row_exp = rng.uniform(-30.0, 10.0) + rng.uniform(-span, span, size=rows)
    m = synth.normal_f64(n, seed=2000 + i, stream=2)
    v = (z * np.exp(1.2 * m)).reshape(rows, cols) * np.exp2(row_exp)[:, None]
    blocks = v.reshape(rows, kb, 16)
    nz = max(1, rows * kb // 50)
    zr = rng.integers(0, rows, size=nz)
    zc = rng.integers(0, kb, size=nz)
    blocks[zr, zc, :] = 0.0
    blocks[zr[: nz // 2], zc[: nz // 2], :] = -0.0
    if dtype == "bf16":
        x = synth.round_bf16(v)
    else:
        x = v.astype(np.float32)
    return rows, cols, dtype, rotate, x


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(x).to("cuda:0")


def bits(v) -> int:
    return int(np.asarray(v, dtype=np.float32).reshape(-1)[0].view(np.uint32))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(nv, i):
    rows, cols, dtype, rotate, x = case(i)
    say(f"case {i}: {rows}x{cols} {dtype} rotate={rotate}")
    xd = to_dev(x)
    oq, os_, og, oa = oracle.quantize(x, rotate)

    q, s, g, a = nv.rotquant(xd, rotate=rotate)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)
    assert bits(g.cpu().numpy()) == bits(og) and bits(a.cpu().numpy()) == bits(oa)

    qs, ss, gs, _ = nv.rotquant_swizzled(xd, rotate=rotate)
    torch.cuda.synchronize()
    assert np.array_equal(qs.cpu().numpy(), oq)
    assert np.array_equal(ss.cpu().numpy(), oracle.swizzle_scales(os_))

    # given scale: an amax a power of two away from the tensor's own
    kept = np.float32(oa) * np.float32(2.0 ** ((i % 5) - 2)) if oa > 0 else np.float32(1.0)
    kd = torch.tensor([kept], dtype=torch.float32, device="cuda:0")
    q2, s2, g2 = nv.quant_from_amax(xd, kd, rotate=rotate)
    torch.cuda.synchronize()
    gq, gs_ = oracle.quantize_given_scale(x, rotate, oracle.global_scale(kept))
    assert np.array_equal(q2.cpu().numpy(), gq) and np.array_equal(s2.cpu().numpy(), gs_)

    if cols % 32 == 0:
        mq, ms = nv.mx_rotquant(xd, rotate=rotate)
        torch.cuda.synchronize()
        omq, oms = oracle.mx_quantize(x, rotate)
        assert np.array_equal(mq.cpu().numpy(), omq) and np.array_equal(ms.cpu().numpy(), oms)
