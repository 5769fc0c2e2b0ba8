"""Caller-supplied output buffers: the library receives only addresses, so the
binding must refuse a buffer of the wrong size, dtype, device or layout before
anything is launched, and must accept a correct one (results equal to those
of the call that allocates its own outputs)."""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu

ROWS, COLS = 64, 256


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_activation_amd as nv
    return nv


@pytest.fixture(scope="module")
def x():
    g = torch.Generator().manual_seed(11)
    return torch.randn(ROWS, COLS, generator=g).to(torch.bfloat16).to("cuda:0")


def u8(n, device="cuda:0"):
    return torch.empty(n, dtype=torch.uint8, device=device)


def f32(n, device="cuda:0"):
    return torch.empty(n, dtype=torch.float32, device=device)


def good4(nv, s_bytes):
    return [u8(ROWS * COLS // 2), u8(s_bytes), f32(1), f32(1)]


BAD = {
    "short": lambda t: t.new_empty(t.numel() - 1),
    "dtype": lambda t: torch.empty(t.numel(), dtype=torch.int32 if t.dtype == torch.uint8
                                   else torch.float64, device=t.device),
    "host": lambda t: torch.empty(t.numel(), dtype=t.dtype),
    "strided": lambda t: t.new_empty(2 * t.numel())[::2],
}


@pytest.mark.parametrize("which", range(4))
@pytest.mark.parametrize("kind", sorted(BAD))
@pytest.mark.parametrize("entry", ["rotquant", "rotquant_timed", "rotquant_swizzled"])
def test_fused_rejects_bad_buffers(nv, x, entry, which, kind):
    s_bytes = (nv.swizzled_scale_bytes(ROWS, COLS) if entry == "rotquant_swizzled"
               else ROWS * COLS // 16)
    bufs = good4(nv, s_bytes)
    if kind == "strided" and which >= 2:
        pytest.skip("a one-element buffer has no layout to get wrong")
    bufs[which] = BAD[kind](bufs[which])
    with pytest.raises((ValueError, TypeError)):
        if entry == "rotquant_timed":
            events = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            for e in events:
                e.record()
            nv.rotquant_timed(x, events, out=tuple(bufs))
        else:
            getattr(nv, entry)(x, out=tuple(bufs))


@pytest.mark.parametrize("entry", ["rotquant", "rotquant_swizzled"])
def test_fused_accepts_exact_buffers(nv, x, entry):
    ref = getattr(nv, entry)(x)
    s_bytes = (nv.swizzled_scale_bytes(ROWS, COLS) if entry == "rotquant_swizzled"
               else ROWS * COLS // 16)
    bufs = good4(nv, s_bytes)
    if entry == "rotquant":
        bufs[0] = bufs[0].view(ROWS, COLS // 2)
        bufs[1] = bufs[1].view(ROWS, COLS // 16)
    got = getattr(nv, entry)(x, out=tuple(bufs))
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.reshape(-1), b.reshape(-1))


@pytest.mark.parametrize("which", range(3))
@pytest.mark.parametrize("kind", sorted(BAD))
def test_quant_from_amax_rejects_bad_buffers(nv, x, which, kind):
    amax = nv.rotamax(x)
    bufs = [u8(ROWS * COLS // 2), u8(ROWS * COLS // 16), f32(1)]
    if kind == "strided" and which == 2:
        pytest.skip("a one-element buffer has no layout to get wrong")
    bufs[which] = BAD[kind](bufs[which])
    with pytest.raises((ValueError, TypeError)):
        nv.quant_from_amax(x, amax, out=tuple(bufs))


@pytest.mark.parametrize("kind", ["dtype", "host", "short"])
def test_amax_argument_checked(nv, x, kind):
    bad = {"dtype": torch.empty(1, dtype=torch.float64, device="cuda:0"),
           "host": torch.empty(1, dtype=torch.float32),
           "short": torch.empty(0, dtype=torch.float32, device="cuda:0")}[kind]
    with pytest.raises((ValueError, TypeError)):
        nv.rotamax(x, amax=bad)
    with pytest.raises((ValueError, TypeError)):
        nv.quant_from_amax(x, bad)


@pytest.mark.parametrize("which", range(2))
@pytest.mark.parametrize("kind", sorted(BAD))
def test_mx_rejects_bad_buffers(nv, x, which, kind):
    bufs = [u8(ROWS * COLS // 2), u8(ROWS * COLS // 32)]
    bufs[which] = BAD[kind](bufs[which])
    with pytest.raises((ValueError, TypeError)):
        nv.mx_rotquant(x, out=tuple(bufs))


@pytest.mark.parametrize("kind", sorted(BAD))
def test_decoders_and_rotate_reject_bad_out(nv, x, kind):
    q, s, g, _ = nv.rotquant(x)
    qs, ss, gs, _ = nv.rotquant_swizzled(x)
    mq, ms = nv.mx_rotquant(x)
    bad = BAD[kind](f32(ROWS * COLS))
    with pytest.raises((ValueError, TypeError)):
        nv.dequant(q, s, g, out=bad)
    with pytest.raises((ValueError, TypeError)):
        nv.dequant_swizzled(qs, ss, gs, out=bad)
    with pytest.raises((ValueError, TypeError)):
        nv.mx_dequant(mq, ms, out=bad)
    with pytest.raises((ValueError, TypeError)):
        nv.rotate16(x, out=bad)


def test_decoders_reject_bad_inputs(nv, x):
    q, s, g, _ = nv.rotquant(x)
    qs, ss, gs, _ = nv.rotquant_swizzled(x)
    with pytest.raises((ValueError, TypeError)):
        nv.dequant(q, s, g.double())
    with pytest.raises((ValueError, TypeError)):
        nv.dequant(q.cpu(), s.cpu(), g.cpu())
    with pytest.raises((ValueError, TypeError)):
        nv.dequant(q, s.to(torch.int16), g)
    with pytest.raises((ValueError, TypeError)):
        nv.dequant_swizzled(qs, ss[:-1], gs)
    with pytest.raises((ValueError, TypeError)):
        nv.dequant_swizzled(qs, ss.cpu(), gs)
