"""Every chunk of the input reaches the global amax, whatever the amax pass's
grid, and repeated fused calls never lose their global scale: a zero tensor with one planted value, moved through every 256-block
chunk (and through the lane and piece positions inside the chunks), must give
the planted value's rotated magnitude each time.  The amax pass maps its
workgroups to the input through an XCD-pairing remap when its grid is a
multiple of 16 and directly otherwise; a mapping that skipped or repeated a
region would lose the planted value there."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_activation_amd as nv
    return nv


@pytest.mark.parametrize("swizzled", [False, True])
@pytest.mark.parametrize("amax_wgs", [None, 48, 24])
@pytest.mark.parametrize("rotate", [True, False])
def test_every_chunk_reaches_the_amax(nv, monkeypatch, amax_wgs, rotate, swizzled):
    """Row-major and swizzled scales (the swizzled call keeps the maxima in its
    scale tiles and the counters in its first code rows; on this zero input the
    codes written over the counters are zero, so a premature head write would
    show as a NaN global scale)."""
    if amax_wgs is None:
        monkeypatch.delenv("NVFP4RQ_AMAX_WGS", raising=False)
    else:
        monkeypatch.setenv("NVFP4RQ_AMAX_WGS", str(amax_wgs))
    rows = cols = 4096
    nchunks = rows * cols // 16 // 256
    say(f"amax coverage: {nchunks} chunks, amax_wgs={amax_wgs}, rotate={rotate}, swizzled={swizzled}")
    dev = "cuda:0"
    x = torch.zeros(rows, cols, dtype=torch.bfloat16, device=dev)
    flat = x.view(-1)
    sbytes = nv.swizzled_scale_bytes(rows, cols) if swizzled else rows * cols // 16
    out = (torch.empty(rows, cols // 2, dtype=torch.uint8, device=dev),
           torch.empty(sbytes, dtype=torch.uint8, device=dev) if swizzled else
           torch.empty(rows, cols // 16, dtype=torch.uint8, device=dev),
           torch.empty(1, dtype=torch.float32, device=dev),
           torch.empty(1, dtype=torch.float32, device=dev))
    call = nv.rotquant_swizzled if swizzled else nv.rotquant
    got = torch.empty(nchunks, dtype=torch.float32, device=dev)
    got_g = torch.empty(nchunks, dtype=torch.float32, device=dev)
    big = 1024.0                       # exact in bf16; rotated, every output is +-256
    # element planted in chunk c: block (c * 37) % 256 of the chunk, lane c % 16
    pos = torch.tensor([(c * 256 + (c * 37) % 256) * 16 + c % 16 for c in range(nchunks)],
                       dtype=torch.int64, device=dev)
    # device-side index views and copies only: the loop never waits for the GPU
    for c in range(nchunks):
        flat.index_fill_(0, pos[c:c + 1], big)
        call(x, rotate=rotate, out=out)
        got[c:c + 1].copy_(out[3])
        got_g[c:c + 1].copy_(out[2])
        flat.index_fill_(0, pos[c:c + 1], 0.0)
    torch.cuda.synchronize()
    want = big / 4 if rotate else big
    missed = (got != want).nonzero().flatten().tolist()
    assert not missed, f"chunks whose planted value was lost: {missed[:20]} ({len(missed)} in all)"
    # the global scale of every call (a NaN would mean the quantize pass gave up
    # waiting for its own workgroups)
    g = np.float32(np.float32(want) / np.float32(6.0)) / np.float32(448.0)
    bad_g = (got_g != float(g)).nonzero().flatten().tolist()
    assert not bad_g, f"calls with a wrong global scale: {bad_g[:20]} ({len(bad_g)} in all)"


@pytest.mark.parametrize("swizzled", [False, True])
@pytest.mark.parametrize("rows,cols,calls", [(16384, 8192, 400), (2048, 8192, 2000), (4096, 4096, 2000)])
def test_repeated_calls_keep_the_global_scale(nv, monkeypatch, rows, cols, calls, swizzled):
    """Back-to-back fused calls on one set of buffers: every call's amax and
    global scale equal the oracle's.  The quantize workgroup that writes the
    head (of q_out, or of s_out and q_out for swizzled scales) first waits for
    every workgroup to have read pass 1's maxima there; a wait that ran out
    would leave a NaN global scale."""
    monkeypatch.delenv("NVFP4RQ_AMAX_WGS", raising=False)
    monkeypatch.delenv("NVFP4RQ_QUANT_WGS", raising=False)
    import oracle
    import synth
    say(f"repeated calls: {rows}x{cols}, {calls} calls")
    x = synth.normal_bf16(rows * cols, seed=rows + cols, stream=3).reshape(rows, cols)
    oq, os_, og, oa = oracle.quantize(x, True)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    sbytes = nv.swizzled_scale_bytes(rows, cols) if swizzled else rows * cols // 16
    out = (torch.empty(rows, cols // 2, dtype=torch.uint8, device="cuda:0"),
           torch.empty(sbytes, dtype=torch.uint8, device="cuda:0") if swizzled else
           torch.empty(rows, cols // 16, dtype=torch.uint8, device="cuda:0"),
           torch.empty(1, dtype=torch.float32, device="cuda:0"),
           torch.empty(1, dtype=torch.float32, device="cuda:0"))
    call = nv.rotquant_swizzled if swizzled else nv.rotquant
    gs = torch.empty(calls, dtype=torch.float32, device="cuda:0")
    am = torch.empty(calls, dtype=torch.float32, device="cuda:0")
    for c in range(calls):
        call(xd, rotate=True, out=out)
        gs[c:c + 1].copy_(out[2])
        am[c:c + 1].copy_(out[3])
    torch.cuda.synchronize()
    bad = ((gs != float(np.float32(og))) | (am != float(np.float32(oa)))).nonzero().flatten().tolist()
    assert not bad, f"calls with a wrong amax or global scale: {bad[:20]} ({len(bad)} in all)"
    want_s = oracle.swizzle_scales(os_) if swizzled else os_
    assert np.array_equal(out[0].cpu().numpy(), oq) and np.array_equal(out[1].cpu().numpy(), want_s)


@pytest.mark.parametrize("swizzled", [False, True])
@pytest.mark.parametrize("rows,cols", [(128, 1024), (257, 4096), (4096, 4096), (1000, 1040)])
def test_back_to_back_calls_over_stale_outputs(nv, rows, cols, swizzled):
    """2000 fused calls in a row, every output buffer filled with 0xFF (and the
    scalars with NaN) before each call, so that the head the next call builds
    in q_out or s_out always starts from stale bytes above any amax: every
    call's codes, scales, global scale and amax equal the first call's, byte
    for byte (compared on the device after each call)."""
    gen = torch.Generator(device="cuda:0").manual_seed(rows + cols)
    v = torch.randn(rows, cols, generator=gen, device="cuda:0")
    x = (v * torch.exp(2 * torch.randn(rows, cols, generator=gen, device="cuda:0"))).to(torch.bfloat16)
    call = nv.rotquant_swizzled if swizzled else nv.rotquant
    ref = [t.clone() for t in call(x)]
    outs = [t.clone() for t in ref]
    bad = torch.zeros((), dtype=torch.int64, device="cuda:0")
    for _ in range(2000):
        for o in outs:
            o.fill_(0xFF if o.dtype == torch.uint8 else float("nan"))
        call(x, out=tuple(outs))
        for a, b in zip(outs, ref):
            bad += (a.view(torch.uint8) != b.view(torch.uint8)).any().to(torch.int64)
    torch.cuda.synchronize()
    say(f"{rows}x{cols} swizzled={swizzled}: {int(bad.item())} of 2000 calls differ")
    assert int(bad.item()) == 0
