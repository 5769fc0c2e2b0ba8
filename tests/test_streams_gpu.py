"""Calls on several streams at once: the library keeps no state between calls
(pass 1's maxima and the arrival counters live at the head of each call's own
q_out), so fused calls with distinct buffers may overlap on different streams
and each must still match the oracle byte for byte."""
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


def make(rows, cols, dtype, seed):
    z = synth.normal_f64(rows * cols, seed=seed, stream=1)
    m = synth.normal_f64(rows * cols, seed=seed, stream=2)
    v = z * np.exp(1.5 * m)
    if dtype == "bf16":
        return synth.round_bf16(v).reshape(rows, cols)
    return v.astype(np.float32).reshape(rows, cols)


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(x).to("cuda:0")


CASES = [(2048, 4096, "bf16"), (1024, 8192, "bf16"), (4096, 1024, "f32"), (300, 4112, "bf16"),
         (64, 1024, "bf16"), (3000, 2048, "f32")]


@pytest.mark.parametrize("entry", ["rotquant", "rotquant_swizzled", "mx_rotquant"])
def test_overlapping_calls_on_separate_streams(nv, entry):
    cases = [cs for cs in CASES if entry != "mx_rotquant" or cs[1] % 32 == 0]
    xs = [make(r, c, d, seed=40 + i) for i, (r, c, d) in enumerate(cases)]
    xd = [to_dev(x) for x in xs]
    streams = [torch.cuda.Stream() for _ in cases]
    torch.cuda.synchronize()
    outs = [None] * len(cases)
    say(f"{entry}: {len(cases)} streams")
    for rep in range(3):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                outs[i] = getattr(nv, entry)(xd[i])   # on the current stream, st
        torch.cuda.synchronize()
        for i, ((r, c, d), x) in enumerate(zip(cases, xs)):
            got = [t.cpu().numpy() for t in outs[i]]
            if entry == "rotquant":
                oq, os_, og, oa = oracle.quantize(x, True)
                assert np.array_equal(got[0], oq) and np.array_equal(got[1], os_), (rep, i)
                assert got[2].view(np.uint32)[0] == np.float32(og).view(np.uint32), (rep, i)
                assert got[3].view(np.uint32)[0] == np.float32(oa).view(np.uint32), (rep, i)
            elif entry == "rotquant_swizzled":
                oq, os_, og, oa = oracle.quantize(x, True)
                assert np.array_equal(got[0], oq), (rep, i)
                assert np.array_equal(got[1], oracle.swizzle_scales(os_)), (rep, i)
                assert got[2].view(np.uint32)[0] == np.float32(og).view(np.uint32), (rep, i)
            else:
                oq, os_ = oracle.mx_quantize(x, True)
                assert np.array_equal(got[0], oq) and np.array_equal(got[1], os_), (rep, i)
