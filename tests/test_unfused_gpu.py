"""The rotation-alone entry point and the unfused three-kernel arrangement
(rotate to fp32 in HBM, amax, quantize: the comparison in the opening
paragraph and "Try this" item 4 of the page "A Fused Hadamard + NVFP4
Quantization Kernel in Triton"), against the oracle and the fused call; and
the section-5 error study through the library."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import read_golden

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


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (127, 16), (300, 4112), (257, 8192), (1000, 1040)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rotate16_matches_oracle(nv, rows, cols, dtype):
    n = rows * cols
    v = synth.normal_f64(n, seed=rows + cols, stream=1) * np.exp(
        2.0 * synth.normal_f64(n, seed=rows + cols, stream=2))
    x = (synth.round_bf16(v) if dtype == "bf16" else v.astype(np.float32)).reshape(rows, cols)
    y = nv.rotate16(to_dev(x)).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), oracle.rotate_tensor(x).view(np.uint32))


def test_rotate16_empty(nv):
    y = nv.rotate16(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda:0"))
    torch.cuda.synchronize()
    assert y.shape == (0, 64)


ROTATED = [name for name, (_, _, _, rots) in synth.WORKLOADS.items() if True in rots]


@pytest.mark.parametrize("name", ROTATED)
def test_three_kernels_equal_fused(nv, name):
    """rotate16, then rotamax and quant_from_amax on the fp32 rotation with
    rotation off: the fused call's bytes, scale and amax, and the oracle's."""
    say(f"[unfused] {name}")
    w = synth.make(name, rotate=True)
    xd = to_dev(w.x)
    fused = [t.cpu() for t in nv.rotquant(xd, rotate=True)]
    y = nv.rotate16(xd)
    a = nv.rotamax(y, rotate=False)
    q, s, g = nv.quant_from_amax(y, a, rotate=False)
    torch.cuda.synchronize()
    for u, v in zip(fused, (q, s, g, a)):
        assert torch.equal(u, v.cpu()), name
    del y, xd
    oq, os_, og, oa = oracle.quantize(w.x, True)
    assert np.array_equal(fused[0].numpy(), oq) and np.array_equal(fused[1].numpy(), os_)
    assert fused[2].numpy()[0] == og and fused[3].numpy()[0] == oa


def test_page_error_table_through_the_library(nv):
    """Section 5's printed table, reproduced by the GPU encode and decode (the
    page's tensors come from PyTorch's CPU generator, seed 0); the MXFP4
    columns agree with the oracle's fp64 round-trip errors."""
    from nvfp4_activation_amd import error_study as es
    expected = {r[0]: (float(r[1]), float(r[2])) for r in read_golden("error_table.txt")}
    tensors = es.section5_cases()
    assert sorted(tensors) == sorted(expected)
    rows = es.study(tensors, torch.from_numpy(synth.random_orthogonal16(0)).to("cuda:0"))
    for name, r in rows.items():
        plain, rot = expected[name]
        assert round(r["nvfp4_plain"], 4) == plain, (name, r)
        assert round(r["nvfp4_rotated"], 4) == rot, (name, r)
        t, cols = tensors[name]
        x = t.numpy().copy()
        mask = None if cols is None else cols.numpy().astype(np.uint8)
        for rotate, key in ((False, "mxfp4_plain"), (True, "mxfp4_rotated")):
            q, s = oracle.mx_quantize(x, rotate)
            if mask is None:
                e = oracle.mx_roundtrip_error(x, rotate, q, s)
                assert abs(r[key] - e) <= 1e-6 * e, (name, key, r[key], e)
            else:   # column subset: fp64 decode from the oracle, norms here
                xr = oracle.mx_dequant_f64(q, s, rotate)[:, mask.astype(bool)]
                xs = x.astype(np.float64)[:, mask.astype(bool)]
                e = np.linalg.norm(xr - xs) / np.linalg.norm(xs)
                assert abs(r[key] - e) <= 1e-6 * e, (name, key, r[key], e)
    say(es.table(rows))
