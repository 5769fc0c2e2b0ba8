"""The calibration entry points (measurement support): the fused call's twin
runs on every launch path of the fused call (small tensors, per-workgroup
maxima, inputs of 512 MiB and more), the single-pass twin with a workgroup
per chunk; both leave their input unchanged and write nothing outside their
two output buffers."""
from __future__ import annotations

import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

GUARD = 4096


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def nv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import nvfp4_activation_amd as nv
    return nv


def guarded(n: int) -> tuple[torch.Tensor, torch.Tensor]:
    full = torch.full((n + 2 * GUARD,), 0xA5, dtype=torch.uint8, device="cuda:0")
    return full, full[GUARD:GUARD + n]


@pytest.mark.parametrize("rows,cols,dtype", [
    (4, 64, torch.bfloat16), (300, 4112, torch.bfloat16), (2048, 4096, torch.bfloat16),
    (4, 64, torch.float32), (2048, 4096, torch.float32), (16384, 16384, torch.bfloat16),
])
def test_calibration_stays_in_its_buffers(nv, rows, cols, dtype):
    say(f"calibrate {rows}x{cols} {dtype}")
    g = torch.Generator(device="cuda:0").manual_seed(rows + cols)
    x = torch.randn(rows, cols, generator=g, device="cuda:0").to(dtype)
    before = x.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).sum(dtype=torch.int64)
    n = rows * cols
    qf, q = guarded(n // 2)
    sf, s = guarded(n // 16)
    for _ in range(2):
        nv.stream_calibrate(x, out=(q, s))
        nv.stream_calibrate_single(x, out=(q, s))
    torch.cuda.synchronize()
    after = x.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).sum(dtype=torch.int64)
    assert torch.equal(before, after)
    for full in (qf, sf):
        assert bool((full[:GUARD] == 0xA5).all()) and bool((full[-GUARD:] == 0xA5).all())
