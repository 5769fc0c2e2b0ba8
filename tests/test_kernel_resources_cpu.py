"""Kernel resource guard (CPU): compile the library's device code for gfx950
and check every kernel's register use.  The quantize pass is pinned to 8 waves
per SIMD (64 VGPRs); past that the compiler spills to scratch memory, which
costs a large part of the pass's bandwidth without changing any result, so
only this test notices it.  Scalar registers the compiler parks in lanes of
a vector register (no memory traffic) are allowed; scratch memory is not."""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "nvfp4_activation_amd", "csrc")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "nvfp4rq.s"
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "nvfp4rq.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    found = {}
    for block in re.findall(r"- \.agpr_count:.*?\.wavefront_size:\s*\d+", text, re.S):
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        found[name] = {key: int(re.search(rf"\.{key}:\s+(\d+)", block).group(1))
                       for key in ("vgpr_count", "vgpr_spill_count", "sgpr_spill_count",
                                   "private_segment_fixed_size")}
    assert found, "no kernel metadata in the assembly"
    return found


def test_no_kernel_spills(kernels):
    for name, r in kernels.items():
        assert r["vgpr_spill_count"] == 0, (name, r)
        assert r["private_segment_fixed_size"] == 0, (name, r)
        assert r["sgpr_spill_count"] <= 8, (name, r)


def test_quantize_pass_fits_eight_waves(kernels):
    quant = {n: r for n, r in kernels.items() if "rotquant_kernel" in n}
    # bf16/fp32 x rotate on/off x (row-major: head, word, given scale;
    # swizzled: head, word, each with 256- and 1024-thread workgroups)
    assert len(quant) == 28
    for name, r in quant.items():
        assert r["vgpr_count"] <= 64, (name, r)
