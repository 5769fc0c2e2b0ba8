"""CPU check of the quantize pass's head protocol indexing.

In the fused call pass 1 leaves its per-workgroup maxima and the arrival
counters in the outputs (row-major: the first 4 KiB of the codes, chunks 0 and
1; swizzled: chunk 0's scale tiles and code rows), and one pass-2 workgroup
alone writes those chunks after waiting for every workgroup to have read the
maxima.  That is only safe if the chunk order visits each chunk once, gives
chunk 0 to workgroup 0 as its last visit, and the skip rule leaves every chunk
written exactly once.  tests/helpers/head_protocol.hip evaluates the
kernels' own index functions on the host for the chunk counts and grids the
library and the GPU tests use, and checks the amax pass's workgroup remap is
a bijection.
"""
from __future__ import annotations

import os
import subprocess

from conftest import ROOT, TESTS


def test_head_protocol_indexing(tmp_path):
    exe = tmp_path / "head_protocol"
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O1", "-std=c++17",
                    "-I", os.path.join(ROOT, "nvfp4_activation_amd", "csrc"),
                    os.path.join(TESTS, "helpers", "head_protocol.hip"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "head protocol indexing ok" in r.stdout
