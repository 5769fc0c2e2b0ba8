"""GPU: the library driven from plain C (tests/helpers/c_consumer.c) through
the C ABI and the HIP runtime's C API alone, compared with the oracle."""
from __future__ import annotations

import os
import subprocess

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu


def test_c_program_matches_oracle(tmp_path):
    libs = {"nvfp4rq": os.path.join(ROOT, "nvfp4_activation_amd"),
            "nvfp4oracle": os.path.join(ROOT, "oracle"),
            "nvfp4synth": os.path.join(ROOT, "synth")}
    exe = tmp_path / "c_consumer"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "helpers", "c_consumer.c"),
           "-o", str(exe), "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    for name, d in libs.items():
        cmd += [f"-L{d}", f"-l{name}", f"-Wl,-rpath,{d}"]
    subprocess.run(cmd, check=True)
    for rows, cols in ((300, 4112), (4096, 8192)):
        r = subprocess.run([str(exe), str(rows), str(cols)], capture_output=True, text=True,
                           timeout=120)
        print(r.stdout.strip(), flush=True)
        assert r.returncode == 0, r.stdout + r.stderr
