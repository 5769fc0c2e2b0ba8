"""Host sanitizer runs (CPU only).

1. The oracle, the input generators and the CPU proof helpers (sweeps,
   division checks), compiled with gcc -fsanitize=address,undefined and driven
   by tests/helpers/sanitize_oracle.c on small, ragged and empty shapes with
   buffers of their exact sizes.
2. The library's host code: nvfp4rq.hip compiled with AddressSanitizer and
   UndefinedBehaviorSanitizer on its host side only (each -fsanitize= behind
   -Xarch_host; the device code is built as usual and never runs here),
   linked with tests/helpers/sanitize_abi.c, which calls every entry point
   with invalid arguments, then with valid ones on shapes up to the largest
   the checks accept.  With no GPU visible, each valid call runs its planning
   code and stops at the first launch, which the runtime rejects.

Any sanitizer report aborts the program (-fno-sanitize-recover=all), so a
non-zero exit with the report on stderr is the failure.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HELPERS = os.path.join(ROOT, "tests", "helpers")
ROCM = "/opt/rocm"

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:halt_on_error=1",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    "OMP_NUM_THREADS": "4",
}


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, **kw)


def _check_built(r):
    assert r.returncode == 0, r.stdout + r.stderr


def test_oracle_and_generators_under_asan_ubsan(tmp_path):
    exe = tmp_path / "san_oracle"
    srcs = [os.path.join(HELPERS, "sanitize_oracle.c"), os.path.join(ROOT, "oracle", "nvfp4_oracle.c"),
            os.path.join(ROOT, "synth", "synth.c"), os.path.join(HELPERS, "sweeps.c"),
            os.path.join(HELPERS, "fastdiv.c")]
    _check_built(_run(["gcc", "-std=c11", "-g", "-O1", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                       "-Wall", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                       "-fno-omit-frame-pointer", *srcs, "-o", str(exe), "-lm"]))
    r = _run([str(exe)], env={**os.environ, **SAN_ENV}, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "clean" in r.stdout


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="hipcc not installed")
def test_c_abi_host_code_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    inc = os.path.join(ROOT, "include")
    lib_o, drv_o, exe = tmp_path / "nvfp4rq_san.o", tmp_path / "sanitize_abi.o", tmp_path / "san_abi"
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _check_built(_run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                       "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                       "-Wall", "-Wno-unused-function", *host_san, "-I", inc, "-c",
                       os.path.join(ROOT, "nvfp4_activation_amd", "csrc", "nvfp4rq.hip"), "-o", str(lib_o)]))
    # the driver and the link: host code only, no .hip file on these lines
    _check_built(_run([clang, "-std=c11", "-O1", "-g", "-Wall", "-fsanitize=address,undefined",
                       "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{inc}",
                       "-c", os.path.join(HELPERS, "sanitize_abi.c"), "-o", str(drv_o)]))
    _check_built(_run([clang + "++", "-fsanitize=address,undefined", str(drv_o), str(lib_o),
                       f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]))
    # no device may be visible to it: fake device addresses are passed
    env = {**os.environ, **SAN_ENV, "HIP_VISIBLE_DEVICES": "-1"}
    r = _run([str(exe)], env=env, timeout=300)
    if r.returncode == 3:
        pytest.skip("a GPU is visible; the driver only runs without one")
    assert r.returncode == 0, r.stdout + r.stderr
    assert "clean" in r.stdout
