"""Shared test setup: marker registration, native builds, helpers."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

import __graft_entry__  # noqa: E402

__graft_entry__.ensure_built()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU test")


GOLDEN = os.path.join(TESTS, "golden")


def read_golden(name: str) -> list[list[str]]:
    """Rows of a whitespace-separated fixture, comments and blank lines dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def sweeps_lib(tmp_path_factory):
    """The exhaustive-sweep helper, compiled against the oracle library."""
    import ctypes
    out = tmp_path_factory.mktemp("sweeps") / "libsweeps.so"
    odir = os.path.join(ROOT, "oracle")
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    os.path.join(TESTS, "helpers", "sweeps.c"), "-o", str(out),
                    f"-L{odir}", "-lnvfp4oracle", f"-Wl,-rpath,{odir}", "-lm"], check=True)
    lib = ctypes.CDLL(str(out))
    for name in ("sweep_e2m1_all", "sweep_e8m0_all"):
        getattr(lib, name).restype = ctypes.c_longlong
        getattr(lib, name).argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    lib.sweep_e4m3_range.restype = ctypes.c_longlong
    lib.sweep_e4m3_range.argtypes = [ctypes.c_uint32, ctypes.c_uint32,
                                     ctypes.POINTER(ctypes.c_uint32)]
    lib.sweep_e4m3_linear.restype = ctypes.c_longlong
    lib.sweep_e4m3_linear.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.POINTER(ctypes.c_uint32)]
    return lib
