"""Host logic of bench.py that needs no GPU: the kernel-source hash that
decides whether the committed counter summaries still describe the kernels."""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_comments_and_layout_do_not_count():
    a = "int f(int x) {\n  return x / 2;  // halve\n}\n"
    b = "/* doc */ int f(int x)\n{ return x / 2; }  // other words\n"
    assert bench.code_tokens(a) == bench.code_tokens(b) == "int f(int x) { return x / 2; }"


def test_code_changes_count():
    assert bench.code_tokens("return x / 2;") != bench.code_tokens("return x / 4;")
    assert bench.code_tokens("a = b;") != bench.code_tokens("a = -b;")


def test_literals_are_kept_whole():
    src = 'const char* s = "a // b /* c */ \\" d"; char q = \'/\';'
    assert bench.code_tokens(src) == src


def test_hash_is_stable():
    h = bench.kernel_source_sha()
    assert h == bench.kernel_source_sha() and len(h) == 16
