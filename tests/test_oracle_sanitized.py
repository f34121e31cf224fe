"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

``oracle/sanitize_driver.c`` calls every entry point of ``oracle/attn_oracle.c``
on small seeded inputs with the edge cases (no keys, no real token, one
token, row subsets, query offset, window 1, extent 1, bf16 profiles, flex
masks).  Both are built with gcc and the sanitizers, and the run must end
cleanly.  A copy with a planted out-of-bounds read shows that the sanitizer
is active in this build.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import oracle

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "attn_oracle.c")
DRIVER = os.path.join(HERE, "sanitize_driver.c")
FLAGS = ["-std=c11", "-g", "-O1", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")


def _build_and_run(src, tmp_path):
    exe = tmp_path / "oracle_san"
    subprocess.run(["gcc", *FLAGS, "-o", str(exe), DRIVER, str(src), "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    return subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)


def test_oracle_is_clean_under_sanitizers(tmp_path):
    res = _build_and_run(SRC, tmp_path)
    assert res.returncode == 0, res.stderr[-3000:]
    assert "all calls ok" in res.stdout


def test_sanitizer_catches_a_planted_out_of_bounds_read(tmp_path):
    src = open(SRC).read()
    stmt = "for (int j = 0; j < Sk; ++j) {\n            int a = allowed("
    assert stmt in src
    bad = tmp_path / "attn_oracle_oob.c"
    bad.write_text(src.replace(stmt, "for (int j = 0; j <= Sk; ++j) {\n            int a = allowed("))
    res = _build_and_run(bad, tmp_path)
    assert res.returncode != 0
    assert "AddressSanitizer" in res.stderr
