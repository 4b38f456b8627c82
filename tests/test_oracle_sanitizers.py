"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer and run over
edge-case shapes by a small C driver (tests/oracle_sanitize.c): no out-of-bounds access, no
use of uninitialised or freed memory, no undefined arithmetic, and the driver's own checks
(finite outputs, prefill equal to the same tokens as decode steps, refused invalid
arguments).  Built serially (no OpenMP), so that the sanitizers see one thread."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
           "-Wno-unused-parameter",  # (nthreads is unused without OpenMP)
           "-o", exe, os.path.join(ROOT, "oracle", "ssd_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize.c"),
           "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "sanitized oracle: ok" in run.stdout
