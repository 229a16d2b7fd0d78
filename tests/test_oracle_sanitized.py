"""The fp64 C oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

Host code only: ``tests/oracle_asan_driver.c`` calls every oracle entry point
(decode contiguous/paged/windowed with a row subset, keys-from-values, the
ring cache, varlen prefill with an empty chunk, the append rows, and the
argument checks) on exact-size heap buffers.  A read or write outside a
buffer, or undefined arithmetic, ends the run with a sanitizer report.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "gqa_oracle.c")
DRIVER_C = os.path.join(ROOT, "tests", "oracle_asan_driver.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    build = subprocess.run(
        ["gcc", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-g", "-O1", "-pthread", ORACLE_C, DRIVER_C, "-lm", "-o", exe],
        capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    # the sanitizer runtime need not come first among preloaded libraries
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stderr[-4000:]
    assert "all calls clean" in run.stdout
