"""The library's host side under AddressSanitizer and UndefinedBehaviorSanitizer.

``tests/abi_host_asan_driver.c`` exercises the launch planner and workspace
sizes over the whole shape domain and its edges (B, capacity and window from
INT_MIN to INT_MAX), the constants, the status strings and the argument checks
of the entry points.  The library's sources are built with the host code
instrumented (the kernels are compiled as usual but never launched: every
entry-point call is one its checks reject), so no GPU is needed.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_slidingdecodegqa_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="needs the ROCm toolchain")
def test_library_host_side_clean_under_sanitizers(tmp_path):
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-g"]
    objs = []
    for src in ("gqa_decode.hip", "gqa_prefill.hip"):
        obj = str(tmp_path / (src + ".o"))
        r = subprocess.run(
            [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", f"-I{ROOT}/include", f"-I{CSRC}",
             *host_san, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result", "-Wno-unused-value", "-c", os.path.join(CSRC, src), "-o", obj],
            capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", f"-I{ROOT}/include", "-c",
                        os.path.join(ROOT, "tests", "abi_host_asan_driver.c"), "-o", drv],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = str(tmp_path / "abi_host_asan")
    r = subprocess.run([CLANGXX, "--hip-link", "--offload-arch=gfx950",
                        "-fsanitize=address,undefined", *objs, drv, "-L/opt/rocm/lib",
                        "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    # the HIP runtime keeps its allocations until exit: leaks are not checked
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stderr[-4000:]
    assert "all calls clean" in run.stdout
