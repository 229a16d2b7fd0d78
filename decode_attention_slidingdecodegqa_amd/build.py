"""Compile the gfx950 HIP library (libgqadecode.so) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "gqa_decode.hip"), os.path.join(CSRC, "gqa_prefill.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libgqadecode.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", f"-I{INCLUDE}",
        # no packed fp32 VALU instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-result", "-Wno-unused-value",
    ]


# per-source extra flags: the kernels keep their MFMA accumulators in VGPRs
# (in AGPRs the compiler copies them to VGPRs and back at every key tile, for
# the rarely taken online-softmax rescale branch)
SOURCE_FLAGS = {
    "gqa_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gqa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd: list[str], verbose: bool) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(x for x in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in x)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Always recompiles (one object per source); returns the library path."""
    tmp = LIBRARY + ".tmp"
    common = [f for f in flags() if f != "-shared"]
    objs = []
    for src in SOURCES:
        obj = os.path.join(PKG, "_build", os.path.basename(src) + ".o")
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        _run([hipcc(), *common, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", src,
              "-o", obj], verbose)
        objs.append(obj)
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
