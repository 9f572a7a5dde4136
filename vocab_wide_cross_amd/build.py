"""Build libvwc.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libvwc.so")
SOURCES = ["vwc_kernels.hip", "vwc_lmhead.hip", "vwc_api.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags(extra=()) -> list[str]:
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        # No packed-fp32 instructions anywhere in device code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *extra,
    ]


def build(out: str = LIB_PATH, extra=(), verbose: bool = False) -> str:
    """Compile the HIP kernels and the C-ABI into one shared library."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *compile_flags(extra), "-shared", "-x", "hip",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
