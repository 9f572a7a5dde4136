"""Build tests/c/abi_client: a plain C program (gcc) that uses libvwc through
include/vwc.h and the HIP runtime only, linked with the oracle for its checks."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "abi_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    pkg = os.path.join(ROOT, "vocab_wide_cross_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", orc, "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "abi_client.c"), "-o", BIN + ".tmp",
           "-L", pkg, "-lvwc", "-L", orc, "-loracle", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../vocab_wide_cross_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())
