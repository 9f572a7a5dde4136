"""AddressSanitizer and UndefinedBehaviorSanitizer on the host code (CPU only).

The oracle (plain C) is rebuilt instrumented and the whole pin suite runs
against it; the library is rebuilt with its host code instrumented (device
code untouched) and the C-ABI argument checks run against it.  Any report
aborts the subprocess, so a clean exit means no out-of-bounds access, no
use of uninitialised memory the sanitizers track, and no undefined behaviour
on those paths."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/"
                            "libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run(args, env):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **env)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           *args], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=900)


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-o", str(lib),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    r = _run([os.path.join(ROOT, "tests", "test_oracle_pins.py")],
             {"ORACLE_LIB": str(lib), "LD_PRELOAD": f"{asan}:{ubsan}"})
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def test_abi_checks_under_asan_and_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if not rt:
        pytest.skip("clang AddressSanitizer runtime not installed")
    import __graft_entry__
    b = __graft_entry__._build_module()
    lib = str(tmp_path / "libvwc_san.so")
    # host code only: each sanitizer flag applies to the host pass
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan"]
    csrc = os.path.join(ROOT, "vocab_wide_cross_amd", "csrc")
    subprocess.run([b.hipcc(), *b.compile_flags(san), "-shared", "-x", "hip",
                    *[os.path.join(csrc, f) for f in b.SOURCES], "-o", lib],
                   check=True, capture_output=True)
    r = _run([os.path.join(ROOT, "tests", "test_abi_cpu.py")],
             {"VWC_TEST_LIB": lib, "LD_PRELOAD": rt})
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
