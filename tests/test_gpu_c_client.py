"""The library driven from plain C: tests/c/abi_client.c allocates with the HIP
runtime, calls the forward, backward and row-set entry points through
include/vwc.h, and checks them against the fp64 oracle (linked as a C
library) and its argument errors.  It runs as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c", "abi_client")


def test_c_client():
    if not os.path.exists(BIN):
        import __graft_entry__
        __graft_entry__._build_c_client()
    print(f"running {BIN}", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.rstrip().endswith("ok")
