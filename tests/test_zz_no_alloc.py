"""The allocation-free forward, vwc_selected_logprob_fwd_noalloc, through the C ABI.

Its segment partials live in a fixed device array the library holds per GPU
instead of a caller workspace.  On the GPU it must give the bits of
vwc_selected_logprob_fwd with a workspace, on consecutive calls of shrinking
size (the array keeps the previous call's contents), and allocate nothing.  On
the host it must refuse a call that needs more than the array before any HIP
call.
"""
import ctypes
import os

import numpy as np
import pytest
# torch first: it brings its own HIP runtime, and the library must bind to that
# one.  Loaded before torch, the library would pull in a second runtime and the
# GPU test below would run its calls on it.
import torch  # noqa: F401

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.environ.get("VWC_TEST_LIB") or os.path.join(ROOT, "vocab_wide_cross_amd", "libvwc.so")
OK, INVALID, UNSUPPORTED = 0, 1, 2
BF16, FP32 = 0, 1
SCRATCH_BYTES = 4 << 20
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


def _noalloc(lib):
    f = lib.vwc_selected_logprob_fwd_noalloc
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [p, ctypes.c_int, i64, i64, i64, p, ctypes.c_float, p, p, p, p]
    f.restype = ctypes.c_int
    return f


def test_noalloc_host_checks():
    lib = ctypes.CDLL(LIB)
    f = _noalloc(lib)
    lib.vwc_last_error.restype = ctypes.c_char_p
    # 248320 bf16 columns = 4 segments = 64 bytes of partials per row.
    rows_max = SCRATCH_BYTES // 64
    assert f(FAKE, BF16, rows_max + 1, 248320, 248320, FAKE, 1.0, FAKE, None, None,
             None) == UNSUPPORTED
    assert b"scratch" in lib.vwc_last_error()
    # fp32 rows of 248320 columns: 8 segments, 128 bytes per row.
    assert f(FAKE, FP32, SCRATCH_BYTES // 128 + 1, 248320, 248320, FAKE, 1.0, FAKE, None, None,
             None) == UNSUPPORTED
    # the usual argument checks come first
    assert f(None, BF16, 4, 16, 16, FAKE, 1.0, FAKE, None, None, None) == INVALID
    assert f(FAKE, BF16, 4, 16, 16, None, 1.0, FAKE, None, None, None) == INVALID
    assert f(FAKE, BF16, 4, 16, 16, FAKE, 0.0, FAKE, None, None, None) == INVALID
    assert f(None, BF16, 0, 16, 16, None, 1.0, None, None, None, None) == OK


@pytest.mark.gpu
def test_noalloc_matches_workspace_forward_on_consecutive_calls():
    import oracle
    import vocab_wide_cross_amd as vwc
    import workloads as W
    from gpu_util import DEV, assert_close_scalar, log, to_dev_logits

    def run(x_host, t_host, tau, what):
        xd, td = to_dev_logits(x_host), torch.from_numpy(t_host).to(DEV)
        n = x_host.shape[0]
        ref = vwc.selected_logprob_fwd(xd, td, tau, want=("logprob", "lse", "entropy"))
        outs = [torch.full((n,), 7.0, device=DEV) for _ in range(3)]
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        vwc.selected_logprob_fwd_noalloc(xd, td, tau, logprob=outs[0], lse=outs[1],
                                         entropy=outs[2])
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.cuda.max_memory_allocated() == before
        for name, a, b in zip(("logprob", "lse", "entropy"), ref, outs):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{what}: {name}"
        # a few rows against the oracle too
        rows = np.array([0, n // 2, n - 1])
        f = oracle.forward(x_host[rows], t_host[rows], tau=tau)
        for name, b in zip(("logprob", "lse", "entropy"), outs):
            assert_close_scalar(b[torch.from_numpy(rows).to(DEV)].cpu().numpy(), f[name],
                                f"{what}: {name}", ulps=4)
        log(f"noalloc {what}: bitwise equal to the workspace forward")

    # 1: bf16 rows of 248320 columns, 4 segments each: partials in the array.
    w = W.scaled("spiked_bf16_8192x248320", 1024, 248320)
    run(W.all_logits(w), W.targets(w), 1.0, "bf16 [1024, 248320]")
    # 2: fewer, wider rows (5 segments, a ragged tail) at another temperature.
    w2 = W.scaled("spiked_bf16_8192x248320", 160, 300001)
    run(W.all_logits(w2), W.targets(w2), 0.7, "bf16 [160, 300001]")
    # 3: fewer still, fp32 (8 segments).
    w3 = W.scaled("extreme_fp32_16384x248320", 48, 248320)
    run(W.all_logits(w3), W.targets(w3), 0.7, "fp32 [48, 248320]")
    # 4: rows merged inside their workgroup (3 segments): the array is not used.
    w4 = W.scaled("masked_bf16_4096x151936", 64, 151936)
    run(W.all_logits(w4), W.targets(w4), 1.0, "bf16 [64, 151936]")
