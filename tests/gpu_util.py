"""Helpers for the GPU tests: upload seeded workloads, compare with tolerances."""
import sys
import time

import numpy as np
import torch

import workloads as W
from helpers import bf16_ulp_distance, fp32_ulp

DEV = torch.device("cuda:0")


def log(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev_logits(host: np.ndarray) -> torch.Tensor:
    if host.dtype == np.uint16:
        return torch.from_numpy(host.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(host).to(DEV)


def upload_workload(w: W.Workload, ld: int | None = None, block_rows: int = 512,
                    keep_rows=None):
    """Generate every row on the host in blocks and copy it into one device tensor.
    With keep_rows (ascending row ids, or True for all), also return a host copy
    of those rows: (device tensor, host array [len(keep_rows), ld])."""
    ld = w.vocab if ld is None else ld
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = torch.empty((w.n_rows, ld), dtype=dt, device=DEV)
    if keep_rows is True:
        keep_rows = np.arange(w.n_rows)
    host = None if keep_rows is None else np.empty((len(keep_rows), ld), dtype=w.np_dtype)
    t0 = time.time()
    last = [t0]

    def sink(r0, blk):
        t[r0:r0 + blk.shape[0]].copy_(to_dev_logits(blk))
        if host is not None:
            a, b = np.searchsorted(keep_rows, [r0, r0 + blk.shape[0]])
            host[a:b] = blk[keep_rows[a:b] - r0]
        if time.time() - last[0] > 10:
            last[0] = time.time()
            log(f"  {w.name}: {r0 + blk.shape[0]} of {w.n_rows} rows uploaded")

    W.fill_logits(w, sink, block_rows=block_rows, ld=ld)
    torch.cuda.synchronize()
    log(f"uploaded {w.name} [{w.n_rows}, {ld}] {w.dtype} in {time.time() - t0:.1f}s")
    return t if host is None else (t, host)


def check_grad_rows(grad, grad_rows, x_host, t_rows, g_rows, what, oracle, tau=1.0,
                    block=256):
    """Every listed gradient row against the oracle, in blocks of rows: bf16 within
    one step of the rounded oracle, fp32 within 1e-6.  grad_rows index `grad`;
    x_host / t_rows / g_rows hold the same rows' logits, targets and incoming
    gradients.  Returns the largest bf16 step count (or fp32 error)."""
    worst = 0.0
    t0 = time.time()
    for a in range(0, len(grad_rows), block):
        b = min(a + block, len(grad_rows))
        gi = torch.from_numpy(np.asarray(grad_rows[a:b], dtype=np.int64)).to(DEV)
        ref = oracle.backward(x_host[a:b], t_rows[a:b], g_rows[a:b], tau=tau)
        got = grad[gi]
        if got.dtype == torch.bfloat16:
            worst = max(worst, assert_bf16_grad(grad_bits(got), ref, f"{what} rows {a}-{b}",
                                                oracle))
        else:
            err = np.abs(got.cpu().numpy().astype(np.float64) - ref).max()
            assert err <= 1e-6, f"{what} rows {a}-{b}: fp32 grad err {err}"
            worst = max(worst, float(err))
        if time.time() - t0 > 10:
            t0 = time.time()
            log(f"  {what}: {b} of {len(grad_rows)} gradient rows checked")
    return worst


def grad_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_close_scalar(got, ref, what, atol=5e-5, ulps=0):
    """|got - ref| <= max(atol, ulps * ulp_fp32(ref)) elementwise (NaN must match)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN pattern differs"
    ok = ~nan_r
    tol = np.maximum(atol, ulps * fp32_ulp(ref[ok])) if ulps else atol
    err = np.abs(got[ok] - ref[ok])
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {ok.sum()} beyond tolerance, max err "
                           f"{err.max():.3g} at {np.argmax(err)}")
    return float(err.max()) if err.size else 0.0


def assert_bf16_grad(got_bits, ref_grad64, what, oracle):
    ref_bits = oracle.bf16_rne(ref_grad64)
    d = bf16_ulp_distance(got_bits, ref_bits)
    assert d.max() <= 1, f"{what}: bf16 gradient {d.max()} steps from the rounded oracle"
    return int(d.max())


def place_rows(host: np.ndarray, off: int):
    """Device copy of host rows [n, ld] inside a flat allocation, starting `off`
    elements in (so every row may start off 16 bytes); returns (flat, [n, ld] view)."""
    n, ld = host.shape
    dt = torch.bfloat16 if host.dtype == np.uint16 else torch.float32
    flat = torch.zeros(n * ld + off + 64, dtype=dt, device=DEV)
    view = flat[off:off + n * ld].view(n, ld)
    view.copy_(to_dev_logits(host))
    return flat, view


def like_layout(view: torch.Tensor, dtype=None) -> torch.Tensor:
    """A zeroed [n, ld] buffer with the view's stride and element offset."""
    n, ld = view.shape
    off = view.storage_offset()
    flat = torch.zeros(n * ld + off + 64, dtype=dtype or view.dtype, device=DEV)
    return flat[off:off + n * ld].view(n, ld)
