"""vwc_selected_logprob_fwd_bwd (forward and backward in one call, the loss
weight known up front) against the fp64 oracle and against the two separate
calls.

Rows that fit on chip take the one-workgroup-per-row kernel; wider rows, a
gradient of another dtype or another 16-byte phase take the two calls.  Bars
as in the other parity tests.  The gradient must also equal, bit for bit,
what the separate backward writes from the lse this call produced (both use
the same per-element code), in place or not.
"""
import numpy as np
import pytest
import torch

import oracle
import vocab_wide_cross_amd as vwc
import workloads as W
from gpu_util import (DEV, assert_bf16_grad, assert_close_scalar, grad_bits, like_layout, log,
                      place_rows)

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _check_grad(got, ref, what):
    if got.dtype == torch.bfloat16:
        assert_bf16_grad(grad_bits(got), ref, what, oracle)
    else:
        err = np.abs(_np(got).astype(np.float64) - ref).max()
        assert err <= 1e-6, f"{what}: fp32 gradient error {err:.3g}"


CASES = [
    # dtype, vocab, ld, offset, tau, n
    ("bf16", 248320, 248320, 0, 1.0, 24),   # the default step's rows: on chip
    ("bf16", 248321, 248321, 0, 1.0, 16),   # odd stride: every row its own phase
    ("bf16", 253952, 253952, 0, 0.7, 8),    # the widest row that fits
    ("bf16", 253953, 253953, 0, 1.0, 8),    # one column wider: the two calls
    ("bf16", 151936, 151936, 3, 1.0, 24),   # base 6 bytes in
    ("bf16", 32000, 32000, 0, 0.7, 40),
    ("bf16", 5, 5, 1, 1.0, 40),             # shorter than a vector
    ("fp32", 70001, 70004, 1, 0.7, 24),
    ("fp32", 126976, 126976, 0, 1.0, 8),    # the widest fp32 row that fits
    ("fp32", 248320, 248320, 0, 1.0, 8),    # the two calls
]


@pytest.mark.parametrize("dtype,vocab,ld,off,tau,n", CASES)
def test_fused_against_oracle_and_separate_calls(dtype, vocab, ld, off, tau, n):
    name = "spiked_bf16_8192x248320" if dtype == "bf16" else "tiny_fp32_64x2048"
    w = W.scaled(name, n, vocab, tau=tau)
    x = W.logits_rows(w, np.arange(n), ld=ld)
    t, g = W.targets(w), W.grad_out(w)
    _, xv = place_rows(x, off)
    xd = xv[:, :vocab]
    td, gd = torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    log(f"{dtype} V={vocab} ld={ld} offset={off} tau={tau}: fused call")
    gbuf = like_layout(xv)[:, :vocab]
    lp, lse, ent, grad = vwc.selected_logprob_fwd_bwd(
        xd, td, gd, w.tau, want=("logprob", "lse", "entropy"), grad_logits=gbuf)
    ref = oracle.forward(x, t, tau=w.tau, vocab=vocab)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], k)
    gref = oracle.backward(x, t, g, tau=w.tau, vocab=vocab)
    _check_grad(grad, gref, "fused gradient")
    # the separate backward from the same lse writes the same bits
    gsep = vwc.selected_logprob_bwd(xd, td, lse, gd, w.tau, grad_logits=like_layout(xv)[:, :vocab])
    assert torch.equal(_bits(grad), _bits(gsep))
    # and the separate forward agrees with this lse to the same bound
    slp, slse, sent = vwc.selected_logprob_fwd(xd, td, w.tau, want=("logprob", "lse", "entropy"))
    for a, b in ((lp, slp), (lse, slse), (ent, sent)):
        assert np.abs(_np(a).astype(np.float64) - _np(b)).max() <= 1e-4
    # in place: the gradient replaces the logits, same bits
    _, xv2 = place_rows(x, off)
    xin = xv2[:, :vocab]
    lp2, lse2, _, gin = vwc.selected_logprob_fwd_bwd(xin, td, gd, w.tau, grad_logits=xin)
    assert gin.data_ptr() == xin.data_ptr()
    assert torch.equal(_bits(lse2), _bits(lse)) and torch.equal(_bits(lp2), _bits(lp))
    assert torch.equal(_bits(gin), _bits(grad))


def test_fused_other_gradient_dtype_and_default_buffer():
    """A gradient of another dtype takes the two calls; a fresh contiguous buffer
    (the binding's default) keeps the rows' phase and the on-chip path."""
    w = W.scaled("spiked_bf16_8192x248320", 16, 50257)
    x, t, g = W.all_logits(w), W.targets(w), W.grad_out(w)
    xd = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    td, gd = torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    gref = oracle.backward(x, t, g)
    lp, lse, _, g32 = vwc.selected_logprob_fwd_bwd(xd, td, gd, grad_dtype=torch.float32)
    assert g32.dtype == torch.float32
    # lse is an fp32 input of the backward, so p carries its rounding: 1e-6 absolute holds
    assert np.abs(_np(g32).astype(np.float64) - gref).max() <= 1e-6
    _, _, _, gb = vwc.selected_logprob_fwd_bwd(xd, td, gd)
    assert_bf16_grad(grad_bits(gb), gref, "default buffer", oracle)
    assert_close_scalar(_np(lp), oracle.forward(x, t)["logprob"], "logprob")


def test_fused_full_size_every_row():
    """The default step's full shape, in the launch the bench times: every row's
    outputs and every live row's gradient against the oracle, and every row
    against the separate calls."""
    w = W.get("spiked_bf16_8192x248320")
    from gpu_util import check_grad_rows, upload_workload
    xd, x = upload_workload(w, keep_rows=True)
    t, g = W.targets(w), W.grad_out(w)
    td, gd = torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    lp, lse, ent, grad = vwc.selected_logprob_fwd_bwd(xd, td, gd,
                                                      want=("logprob", "lse", "entropy"))
    torch.cuda.synchronize()
    gsep = vwc.selected_logprob_bwd(xd, td, lse, gd)
    assert torch.equal(_bits(grad), _bits(gsep))
    del gsep
    slp, slse, _ = vwc.selected_logprob_fwd(xd, td)
    assert np.abs(_np(slse).astype(np.float64) - _np(lse)).max() <= 1e-4
    assert np.abs(_np(slp).astype(np.float64) - _np(lp)).max() <= 1e-4
    ref = oracle.forward(x, t)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        e = assert_close_scalar(_np(v), ref[k], k)
        log(f"one call {k}: max err {e:.3g} over all {w.n_rows} rows")
    zero = np.flatnonzero(g == 0)
    assert torch.all(grad[torch.from_numpy(zero).to(DEV)].view(torch.int16) == 0)
    live = np.flatnonzero(g != 0)
    steps = check_grad_rows(grad, live, x[live], t[live], g[live], "one-call grad", oracle)
    log(f"one call grad: all {live.size} live rows within {steps} bf16 step(s)")


def test_fused_special_values():
    """-inf logits (masked entries, whole leading stretches of them), a NaN
    logit, an out-of-range target: the one call agrees with the two calls."""
    w = W.scaled("tiny_fp32_64x2048", 16, 3001)
    x, t, g = W.all_logits(w), W.targets(w), W.grad_out(w)
    rng = np.random.default_rng(5)
    mask = rng.random(x.shape) < 0.3
    mask[:, :300] = True
    mask[np.arange(16), t] = False
    x = x.copy()
    x[mask] = -np.inf
    x[7, 2000] = np.nan
    t = t.copy()
    t[9] = 3001  # outside the row: NaN logprob, as in the forward
    xd = torch.from_numpy(x).to(DEV)
    td, gd = torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    lp, lse, ent, grad = vwc.selected_logprob_fwd_bwd(xd, td, gd,
                                                      want=("logprob", "lse", "entropy"))
    slp, slse, sent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    for a, b in ((lp, slp), (lse, slse), (ent, sent)):
        a, b = _np(a).astype(np.float64), _np(b).astype(np.float64)
        assert np.array_equal(np.isnan(a), np.isnan(b))
        ok = ~np.isnan(a)
        assert np.abs(a[ok] - b[ok]).max() <= 1e-4
    assert np.isnan(_np(lp)[7]) and np.isnan(_np(lp)[9]) and np.isfinite(_np(lse)[9])
    gsep = vwc.selected_logprob_bwd(xd, td, lse, gd)
    assert torch.equal(_bits(grad), _bits(gsep))
    rows = np.array([r for r in range(16) if r not in (7, 9)])
    gref = oracle.backward(x[rows], t[rows], g[rows])
    assert np.abs(_np(grad)[rows].astype(np.float64) - gref).max() <= 1e-6


@pytest.mark.parametrize("dtype,vocab,ld,off", [("bf16", 248320, 248320, 0),
                                                ("bf16", 20011, 20011, 0),
                                                ("fp32", 7001, 7004, 1)])
def test_fused_row_sets(dtype, vocab, ld, off):
    """Compact and scatter gradients over a row list (with a bad id), against the
    oracle and, bit for bit, against the separate `_rows` backward from the same lse."""
    name = "spiked_bf16_8192x248320" if dtype == "bf16" else "tiny_fp32_64x2048"
    n = 24
    w = W.scaled(name, n, vocab)
    x = W.logits_rows(w, np.arange(n), ld=ld)
    t = W.targets(w)
    _, xv = place_rows(x, off)
    xd = xv[:, :vocab]
    td = torch.from_numpy(t).to(DEV)
    rows = np.array([5, 0, 23, 11, 17, 2, 8], dtype=np.int32)
    gr = W.grad_out(W.scaled(name, rows.size, vocab))
    gr[1] = 0.0
    idx, grd = torch.from_numpy(rows).to(DEV), torch.from_numpy(gr).to(DEV)
    ref = oracle.forward(x, t, rows=rows, vocab=vocab)
    gref = oracle.backward(x, t, gr, rows=rows, vocab=vocab)
    for layout in (vwc.VWC_GRAD_SCATTER, vwc.VWC_GRAD_COMPACT):
        gbuf = like_layout(xv)[:, :vocab] if layout == vwc.VWC_GRAD_SCATTER else None
        lp, lse, ent, grad = vwc.selected_logprob_fwd_bwd_rows(
            xd, td, idx, grd, want=("logprob", "lse", "entropy"), grad_logits=gbuf,
            layout=layout)
        for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
            assert_close_scalar(_np(v), ref[k], k)
        got = grad[idx.long()] if layout == vwc.VWC_GRAD_SCATTER else grad
        _check_grad(got, gref, f"rows, layout {layout}")
        sep = vwc.selected_logprob_bwd_rows(
            xd, td, idx, lse, grd, layout=layout,
            grad_logits=like_layout(xv)[:, :vocab] if layout == vwc.VWC_GRAD_SCATTER else None)
        assert torch.equal(_bits(grad), _bits(sep))
        if layout == vwc.VWC_GRAD_SCATTER:
            others = torch.from_numpy(np.setdiff1d(np.arange(n), rows)).to(DEV).long()
            assert torch.count_nonzero(grad[others]) == 0
    # a row id outside the tensor: NaN outputs, and its gradient row stays untouched
    bad = torch.tensor([3, n + 4], dtype=torch.int32, device=DEV)
    gb = torch.full((2, vocab), 7.0, dtype=xd.dtype, device=DEV)
    lp, lse, _, gb = vwc.selected_logprob_fwd_bwd_rows(xd, td, bad, grd[:2], grad_logits=gb)
    assert np.isnan(_np(lp)[1]) and np.isnan(_np(lse)[1]) and np.isfinite(_np(lse)[0])
    assert torch.all(gb[1] == 7.0)
