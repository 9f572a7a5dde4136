"""Rows that do not start on 16 bytes, against the fp64 oracle.

The kernels stream 16-byte vectors from each row's first 16-byte boundary and
take the elements before it and past the last whole vector one by one.  With
an odd row stride every row has another phase; with a view that starts a few
elements into an allocation every row has the same non-zero phase.  The
backward keeps the vector path when each row's boundary is a 16-byte boundary
of its gradient row too (same layout, same stride and row index, or in
place) and goes element by element otherwise; both are checked.  Bars as in
the other parity tests: 5e-5 on logprob / lse / entropy, one bf16 step on a
bf16 gradient, 1e-6 on an fp32 gradient.
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


def _check_grad(got, ref, what):
    if got.dtype == torch.bfloat16:
        assert_bf16_grad(grad_bits(got), ref, what, oracle)
    else:
        err = np.abs(_np(got).astype(np.float64) - ref).max()
        assert err <= 1e-6, f"{what}: fp32 gradient error {err:.3g}"


CASES = [
    # dtype, vocab, ld, offset (elements)
    ("bf16", 20011, 20011, 0),     # odd stride: each row its own phase
    ("bf16", 4099, 4101, 3),
    ("bf16", 248320, 248320, 3),   # whole-vector stride, base 6 bytes in: one phase, 4 segments
    ("bf16", 151936, 151937, 1),   # in-block merge, odd stride
    ("bf16", 5, 5, 1),             # shorter than the head
    ("fp32", 5003, 5003, 0),
    ("fp32", 70001, 70004, 1),     # whole-vector stride, base 4 bytes in
    ("fp32", 98304, 98305, 2),     # three segments merged in-block
]


@pytest.mark.parametrize("dtype,vocab,ld,off", CASES)
def test_forward_and_backward(dtype, vocab, ld, off):
    name = "spiked_bf16_8192x248320" if dtype == "bf16" else "tiny_fp32_64x2048"
    n = 24 if vocab > 100000 else 40
    w = W.scaled(name, n, vocab)
    x = W.logits_rows(w, np.arange(n), ld=ld)
    t, g = W.targets(w), W.grad_out(w)
    flat, xv = place_rows(x, off)
    xd = xv[:, :vocab]
    td, gd = torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    log(f"{dtype} V={vocab} ld={ld} offset={off}: forward")
    lp, lse, ent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    ref = oracle.forward(x, t, vocab=vocab)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], k)
    gref = oracle.backward(x, t, g, vocab=vocab)

    log("  backward, gradient in the logits' layout")
    gsame = like_layout(xv)[:, :vocab]
    vwc.selected_logprob_bwd(xd, td, lse, gd, grad_logits=gsame)
    _check_grad(gsame, gref, "same layout")
    log("  backward, gradient rows with another stride")
    gother = torch.zeros((n, ld + 1), dtype=xd.dtype, device=DEV)[:, :vocab]
    vwc.selected_logprob_bwd(xd, td, lse, gd, grad_logits=gother)
    _check_grad(gother, gref, "other stride")
    log("  backward, other gradient dtype")
    gdt = torch.float32 if dtype == "bf16" else torch.bfloat16
    gcast = like_layout(xv, gdt)[:, :vocab]
    vwc.selected_logprob_bwd(xd, td, lse, gd, grad_logits=gcast)
    # (an fp32 gradient from bf16 logits: lse is an fp32 input, so p carries its
    # rounding; 1e-6 absolute still holds)
    _check_grad(gcast, gref, f"{gdt} gradient of {dtype} logits")
    log("  backward in place, with the entropy term")
    h = W.grad_out(W.scaled(name, n, vocab + 1))
    hd = torch.from_numpy(h).to(DEV)
    gent = vwc.logprob_entropy_bwd(xd, td, lse, ent, grad_logprob=gd, grad_entropy=hd)
    flat2, xv2 = place_rows(x, off)
    xin = xv2[:, :vocab]
    gin = vwc.logprob_entropy_bwd(xin, td, lse, ent, grad_logprob=gd, grad_entropy=hd,
                                  grad_logits=xin)
    assert gin.data_ptr() == xin.data_ptr()
    assert torch.equal(gin.contiguous().view(torch.int16 if gin.dtype == torch.bfloat16
                                             else torch.int32),
                       gent.contiguous().view(torch.int16 if gent.dtype == torch.bfloat16
                                              else torch.int32))
    # the padding columns and the bytes around the rows are untouched
    assert torch.count_nonzero(flat2[:off]) == 0
    if ld > vocab:
        pad = torch.cat([xv2[:, vocab:].reshape(-1), flat2[off + n * ld:]])
        ref_pad = torch.cat([xv[:, vocab:].reshape(-1), flat[off + n * ld:]])
        assert torch.equal(pad.float(), ref_pad.float())


@pytest.mark.parametrize("dtype,vocab,ld,off", [("bf16", 20011, 20011, 0),
                                                ("bf16", 248320, 248320, 5),
                                                ("fp32", 7001, 7003, 1)])
def test_row_sets(dtype, vocab, ld, off):
    name = "spiked_bf16_8192x248320" if dtype == "bf16" else "tiny_fp32_64x2048"
    n = 32
    w = W.scaled(name, n, vocab)
    x = W.logits_rows(w, np.arange(n), ld=ld)
    t, g = W.targets(w), W.grad_out(w)
    _, xv = place_rows(x, off)
    xd = xv[:, :vocab]
    td = torch.from_numpy(t).to(DEV)
    rows = np.array([3, 0, 17, 31, 8, 9, 22], dtype=np.int32)
    idx = torch.from_numpy(rows).to(DEV)
    gr = torch.from_numpy(g[rows].copy()).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd_rows(xd, td, idx, want=("logprob", "lse", "entropy"))
    ref = oracle.forward(x, t, rows=rows, vocab=vocab)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], k)
    gref = oracle.backward(x, t, g[rows], rows=rows, vocab=vocab)
    # scatter into the logits' layout: gradient row = row id, vector path
    gs = like_layout(xv)[:, :vocab]
    vwc.selected_logprob_bwd_rows(xd, td, idx, lse, gr, grad_logits=gs,
                                  layout=vwc.VWC_GRAD_SCATTER)
    _check_grad(gs[idx.long()], gref, "scatter")
    others = np.setdiff1d(np.arange(n), rows)
    assert torch.count_nonzero(gs[torch.from_numpy(others).to(DEV).long()]) == 0
    # compact rows: gradient row = output index, element path unless the phases agree
    gc = vwc.selected_logprob_bwd_rows(xd, td, idx, lse, gr)
    _check_grad(gc, gref, "compact")


def test_split_vocabulary_at_odd_boundaries():
    """Slices that start anywhere in a row: each slice's head is its own."""
    w = W.scaled("spiked_bf16_8192x248320", 24, 30011)
    x, t = W.all_logits(w), W.targets(w)
    xd, td = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16), \
        torch.from_numpy(t).to(DEV)
    bounds = [0, 7, 1000, 1003, 17777, 30011]
    parts = torch.stack([vwc.vocab_partial(xd[:, a:b], a, targets=td)
                         for a, b in zip(bounds[:-1], bounds[1:])])
    lp, lse, ent = vwc.partial_combine(parts)
    ref = oracle.forward(x, t)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], f"split {k}")
