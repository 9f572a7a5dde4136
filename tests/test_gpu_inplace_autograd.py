"""The in-place backward (the gradient written over the logits it is computed
from) and the autograd wrapper.

In place, every backward call must give the bits of the same call with a
separate gradient buffer; the autograd wrapper must give the bits of the
library calls it stands for, and the fp64 oracle's gradient (one bf16 step,
fp32 within 1e-6).  Shapes span several 64 KiB backward segments and a ragged
tail; row sets include duplicates, whose gradients add.
"""
import numpy as np
import pytest
import torch

import oracle
import vocab_wide_cross_amd as vwc
import workloads as W
from gpu_util import DEV, assert_bf16_grad, grad_bits, log, to_dev_logits

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _case(dtype, n, vocab):
    name = "spiked_bf16_8192x248320" if dtype == "bf16" else "tiny_fp32_64x2048"
    w = W.scaled(name, n, vocab)
    return w, W.all_logits(w), W.targets(w), W.grad_out(w)


def _same(a, b):
    return torch.equal(a.contiguous().view(torch.int16 if a.dtype == torch.bfloat16
                                           else torch.int32),
                       b.contiguous().view(torch.int16 if b.dtype == torch.bfloat16
                                           else torch.int32))


@pytest.mark.parametrize("dtype,vocab", [("bf16", 151939), ("fp32", 70001), ("bf16", 4000)])
def test_inplace_dense_backward_bitwise(dtype, vocab):
    w, x, t, g = _case(dtype, 24, vocab)
    log(f"in-place dense backward {dtype} [{w.n_rows}, {vocab}]")
    xd, td, gd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    ref = vwc.selected_logprob_bwd(xd, td, lse, gd)
    y = xd.clone()
    out = vwc.selected_logprob_bwd(y, td, lse, gd, grad_logits=y)
    assert out.data_ptr() == y.data_ptr() and _same(y, ref)
    # the fused logprob + entropy backward
    h = torch.from_numpy(np.random.default_rng(3).uniform(-1, 1, w.n_rows).astype(np.float32)).to(DEV)
    ref2 = vwc.logprob_entropy_bwd(xd, td, lse, ent, gd, h)
    y2 = xd.clone()
    vwc.logprob_entropy_bwd(y2, td, lse, ent, gd, h, grad_logits=y2)
    assert _same(y2, ref2)


def test_inplace_scatter_rows_bitwise():
    w, x, t, g = _case("bf16", 40, 151936)
    rows = np.array([39, 0, 7, 22, 8], np.int32)  # distinct ids
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    rd = torch.from_numpy(rows).to(DEV)
    gc = torch.from_numpy(g[rows]).to(DEV)
    lp, lse, _ = vwc.selected_logprob_fwd_rows(xd, td, rd)
    ref = torch.zeros_like(xd)
    vwc.selected_logprob_bwd_rows(xd, td, rd, lse, gc, grad_logits=ref,
                                  layout=vwc.VWC_GRAD_SCATTER)
    y = xd.clone()
    vwc.selected_logprob_bwd_rows(y, td, rd, lse, gc, grad_logits=y, layout=vwc.VWC_GRAD_SCATTER)
    assert _same(y[rd.long()], ref[rd.long()])
    others = np.setdiff1d(np.arange(w.n_rows), rows)
    assert _same(y[others], xd[others])  # rows outside the set keep their logits
    with pytest.raises(vwc.VwcError):  # compact gradient rows cannot alias the logits
        vwc.selected_logprob_bwd_rows(y, td, rd, lse, gc, grad_logits=y,
                                      layout=vwc.VWC_GRAD_COMPACT)


@pytest.mark.parametrize("mode", [vwc.VWC_KL_TRUNCATED, vwc.VWC_KL_TAIL])
def test_inplace_topk_kl_backward_bitwise(mode):
    w = W.scaled("distill_bf16_4096x248320_k128", 12, 151936)
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    g = np.random.default_rng(6).uniform(-1, 1, w.n_rows).astype(np.float32)
    xd = to_dev_logits(x)
    idd, tld, gd = (torch.from_numpy(a).to(DEV) for a in (idx, tlp, g))
    fwd = vwc.topk_kl_fwd(xd, idd, tld, mode)
    ref = vwc.topk_kl_bwd(xd, idd, tld, fwd, gd, mode)
    y = xd.clone()
    vwc.topk_kl_bwd(y, idd, tld, fwd, gd, mode, grad_logits=y)
    assert _same(y, ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("with_entropy", [False, True])
def test_autograd_dense(dtype, with_entropy):
    w, x, t, g = _case(dtype, 16, 70001)
    log(f"autograd dense {dtype} entropy={with_entropy}")
    xd, td, gd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    h = np.random.default_rng(4).uniform(-1, 1, w.n_rows).astype(np.float32)
    hd = torch.from_numpy(h).to(DEV)
    leaf = xd.clone().requires_grad_(True)
    if with_entropy:
        lp, ent = vwc.selected_logprob(leaf, td, 0.7, with_entropy=True)
        (lp * gd + ent * hd).sum().backward()
    else:
        lp = vwc.selected_logprob(leaf, td, 0.7)
        (lp * gd).sum().backward()
    # the library calls it stands for
    lp0, lse0, ent0 = vwc.selected_logprob_fwd(xd, td, 0.7, want=("logprob", "lse", "entropy"))
    assert _same(lp.detach(), lp0)
    if with_entropy:
        # the fused call's own parity (with its allowance where the entropy
        # factor cancels) is covered by the entropy-gradient tests
        ref = vwc.logprob_entropy_bwd(xd, td, lse0, ent0, gd, hd, 0.7)
    else:
        ref = vwc.selected_logprob_bwd(xd, td, lse0, gd, 0.7)
    assert leaf.grad.dtype == xd.dtype and _same(leaf.grad, ref)
    if not with_entropy:
        oref = oracle.backward(x, t, g, tau=0.7)
        if dtype == "bf16":
            assert_bf16_grad(grad_bits(leaf.grad), oref, "autograd grad", oracle)
        else:
            assert np.abs(_np(leaf.grad).astype(np.float64) - oref).max() <= 1e-6


def test_autograd_rows_with_duplicates_and_inplace():
    w, x, t, g = _case("bf16", 20, 151939)
    rows = np.array([3, 17, 3, 0, 19], np.int32)  # row 3 twice
    gc = np.random.default_rng(5).uniform(-1, 1, rows.size).astype(np.float32)
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    rd, gcd = torch.from_numpy(rows).to(DEV), torch.from_numpy(gc).to(DEV)
    leaf = xd.clone().requires_grad_(True)
    lp = vwc.selected_logprob(leaf, td, row_idx=rd)
    (lp * gcd).sum().backward()
    ref_lp = oracle.forward(x, t, rows=rows)["logprob"]
    assert np.abs(_np(lp).astype(np.float64) - ref_lp).max() <= 5e-5
    # oracle: the gradient of each listed row, duplicates summed, zero elsewhere
    gsum = np.zeros(w.n_rows, np.float32)
    np.add.at(gsum, rows, gc)
    oref = oracle.backward(x, t, gsum)
    assert_bf16_grad(grad_bits(leaf.grad), oref, "autograd rows grad", oracle)
    unlisted = np.setdiff1d(np.arange(w.n_rows), rows)
    assert np.all(grad_bits(leaf.grad)[unlisted] == 0)
    # in place: the same bits, written over the logits themselves.  The logits
    # here come out of an op (as from an LM head), so their gradient flows on
    # to that op's backward rather than into a leaf's .grad.
    base = xd.clone().requires_grad_(True)
    logits = base * 1.0
    lp2 = vwc.selected_logprob(logits, td, row_idx=rd, inplace_backward=True)
    (lp2 * gcd).sum().backward()
    assert _same(logits.detach(), leaf.grad)  # the logits' storage now holds the gradient
    assert _same(base.grad, leaf.grad)


@pytest.mark.parametrize("dtype,vocab", [("bf16", 151939), ("fp32", 20011), ("bf16", 253953)])
def test_weighted_nll_one_call(dtype, vocab):
    """weighted_nll: the loss -sum w lp and its gradient from the one-call kernel in
    the forward (the two calls for a row too wide to hold), scaled in the backward;
    against the oracle, the direct one call's bits, and in place."""
    w, x, t, wt = _case(dtype, 24, vocab)
    xd, td, wd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(wt).to(DEV)
    leaf = xd.clone().requires_grad_(True)
    loss, lp = vwc.weighted_nll(leaf, td, wd)
    assert not lp.requires_grad
    loss.backward()
    ref = oracle.forward(x, t)
    want = -float((wt.astype(np.float64) * ref["logprob"]).sum())
    assert abs(float(loss.detach()) - want) <= 24 * 5e-5
    assert np.abs(_np(lp).astype(np.float64) - ref["logprob"]).max() <= 5e-5
    gref = oracle.backward(x, t, -wt)
    if dtype == "bf16":
        assert_bf16_grad(grad_bits(leaf.grad), gref, "weighted_nll grad", oracle)
    else:
        assert np.abs(_np(leaf.grad).astype(np.float64) - gref).max() <= 1e-6
    _, _, _, direct = vwc.selected_logprob_fwd_bwd(xd, td, -wd)
    assert _same(leaf.grad, direct)
    assert np.all(grad_bits(leaf.grad)[wt == 0] == 0)
    # a scaled loss: the gradient times the scale, as torch multiplies it
    leaf2 = xd.clone().requires_grad_(True)
    loss2, _ = vwc.weighted_nll(leaf2, td, wd)
    (2.5 * loss2).backward()
    assert _same(leaf2.grad, direct * torch.tensor(2.5, dtype=direct.dtype, device=DEV))
    # in place: the gradient is written over the logits in the forward
    base = xd.clone().requires_grad_(True)
    logits = base * 1.0
    loss3, _ = vwc.weighted_nll(logits, td, wd, inplace=True)
    assert torch.equal(loss3, loss)
    assert _same(logits.detach(), direct)
    loss3.backward()
    assert _same(base.grad, direct)
