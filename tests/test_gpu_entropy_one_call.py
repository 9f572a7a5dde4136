"""GPU parity of the one-call forward + logprob/entropy backward
(vwc_logprob_entropy_fwd_bwd[_rows]).

The outputs against the fp64 oracle (abs 5e-5); the gradient equal, bit for bit,
to what the separate backward (vwc_logprob_entropy_bwd) writes from the call's own
lse and entropy, and within the entropy-gradient bar of the oracle (one bf16 step,
or fp32 1e-6, plus the first-order allowance where z - lse + H cancels).  Rows on
chip and rows too wide for it (the two calls), both temperatures, rows without
either weight, without the logprob weight (no targets), in place, and row sets.
"""
import numpy as np
import pytest
import torch

import oracle
import vocab_wide_cross_amd as vwc
import workloads as W
from gpu_util import DEV, grad_bits, log, to_dev_logits
from test_gpu_entropy_grad import _h, check_entropy_grad

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy()


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


CASES = [("bf16", 248320, 1.0), ("bf16", 151939, 0.7), ("bf16", 253953, 1.0),
         ("fp32", 70001, 0.7), ("fp32", 130001, 1.0)]


@pytest.mark.parametrize("dtype,vocab,tau", CASES, ids=[f"{a}-V{b}-tau{c}" for a, b, c in CASES])
def test_entropy_one_call_against_oracle_and_separate_calls(dtype, vocab, tau):
    base = "spiked_bf16_8192x248320" if dtype == "bf16" else "tiny_fp32_64x2048"
    w = W.scaled(base, 20, vocab)
    x, t, g = W.all_logits(w), W.targets(w), W.grad_out(w)
    h = _h(w.n_rows, 9)
    g[3] = 0.0
    h[3] = 0.0  # neither weight: +0.0
    g[4] = 0.0  # entropy only
    h[5] = 0.0  # logprob only
    log(f"entropy one call {dtype} V={vocab} tau={tau}")
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    gd, hd = torch.from_numpy(g).to(DEV), torch.from_numpy(h).to(DEV)
    lp, lse, ent, grad = vwc.logprob_entropy_fwd_bwd(xd, td, gd, hd, tau)
    ref = oracle.forward(x, t, tau=tau)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert np.abs(_np(v).astype(np.float64) - ref[k]).max() <= 5e-5, k
    sep = vwc.logprob_entropy_bwd(xd, td, lse, ent, gd, hd, tau)
    assert torch.equal(_bits(grad), _bits(sep))
    if dtype == "bf16":
        check_entropy_grad(x, t, g, h, tau, grad_bits(grad), _np(lse), _np(ent),
                           what=f"one call V={vocab}")
    else:
        gref = oracle.backward_entropy(x, t, g, h, tau=tau)
        assert np.abs(_np(grad).astype(np.float64) - gref).max() <= 1e-6
    assert torch.all(_bits(grad)[3] == 0)
    # in place: the same bits over the logits
    xin = to_dev_logits(x)
    lp2, lse2, ent2, gin = vwc.logprob_entropy_fwd_bwd(xin, td, gd, hd, tau, grad_logits=xin)
    assert gin.data_ptr() == xin.data_ptr()
    assert torch.equal(lse2, lse) and torch.equal(ent2, ent) and torch.equal(lp2, lp)
    assert torch.equal(_bits(gin), _bits(grad))


def test_entropy_one_call_without_logprob_weight():
    """grad_logprob absent (g = 0) and no targets: the entropy's gradient alone, as the
    separate backward writes it; no logprob output."""
    w = W.scaled("spiked_bf16_8192x248320", 12, 151936)
    x = W.all_logits(w)
    h = _h(w.n_rows, 10)
    xd, hd = to_dev_logits(x), torch.from_numpy(h).to(DEV)
    lp, lse, ent, grad = vwc.logprob_entropy_fwd_bwd(xd, None, None, hd, want=("lse", "entropy"))
    assert lp is None
    sep = vwc.logprob_entropy_bwd(xd, None, lse, ent, None, hd)
    assert torch.equal(_bits(grad), _bits(sep))
    # (the oracle's forward wants targets for its logprob; they do not enter here)
    check_entropy_grad(x, np.zeros(w.n_rows, np.int32), None, h, 1.0, grad_bits(grad),
                       _np(lse), _np(ent), what="entropy only")


def test_entropy_one_call_rows_equal_dense_rows():
    """The row-set call gives each listed row the dense call's bits, compact and
    scatter; a bad row id gives NaN outputs and no gradient row."""
    w = W.scaled("spiked_bf16_8192x248320", 16, 151936)
    x, t, g = W.all_logits(w), W.targets(w), W.grad_out(w)
    h = _h(w.n_rows, 11)
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    gd, hd = torch.from_numpy(g).to(DEV), torch.from_numpy(h).to(DEV)
    dense = vwc.logprob_entropy_fwd_bwd(xd, td, gd, hd)
    rows = np.array([15, 0, 5, 9, 3], np.int32)
    rd, rl = torch.from_numpy(rows).to(DEV), torch.from_numpy(rows).to(DEV).long()
    sub = vwc.logprob_entropy_fwd_bwd_rows(xd, td, rd, gd[rl].contiguous(), hd[rl].contiguous())
    for a, b in zip(sub[:3], dense[:3]):
        assert torch.equal(a, b[rl])
    assert torch.equal(_bits(sub[3]), _bits(dense[3][rl]))
    scat = torch.full_like(xd, 7.0)
    vwc.logprob_entropy_fwd_bwd_rows(xd, td, rd, gd[rl].contiguous(), hd[rl].contiguous(),
                                     grad_logits=scat, layout=vwc.VWC_GRAD_SCATTER)
    assert torch.equal(_bits(scat[rl]), _bits(dense[3][rl]))
    others = torch.from_numpy(np.setdiff1d(np.arange(w.n_rows), rows)).to(DEV)
    assert torch.all(scat[others].float() == 7.0)
    bad = torch.tensor([2, -1], dtype=torch.int32, device=DEV)
    cg = torch.full((2, w.vocab), 7.0, dtype=torch.bfloat16, device=DEV)
    b = vwc.logprob_entropy_fwd_bwd_rows(xd, td, bad, gd[:2].contiguous(), hd[:2].contiguous(),
                                         grad_logits=cg)
    assert torch.isnan(b[1][1]) and torch.isnan(b[2][1])
    assert torch.all(cg[1].float() == 7.0)
