"""The differentiable top-k KL (vocab_wide_cross_amd.topk_kl): one library call in
the forward and one in the backward.  Loss and gradient against the fp64 oracle,
the gradient equal bit for bit to the direct backward call, in place or not, and
a row subset's gradient scattered into a zeroed tensor."""
import numpy as np
import pytest
import torch

import oracle
import vocab_wide_cross_amd as vwc
import workloads as W
from gpu_util import DEV, to_dev_logits
from test_gpu_topk_kl import MODES, check_fwd

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_topk_kl_autograd_fp32(mode, tau):
    w = W.get("distill_fp32_192x2048_k32")
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    wt = np.random.default_rng(3).uniform(-1, 1, w.n_rows).astype(np.float32)
    xd = to_dev_logits(x).requires_grad_(True)
    idd, tld = torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV)
    loss = vwc.topk_kl(xd, idd, tld, mode, temperature=tau)
    ref = oracle.topk_kl_forward(x, idx, tlp, mode, tau=tau)
    np.testing.assert_allclose(loss.detach().cpu().numpy(), ref["loss"], rtol=0, atol=5e-5)
    (loss * torch.from_numpy(wt).to(DEV)).sum().backward()
    gref = oracle.topk_kl_backward(x, idx, tlp, mode, wt, tau=tau)
    assert np.abs(xd.grad.cpu().numpy().astype(np.float64) - gref).max() <= 1e-6
    with torch.no_grad():
        fwd = vwc.topk_kl_fwd(xd, idd, tld, mode, temperature=tau)
        direct = vwc.topk_kl_bwd(xd, idd, tld, fwd, torch.from_numpy(wt).to(DEV), mode,
                                 temperature=tau)
    assert torch.equal(_bits(xd.grad), _bits(direct))


def test_topk_kl_autograd_bf16_inplace_and_rows():
    w = W.scaled("distill_bf16_4096x248320_k128", 12, 151936)
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    wt = np.random.default_rng(5).uniform(-1, 1, w.n_rows).astype(np.float32)
    wd = torch.from_numpy(wt).to(DEV)
    idd, tld = torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV)
    mode = vwc.VWC_KL_TAIL
    # separate gradient buffer
    xa = to_dev_logits(x).requires_grad_(True)
    la = vwc.topk_kl(xa, idd, tld, mode)
    (la * wd).sum().backward()
    check_fwd({"loss": la.detach(), **{k: v for k, v in vwc.topk_kl_fwd(
        xa.detach(), idd, tld, mode).items() if k != "loss"}}, x, idx, tlp, mode, 1.0)
    # in place: the same bits, written over the logits themselves.  The logits come
    # out of an op (as from an LM head), so their gradient flows on to that op's
    # backward.
    base = to_dev_logits(x).requires_grad_(True)
    logits = base * 1.0
    lb = vwc.topk_kl(logits, idd, tld, mode, inplace_backward=True)
    assert torch.equal(lb.detach(), la.detach())
    (lb * wd).sum().backward()
    assert torch.equal(_bits(logits.detach()), _bits(xa.grad))  # the storage holds it
    assert torch.equal(_bits(base.grad), _bits(xa.grad))
    # a row subset: the listed rows' loss and gradient as the dense call's, zero elsewhere
    rows = np.array([11, 0, 4, 7], np.int32)
    rl = torch.from_numpy(rows).to(DEV).long()
    xc = to_dev_logits(x).requires_grad_(True)
    lc = vwc.topk_kl(xc, idd[rl].contiguous(), tld[rl].contiguous(), mode,
                     row_idx=torch.from_numpy(rows).to(DEV))
    assert torch.equal(lc.detach(), la.detach()[rl])
    (lc * wd[rl]).sum().backward()
    assert torch.equal(_bits(xc.grad[rl]), _bits(xa.grad[rl]))
    others = torch.from_numpy(np.setdiff1d(np.arange(w.n_rows), rows)).to(DEV)
    assert torch.all(xc.grad[others] == 0)
    with pytest.raises(ValueError):
        vwc.topk_kl(xc, idd[rl].contiguous(), tld[rl].contiguous(), mode,
                    row_idx=torch.from_numpy(rows).to(DEV), inplace_backward=True)


@pytest.mark.parametrize("mode", MODES)
def test_weighted_topk_kl_one_call(mode):
    """weighted_topk_kl: sum w KL and its gradient from the one-call top-k KL in the
    forward, scaled in the backward; equal to topk_kl's loss and gradient computed by
    the one call directly, and in place."""
    w = W.scaled("distill_bf16_4096x248320_k128", 12, 151936)
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    wt = np.random.default_rng(6).uniform(-1, 1, w.n_rows).astype(np.float32)
    wt[3] = 0.0
    wd = torch.from_numpy(wt).to(DEV)
    idd, tld = torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV)
    xd = to_dev_logits(x)
    out, direct = vwc.topk_kl_fwd_bwd(xd, idd, tld, wd, mode)
    leaf = xd.clone().requires_grad_(True)
    loss, rows = vwc.weighted_topk_kl(leaf, idd, tld, wd, mode)
    assert not rows.requires_grad and torch.equal(rows, out["loss"])
    assert torch.equal(loss.detach(), (wd * out["loss"]).sum())
    (3.0 * loss).backward()
    assert torch.equal(_bits(leaf.grad), _bits(direct * torch.tensor(3.0, dtype=direct.dtype,
                                                                     device=DEV)))
    ref = oracle.topk_kl_backward(x, idx, tlp, mode, wt)
    from test_gpu_topk_kl import check_bf16_grad, grad_bound
    from gpu_util import grad_bits
    ref_fwd = check_fwd(out, x, idx, tlp, mode, 1.0)
    check_bf16_grad(grad_bits(direct), ref, grad_bound(x, idx, tlp, mode, 1.0, out, ref_fwd, wt))
    base = xd.clone().requires_grad_(True)
    logits = base * 1.0
    loss2, _ = vwc.weighted_topk_kl(logits, idd, tld, wd, mode, inplace=True)
    assert torch.equal(loss2, loss.detach())
    loss2.backward()
    assert torch.equal(_bits(logits.detach()), _bits(direct))
    assert torch.equal(_bits(base.grad), _bits(direct))
