"""Differentiable selected-token log-probability (and entropy) over the C-ABI.

The pages' user-facing form is an autograd function whose forward keeps the
logits, the targets and the per-row logZ, and whose backward recomputes the
softmax and writes (onehot - softmax) * grad_output into a gradient of the
logits' dtype ("fix: chunk target logprobs without tensor parallelism",
section "Changes"; "[megatron] feat: add memory-efficient chunked top-k KL
computation", section "Design & Code Changes": keep the logits and an fp32
logZ, recompute in the backward).  Here the forward and the backward are each
one call into the library; this module only moves arguments.

A row subset (the loss-mask rows, "[Bug] Training/log-prob forward
materializes full-vocab fp32 logits ...", maintainer comment) is computed in
compact form; its gradient is the full [rows, vocab] tensor with +0.0 on the
rows outside the subset (written by the library, which reads no logits for
them).  Duplicate row ids add their gradients.
"""
from __future__ import annotations

import torch

from . import _binding as B


def _dense_rows(values, row_idx, n, like):
    """Length-n vector with values[i] added at row_idx[i] (0 elsewhere)."""
    out = torch.zeros(n, dtype=torch.float32, device=like.device)
    if values is not None:
        out.index_add_(0, row_idx.long(), values.float())
    return out


def _dense_copy(values, row_idx, n, like):
    out = torch.zeros(n, dtype=torch.float32, device=like.device)
    out.index_copy_(0, row_idx.long(), values)
    return out


class _SelectedLogprob(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, targets, temperature, row_idx, with_entropy, inplace_backward):
        want = ("logprob", "lse", "entropy") if with_entropy else ("logprob", "lse")
        if row_idx is None:
            lp, lse, ent = B.selected_logprob_fwd(logits, targets, temperature, want=want)
        else:
            lp, lse, ent = B.selected_logprob_fwd_rows(logits, targets, row_idx, temperature,
                                                       want=want)
        ctx.temperature = temperature
        ctx.with_entropy = with_entropy
        ctx.inplace_backward = inplace_backward
        ctx.has_rows = row_idx is not None
        saved = [logits, targets, lse]
        if with_entropy:
            saved.append(ent)
        if row_idx is not None:
            saved.append(row_idx)
        ctx.save_for_backward(*saved)
        if with_entropy:
            return lp, ent
        return lp

    @staticmethod
    def backward(ctx, grad_lp, grad_ent=None):
        saved = list(ctx.saved_tensors)
        logits, targets, lse = saved[:3]
        ent = saved[3] if ctx.with_entropy else None
        row_idx = saved[-1] if ctx.has_rows else None
        if grad_lp is None and grad_ent is None:
            return None, None, None, None, None, None
        n = logits.size(0)
        if row_idx is not None:  # compact outputs -> every row, 0 outside the subset
            grad_lp = _dense_rows(grad_lp, row_idx, n, logits) if grad_lp is not None else None
            grad_ent = _dense_rows(grad_ent, row_idx, n, logits) if grad_ent is not None else None
            lse = _dense_copy(lse, row_idx, n, logits)
            if ent is not None:
                ent = _dense_copy(ent, row_idx, n, logits)
        out = logits if ctx.inplace_backward else None
        if ent is not None and grad_ent is not None:
            g = B.logprob_entropy_bwd(logits, targets, lse, ent, grad_lp.contiguous()
                                      if grad_lp is not None else None, grad_ent.contiguous(),
                                      ctx.temperature, grad_logits=out)
        else:
            g = B.selected_logprob_bwd(logits, targets, lse, grad_lp.contiguous(),
                                       ctx.temperature, grad_logits=out)
        return g, None, None, None, None, None


def selected_logprob(logits, targets, temperature=1.0, row_idx=None, with_entropy=False,
                     inplace_backward=False):
    """logprob[i] = log_softmax(logits[r] / temperature)[targets[r]] for r = row_idx[i]
    (every row when row_idx is None), differentiable with respect to `logits`.

    with_entropy=True also returns the entropy of each row's softmax, and the
    backward takes the gradients of both outputs in one pass.  With
    inplace_backward=True the backward writes the gradient over `logits` itself
    (no second [rows, vocab] buffer) and returns that tensor as the gradient; the
    logits are gone afterwards."""
    return _SelectedLogprob.apply(logits, targets, float(temperature), row_idx,
                                  bool(with_entropy), bool(inplace_backward))


class _TopkKL(torch.autograd.Function):
    """The chunked top-k KL of "[megatron] feat: add memory-efficient chunked top-k KL
    computation" ("Design & Code Changes"): the forward keeps the student logits, the
    teacher's top-k payload and the per-row logZ with the payload's masses and sum; the
    backward recomputes the student softmax in one library call."""

    @staticmethod
    def forward(ctx, logits, topk_idx, teacher_logprob, mode, tail_mass_eps, temperature,
                row_idx, inplace_backward):
        kw = dict(mode=mode, tail_mass_eps=tail_mass_eps, temperature=temperature)
        if row_idx is None:
            fwd = B.topk_kl_fwd(logits, topk_idx, teacher_logprob, **kw)
        else:
            fwd = B.topk_kl_fwd_rows(logits, row_idx, topk_idx, teacher_logprob, **kw)
        ctx.kw = kw
        ctx.inplace_backward = inplace_backward
        ctx.has_rows = row_idx is not None
        saved = [logits, topk_idx, teacher_logprob, fwd["lse"], fwd["student_mass"],
                 fwd["teacher_mass"], fwd["topk_sum"]]
        if row_idx is not None:
            saved.append(row_idx)
        ctx.save_for_backward(*saved)
        return fwd["loss"]

    @staticmethod
    def backward(ctx, grad_loss):
        saved = list(ctx.saved_tensors)
        logits, idx, tlp = saved[:3]
        fwd = dict(zip(("lse", "student_mass", "teacher_mass", "topk_sum"), saved[3:7]))
        g = grad_loss.contiguous().float()
        if not ctx.has_rows:
            out = logits if ctx.inplace_backward else None
            grad = B.topk_kl_bwd(logits, idx, tlp, fwd, g, grad_logits=out, **ctx.kw)
        else:  # the listed rows scattered into a zeroed [rows, vocab] gradient
            grad = torch.zeros_like(logits)
            B.topk_kl_bwd_rows(logits, saved[7], idx, tlp, fwd, g, grad_logits=grad,
                               layout=B.VWC_GRAD_SCATTER, **ctx.kw)
        return grad, None, None, None, None, None, None, None


def topk_kl(logits, topk_idx, teacher_logprob, mode=B.VWC_KL_TAIL, tail_mass_eps=1e-6,
            temperature=1.0, row_idx=None, inplace_backward=False):
    """Per-row top-k KL between a teacher's top-k payload (column ids topk_idx and
    log-probabilities teacher_logprob, [rows, k]) and the student softmax of
    logits / temperature, differentiable with respect to `logits`.

    mode: VWC_KL_TAIL (the k + 1-category KL with the tail masses) or
    VWC_KL_TRUNCATED (the top-k sum, clamped at 0).  row_idx (distinct int32 row
    ids) computes only those rows, with the payload given per listed row ([m, k]);
    their gradient is scattered into a zeroed [rows, vocab] tensor.  With
    inplace_backward=True (dense rows only) the backward writes the gradient over
    `logits` itself and returns that tensor; the logits are gone afterwards."""
    if inplace_backward and row_idx is not None:
        raise ValueError("inplace_backward needs every row (row_idx=None)")
    return _TopkKL.apply(logits, topk_idx, teacher_logprob, int(mode), float(tail_mass_eps),
                         float(temperature), row_idx, bool(inplace_backward))


class _WeightedNLL(torch.autograd.Function):
    """loss = -sum_r w_r logprob_r with the weights known before the forward (a token
    mean, say): the forward is the one-call forward + backward, which reads each row
    once and writes the gradient of the loss with respect to the logits; the backward
    only scales it by the incoming gradient (nothing when that is 1)."""

    @staticmethod
    def forward(ctx, logits, targets, weights, temperature, inplace):
        w = weights.contiguous().float()
        lp, _, _, grad = B.selected_logprob_fwd_bwd(
            logits, targets, -w, temperature, want=("logprob", "lse"),
            grad_logits=logits if inplace else None)
        if inplace:  # the library overwrote the logits: let autograd see the write
            torch.autograd.graph.increment_version(logits)
        ctx.save_for_backward(grad)
        ctx.mark_non_differentiable(lp)
        return -(w * lp).sum(), lp

    @staticmethod
    def backward(ctx, grad_loss, grad_lp=None):
        (grad,) = ctx.saved_tensors
        if grad_loss is None:
            return None, None, None, None, None
        if not (grad_loss.numel() == 1 and float(grad_loss) == 1.0):
            grad = grad * grad_loss.to(grad.dtype)
        return grad, None, None, None, None


def weighted_nll(logits, targets, weights, temperature=1.0, inplace=False):
    """The weighted negative log-likelihood -sum_r weights[r] * logprob[r] (logprob as in
    selected_logprob), differentiable with respect to `logits`, for weights known
    before the forward.  The gradient is computed in the forward by the one-call
    kernel (one read and one write of the logits instead of two reads and one write)
    and kept until the backward; with inplace=True it is written over `logits`, which
    are gone afterwards (no second [rows, vocab] tensor).  Returns (loss, logprob),
    logprob detached."""
    return _WeightedNLL.apply(logits, targets, weights, float(temperature), bool(inplace))


class _WeightedTopkKL(torch.autograd.Function):
    """loss = sum_r w_r KL_r (the top-k KL of topk_kl) with the weights known before the
    forward: the forward is the one-call top-k KL, which writes the loss's gradient
    while it holds each row; the backward only scales it."""

    @staticmethod
    def forward(ctx, logits, topk_idx, teacher_logprob, weights, mode, tail_mass_eps,
                temperature, inplace):
        w = weights.contiguous().float()
        out, grad = B.topk_kl_fwd_bwd(logits, topk_idx, teacher_logprob, w, mode=mode,
                                      tail_mass_eps=tail_mass_eps, temperature=temperature,
                                      grad_logits=logits if inplace else None)
        if inplace:  # the library overwrote the logits: let autograd see the write
            torch.autograd.graph.increment_version(logits)
        ctx.save_for_backward(grad)
        ctx.mark_non_differentiable(out["loss"])
        return (w * out["loss"]).sum(), out["loss"]

    @staticmethod
    def backward(ctx, grad_loss, grad_rows=None):
        (grad,) = ctx.saved_tensors
        if grad_loss is None:
            return None, None, None, None, None, None, None, None
        if not (grad_loss.numel() == 1 and float(grad_loss) == 1.0):
            grad = grad * grad_loss.to(grad.dtype)
        return grad, None, None, None, None, None, None, None


def weighted_topk_kl(logits, topk_idx, teacher_logprob, weights, mode=B.VWC_KL_TAIL,
                     tail_mass_eps=1e-6, temperature=1.0, inplace=False):
    """sum_r weights[r] * KL_r (KL_r as topk_kl computes it), differentiable with respect
    to `logits`, for weights known before the forward (a token mean).  The gradient is
    computed in the forward by the one-call top-k KL (one read and one write of the
    logits where the row fits on chip) and kept until the backward; with inplace=True
    it is written over `logits`, which are gone afterwards.  Returns (loss, per-row KL),
    the latter detached."""
    return _WeightedTopkKL.apply(logits, topk_idx, teacher_logprob, weights, int(mode),
                                 float(tail_mass_eps), float(temperature), bool(inplace))
