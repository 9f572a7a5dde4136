"""Device-memory footprint of each call: what the caching allocator had to hand
out beyond the inputs, read as `max_memory_allocated` growth around the call.

The method's point is that no [rows, vocab] float32 tensor (nor, on the fused
LM head, any logits tensor) is ever allocated: beyond its outputs, a call may
only use O(rows) bytes of workspace (a few 16-byte partials per row, plus the
kept hidden rows on the LM head).  Shapes are the full vocabulary width with
8192 rows, so a single stray [rows, vocab] fp32 buffer (8.1 GB) would show.
"""
import pytest
import torch

import vocab_wide_cross_amd as vwc
from gpu_util import DEV, log

pytestmark = pytest.mark.gpu

N, V = 8192, 248320
# Allocator rounding: small blocks go to 512-byte multiples, and a cached large
# block is handed out whole when splitting it would leave at most 1 MiB.
SLACK = 2 << 20
PER_ROW_CAP = 1024                    # bytes of workspace + outputs a row may cost


def _peak_growth(fn):
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    out = fn()
    torch.cuda.synchronize()
    return torch.cuda.max_memory_allocated() - base, out


@pytest.fixture(scope="module")
def inputs():
    g = torch.Generator(device=DEV).manual_seed(11)
    logits = torch.empty(N, V, dtype=torch.bfloat16, device=DEV).normal_(0.0, 3.0, generator=g)
    targets = torch.randint(0, V, (N,), dtype=torch.int32, device=DEV, generator=g)
    grad_out = torch.randn(N, dtype=torch.float32, device=DEV, generator=g)
    return logits, targets, grad_out


def _bytes(*ts):
    return sum(t.numel() * t.element_size() for t in ts if t is not None)


def test_forward_allocates_only_outputs_and_row_workspace(inputs):
    logits, targets, _ = inputs
    ws = vwc.workspace_bytes(N, V, torch.bfloat16)
    grew, outs = _peak_growth(lambda: vwc.selected_logprob_fwd(
        logits, targets, want=("logprob", "lse", "entropy")))
    log(f"fwd: grew {grew} B, outputs {_bytes(*outs)} B, workspace {ws} B")
    assert grew <= _bytes(*outs) + ws + SLACK
    assert _bytes(*outs) + ws <= PER_ROW_CAP * N


def test_row_set_forward_scales_with_kept_rows(inputs):
    logits, targets, _ = inputs
    idx = torch.arange(0, N, 2, dtype=torch.int32, device=DEV)
    m = idx.numel()
    grew, outs = _peak_growth(lambda: vwc.selected_logprob_fwd_rows(
        logits, targets, idx, want=("logprob", "lse", "entropy")))
    log(f"fwd_rows: grew {grew} B for {m} rows")
    assert grew <= _bytes(*outs) + vwc.workspace_bytes(m, V, torch.bfloat16) + SLACK
    assert grew <= PER_ROW_CAP * m + SLACK


def test_backward_allocates_only_the_gradient(inputs):
    logits, targets, grad_out = inputs
    _, lse, _ = vwc.selected_logprob_fwd(logits, targets, want=("lse",))
    grew, g = _peak_growth(lambda: vwc.selected_logprob_bwd(logits, targets, lse, grad_out))
    log(f"bwd: grew {grew} B, gradient {_bytes(g)} B")
    assert g.dtype == torch.bfloat16
    assert grew <= _bytes(g) + SLACK


def test_inplace_backward_allocates_nothing(inputs):
    logits, targets, grad_out = inputs
    x = logits.clone()
    _, lse, _ = vwc.selected_logprob_fwd(x, targets, want=("lse",))
    grew, g = _peak_growth(lambda: vwc.selected_logprob_bwd(x, targets, lse, grad_out,
                                                            grad_logits=x))
    log(f"bwd in place: grew {grew} B")
    assert g.data_ptr() == x.data_ptr()
    assert grew <= SLACK


def test_one_call_forward_backward_allocates_only_its_outputs(inputs):
    logits, targets, grad_out = inputs
    grew, outs = _peak_growth(lambda: vwc.selected_logprob_fwd_bwd(logits, targets, grad_out))
    log(f"fwd+bwd in one call: grew {grew} B")
    assert grew <= _bytes(*outs) + vwc.workspace_bytes(N, V, torch.bfloat16) + SLACK


def test_entropy_one_call_allocates_only_its_outputs(inputs):
    logits, targets, grad_out = inputs
    h = grad_out.flip(0).contiguous()
    grew, outs = _peak_growth(lambda: vwc.logprob_entropy_fwd_bwd(logits, targets, grad_out, h))
    log(f"logprob + entropy fwd+bwd in one call: grew {grew} B")
    assert grew <= _bytes(*outs) + vwc.workspace_bytes(N, V, torch.bfloat16) + SLACK


def test_weighted_nll_in_place_allocates_only_row_outputs(inputs):
    """weighted_nll with inplace=True: the one call writes the gradient over the
    logits, so its forward allocates only per-row outputs and workspace."""
    logits, targets, grad_out = inputs
    base = logits.clone().requires_grad_(True)
    x = base * 1.0  # the logits as an op's output, as from an LM head
    w = grad_out.abs()
    grew, (loss, lp) = _peak_growth(lambda: vwc.weighted_nll(x, targets, w, inplace=True))
    log(f"weighted_nll in place: grew {grew} B")
    assert grew <= N * PER_ROW_CAP + SLACK
    del loss, lp, x, base


def test_entropy_gradient_allocates_only_the_gradient(inputs):
    logits, targets, grad_out = inputs
    _, lse, ent = vwc.selected_logprob_fwd(logits, targets, want=("lse", "entropy"))
    grew, g = _peak_growth(lambda: vwc.logprob_entropy_bwd(
        logits, targets, lse, ent, grad_logprob=grad_out, grad_entropy=grad_out))
    log(f"logprob+entropy bwd: grew {grew} B")
    assert grew <= _bytes(g) + SLACK


def test_topk_kl_allocates_only_outputs_and_row_workspace(inputs):
    logits, _, grad_out = inputs
    k = 64
    g = torch.Generator(device=DEV).manual_seed(12)
    idx = torch.stack([torch.randperm(V, device=DEV, generator=g)[:k] for _ in range(4)])
    idx = idx.repeat(N // 4, 1).to(torch.int32).contiguous()
    tlp = torch.log_softmax(torch.randn(N, k, device=DEV, generator=g), dim=1) - 0.1
    grew, fwd = _peak_growth(lambda: vwc.topk_kl_fwd(logits, idx, tlp))
    log(f"top-k KL fwd: grew {grew} B")
    assert grew <= _bytes(*fwd.values()) + vwc.workspace_bytes(N, V, torch.bfloat16) + SLACK
    grew, gl = _peak_growth(lambda: vwc.topk_kl_bwd(logits, idx, tlp, fwd, grad_out))
    log(f"top-k KL bwd: grew {grew} B")
    assert grew <= _bytes(gl) + SLACK
    del gl
    grew, (f1, g1) = _peak_growth(lambda: vwc.topk_kl_fwd_bwd(logits, idx, tlp, grad_out))
    log(f"top-k KL one call: grew {grew} B")
    assert grew <= (_bytes(g1, *f1.values()) + vwc.workspace_bytes(N, V, torch.bfloat16) +
                    SLACK)


def test_lmhead_never_allocates_logits():
    m, d = 4096, 2560
    g = torch.Generator(device=DEV).manual_seed(13)
    hidden = torch.empty(2 * m, d, dtype=torch.bfloat16, device=DEV).normal_(0, 1, generator=g)
    weight = torch.empty(V, d, dtype=torch.bfloat16, device=DEV).normal_(0, 0.02, generator=g)
    targets = torch.randint(0, V, (2 * m,), dtype=torch.int32, device=DEV, generator=g)
    idx = torch.arange(1, 2 * m, 2, dtype=torch.int32, device=DEV)
    ws = vwc.lmhead_workspace_bytes(m, V, d)
    grew, outs = _peak_growth(lambda: vwc.lmhead_logprob_fwd(
        hidden, weight, targets, row_idx=idx, want=("logprob", "lse", "entropy")))
    log(f"LM head: grew {grew} B, workspace {ws} B (kept hidden rows {m * d * 2} B)")
    assert grew <= _bytes(*outs) + ws + SLACK
    # the workspace is the kept hidden rows plus one 16-byte partial per 1024 vocabulary
    # entries of a row: 1/256 of even bf16 logits
    assert ws - m * d * 2 <= 16 * (V // 1024 + 1) * m
    assert grew < m * V * 2 // 8
