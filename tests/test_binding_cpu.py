"""The Python binding refuses, before any library call, arguments the kernels
would read out of bounds or from host memory (no GPU needed: these raise first)."""
import pytest
import torch

import vocab_wide_cross_amd as vwc


def _x(n=4, v=16, dtype=torch.bfloat16):
    return torch.zeros(n, v, dtype=dtype)


def test_host_tensors_are_refused():
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        vwc.selected_logprob_fwd(_x(), t)
    with pytest.raises(ValueError, match="GPU"):
        vwc.mask_to_index(torch.ones(8, dtype=torch.uint8))


def test_short_or_mistyped_inputs_are_refused():
    x = _x()
    t = torch.zeros(4, dtype=torch.int32)
    f32 = torch.zeros(4)
    with pytest.raises(ValueError, match="at least 4"):
        vwc.selected_logprob_fwd(x, t[:2])
    with pytest.raises(TypeError, match="int32"):
        vwc.selected_logprob_fwd(x, t.long())
    with pytest.raises(ValueError, match="lse"):
        vwc.selected_logprob_bwd(x, t, f32.half(), f32)
    with pytest.raises(ValueError, match="grad_logprob"):
        vwc.selected_logprob_bwd(x, t, f32, f32[:3])
    with pytest.raises(ValueError, match="grad_logits"):
        vwc.selected_logprob_bwd(x, t, f32, f32, grad_logits=_x(3))
    rows = torch.tensor([0, 2], dtype=torch.int32)
    with pytest.raises(ValueError, match="grad_logits"):  # scatter layout needs every row
        vwc.selected_logprob_bwd_rows(x, t, rows, f32[:2], f32[:2], grad_logits=_x(2),
                                      layout=vwc.VWC_GRAD_SCATTER)
    with pytest.raises(ValueError, match="entropy"):
        vwc.logprob_entropy_bwd(x, t, f32, f32[:1], f32, f32)
    with pytest.raises(TypeError, match="dtype"):
        vwc.selected_logprob_fwd(_x(dtype=torch.float16), t)
    with pytest.raises(ValueError, match="unit column stride"):
        vwc.selected_logprob_fwd(_x().t(), t)


def test_topk_and_lmhead_shapes_are_checked():
    x = _x()
    idx = torch.zeros(4, 3, dtype=torch.int32)
    tlp = torch.zeros(4, 3)
    fwd = {k: torch.zeros(4) for k in ("lse", "student_mass", "teacher_mass", "topk_sum")}
    with pytest.raises(ValueError, match="teacher_logprob"):
        vwc.topk_kl_bwd(x, idx, tlp[:, :2], fwd, torch.zeros(4))
    with pytest.raises(ValueError, match="student_mass"):
        vwc.topk_kl_bwd(x, idx, tlp, dict(fwd, student_mass=torch.zeros(2)), torch.zeros(4))
    h = torch.zeros(4, 8, dtype=torch.bfloat16)
    w = torch.zeros(16, 8, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="bfloat16"):
        vwc.lmhead_logprob_fwd(h.float(), w, torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="targets"):
        vwc.lmhead_logprob_fwd(h, w, torch.zeros(2, dtype=torch.int32))


def test_topk_kl_autograd_refuses_inplace_rows():
    x = _x()
    idx = torch.zeros(2, 3, dtype=torch.int32)
    tlp = torch.zeros(2, 3)
    rows = torch.tensor([0, 2], dtype=torch.int32)
    with pytest.raises(ValueError, match="inplace_backward"):
        vwc.topk_kl(x, idx, tlp, row_idx=rows, inplace_backward=True)
    with pytest.raises(ValueError, match="GPU"):  # host tensors never reach the library
        vwc.topk_kl(x, torch.zeros(4, 3, dtype=torch.int32), torch.zeros(4, 3))


def test_weighted_losses_refuse_host_tensors():
    x = _x()
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        vwc.weighted_nll(x, t, torch.zeros(4))
    with pytest.raises(ValueError, match="GPU"):
        vwc.weighted_topk_kl(x, torch.zeros(4, 3, dtype=torch.int32), torch.zeros(4, 3),
                             torch.zeros(4))
