"""Selected-token log-probabilities, entropy and logit gradients on MI355X.

The computation runs in the HIP library ``libvwc.so`` (hand-written gfx950
kernels behind a C ABI declared in ``include/vwc.h``).  This package is its
thin Python binding: it turns torch tensors into pointers, sizes and a stream
and calls the library.  There is no fallback: if the library is missing the
import of the binding raises.
"""
from ._binding import (  # noqa: F401
    VWC_BF16, VWC_FP32, VWC_GRAD_COMPACT, VWC_GRAD_SCATTER, VWC_KL_TAIL, VWC_KL_TRUNCATED,
    VwcError, abi_version, entropy,
    entropy_rows, library_path, lmhead_logprob_fwd, lmhead_workspace_bytes,
    logprob_entropy_bwd, logprob_entropy_bwd_rows, logprob_entropy_fwd_bwd,
    logprob_entropy_fwd_bwd_rows, mask_to_index, mask_to_index_workspace_bytes,
    partial_combine, selected_logprob_bwd, selected_logprob_bwd_rows, selected_logprob_fwd,
    selected_logprob_fwd_bwd, selected_logprob_fwd_bwd_rows, selected_logprob_fwd_noalloc,
    selected_logprob_fwd_rows, topk_kl_bwd, topk_kl_bwd_rows, topk_kl_fwd, topk_kl_fwd_bwd,
    topk_kl_fwd_bwd_rows, topk_kl_fwd_rows,
    vocab_partial, workspace_bytes,
)
from .autograd import selected_logprob, topk_kl, weighted_nll, weighted_topk_kl  # noqa: F401,E402
