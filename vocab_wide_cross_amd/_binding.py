"""ctypes binding of libvwc.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks their
dtypes/shapes just enough to build the C call, and launches on the current
torch stream (or ``stream``).  All arithmetic happens in the library's HIP
kernels.  Output tensors are allocated by the caller, or here with torch when
``None`` is passed (device memory is PyTorch's job).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libvwc.so")

VWC_OK, VWC_ERR_INVALID_ARG, VWC_ERR_UNSUPPORTED, VWC_ERR_HIP = 0, 1, 2, 3
VWC_BF16, VWC_FP32 = 0, 1
VWC_GRAD_COMPACT, VWC_GRAD_SCATTER = 0, 1
VWC_KL_TRUNCATED, VWC_KL_TAIL = 0, 1
PARTIAL_BYTES = 16


class VwcError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64, f32, i32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                            ctypes.c_size_t)
    sig = {
        "vwc_workspace_bytes": ([i64, i64, i32], sz),
        "vwc_selected_logprob_fwd": ([p, i32, i64, i64, i64, p, f32, p, p, p, p, sz, p], i32),
        "vwc_selected_logprob_fwd_noalloc": ([p, i32, i64, i64, i64, p, f32, p, p, p, p], i32),
        "vwc_selected_logprob_fwd_rows": ([p, i32, i64, i64, i64, p, p, i64, f32, p, p, p, p, sz,
                                           p], i32),
        "vwc_entropy": ([p, i32, i64, i64, i64, f32, p, p, p, sz, p], i32),
        "vwc_entropy_rows": ([p, i32, i64, i64, i64, p, i64, f32, p, p, p, sz, p], i32),
        "vwc_selected_logprob_bwd": ([p, i32, i64, i64, i64, p, f32, p, p, p, i32, i64, p], i32),
        "vwc_selected_logprob_fwd_bwd": ([p, i32, i64, i64, i64, p, f32, p, p, p, p, p, i32, i64,
                                          p, sz, p], i32),
        "vwc_selected_logprob_fwd_bwd_rows": ([p, i32, i64, i64, i64, p, p, i64, f32, p, p, p, p, p,
                                               i32, i64, i32, p, sz, p], i32),
        "vwc_logprob_entropy_fwd_bwd": ([p, i32, i64, i64, i64, p, f32, p, p, p, p, p, p, i32, i64,
                                         p, sz, p], i32),
        "vwc_logprob_entropy_fwd_bwd_rows": ([p, i32, i64, i64, i64, p, p, i64, f32, p, p, p, p, p,
                                              p, i32, i64, i32, p, sz, p], i32),
        "vwc_selected_logprob_bwd_rows": ([p, i32, i64, i64, i64, p, p, i64, f32, p, p, p, i32,
                                           i64, i32, p], i32),
        "vwc_logprob_entropy_bwd": ([p, i32, i64, i64, i64, p, f32, p, p, p, p, p, i32, i64, p], i32),
        "vwc_logprob_entropy_bwd_rows": ([p, i32, i64, i64, i64, p, p, i64, f32, p, p, p, p, p, i32,
                                          i64, i32, p], i32),
        "vwc_topk_kl_fwd": ([p, i32, i64, i64, i64, p, p, ctypes.c_int32, i32, f32, f32, p, p, p,
                             p, p, p, sz, p], i32),
        "vwc_topk_kl_bwd": ([p, i32, i64, i64, i64, p, p, ctypes.c_int32, i32, f32, f32, p, p, p,
                             p, p, p, i32, i64, p], i32),
        "vwc_topk_kl_fwd_rows": ([p, i32, i64, i64, i64, p, i64, p, p, ctypes.c_int32, i32, f32,
                                  f32, p, p, p, p, p, p, sz, p], i32),
        "vwc_topk_kl_bwd_rows": ([p, i32, i64, i64, i64, p, i64, p, p, ctypes.c_int32, i32, f32,
                                  f32, p, p, p, p, p, p, i32, i64, i32, p], i32),
        "vwc_topk_kl_fwd_bwd": ([p, i32, i64, i64, i64, p, p, ctypes.c_int32, i32, f32, f32, p,
                                 p, p, p, p, p, p, i32, i64, p, sz, p], i32),
        "vwc_topk_kl_fwd_bwd_rows": ([p, i32, i64, i64, i64, p, i64, p, p, ctypes.c_int32, i32,
                                      f32, f32, p, p, p, p, p, p, p, i32, i64, i32, p, sz, p],
                                     i32),
        "vwc_vocab_partial": ([p, i32, i64, i64, i64, i64, p, p, i64, f32, p, p, sz, p], i32),
        "vwc_partial_combine": ([p, ctypes.c_int32, i64, f32, p, p, p, p], i32),
        "vwc_mask_to_index": ([p, i64, p, p, p], i32),
        "vwc_mask_to_index_workspace_bytes": ([i64], sz),
        "vwc_mask_to_index_ws": ([p, i64, p, p, p, sz, p], i32),
        "vwc_lmhead_workspace_bytes": ([i64, i64, i64], sz),
        "vwc_lmhead_logprob_fwd": ([p, i64, i64, p, i64, i64, i64, p, p, i64, f32, p, p, p, p, sz,
                                    p], i32),
        "vwc_status_string": ([i32], ctypes.c_char_p),
        "vwc_last_error": ([], ctypes.c_char_p),
        "vwc_abi_version": ([], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def _check(status: int):
    if status != VWC_OK:
        raise VwcError(status, _lib.vwc_last_error().decode() or
                       _lib.vwc_status_string(status).decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:  # a host address handed to a kernel would fault the GPU
        raise ValueError("every tensor argument must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, like: torch.Tensor):
    s = stream if stream is not None else torch.cuda.current_stream(like.device)
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return VWC_BF16
    if t.dtype == torch.float32:
        return VWC_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _rows_view(logits: torch.Tensor):
    """(n_rows, vocab, ld) of a 2-D row-major view (unit column stride)."""
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [rows, vocab]")
    if logits.size(1) > 1 and logits.stride(1) != 1:
        raise ValueError("logits must have unit column stride")
    ld = logits.stride(0) if logits.size(0) > 1 else max(logits.size(1), 1)
    return logits.size(0), logits.size(1), ld


def _f32(n, like, out):
    if out is None:
        return torch.empty(n, dtype=torch.float32, device=like.device)
    if out.dtype != torch.float32 or out.numel() != n or not out.is_contiguous():
        raise ValueError("float32 outputs must be contiguous with one entry per row")
    return out


def _i32(t: torch.Tensor, name: str, n: int | None = None):
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    if n is not None and t.numel() < n:
        raise ValueError(f"{name} needs at least {n} entries, got {t.numel()}")
    return t


def _f32_in(t, n: int, name: str):
    """A float32 input the kernels read n entries of (None passes through)."""
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name} must be a contiguous float32 tensor of at least {n} entries")
    return t


def _grad_rows(g, rows: int, vocab: int):
    gn, gv, gld = _rows_view(g)
    if gn < rows or gv < vocab:
        raise ValueError(f"grad_logits must be at least [{rows}, {vocab}]")
    return gld


def workspace_bytes(rows: int, vocab: int, dtype) -> int:
    dt = dtype if isinstance(dtype, int) else _dtype(torch.empty(0, dtype=dtype))
    return int(_lib.vwc_workspace_bytes(rows, vocab, dt))


def _workspace(rows, vocab, logits, workspace):
    need = workspace_bytes(rows, vocab, _dtype(logits))
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    return workspace, workspace.numel() * workspace.element_size()


def abi_version() -> int:
    return int(_lib.vwc_abi_version())


def selected_logprob_fwd(logits, targets, temperature=1.0, logprob=None, lse=None,
                         entropy=None, want=("logprob", "lse"), workspace=None, stream=None):
    """Dense forward; returns (logprob, lse, entropy), None for outputs not asked for."""
    n, v, ld = _rows_view(logits)
    _i32(targets, "targets", n)
    lp = _f32(n, logits, logprob) if (logprob is not None or "logprob" in want) else None
    ls = _f32(n, logits, lse) if (lse is not None or "lse" in want) else None
    en = _f32(n, logits, entropy) if (entropy is not None or "entropy" in want) else None
    ws, wsb = _workspace(n, v, logits, workspace)
    _check(_lib.vwc_selected_logprob_fwd(_ptr(logits), _dtype(logits), n, v, ld, _ptr(targets),
                                         float(temperature), _ptr(lp), _ptr(ls), _ptr(en),
                                         _ptr(ws), wsb, _stream(stream, logits)))
    return lp, ls, en


def selected_logprob_fwd_noalloc(logits, targets, temperature=1.0, logprob=None, lse=None,
                                 entropy=None, want=("logprob", "lse"), stream=None):
    """selected_logprob_fwd without a workspace: the library's fixed per-GPU scratch
    array holds the segment partials (outputs are still allocated here when None)."""
    n, v, ld = _rows_view(logits)
    _i32(targets, "targets", n)
    lp = _f32(n, logits, logprob) if (logprob is not None or "logprob" in want) else None
    ls = _f32(n, logits, lse) if (lse is not None or "lse" in want) else None
    en = _f32(n, logits, entropy) if (entropy is not None or "entropy" in want) else None
    _check(_lib.vwc_selected_logprob_fwd_noalloc(_ptr(logits), _dtype(logits), n, v, ld,
                                                 _ptr(targets), float(temperature), _ptr(lp),
                                                 _ptr(ls), _ptr(en), _stream(stream, logits)))
    return lp, ls, en


def selected_logprob_fwd_rows(logits, targets, row_idx, temperature=1.0, logprob=None, lse=None,
                              entropy=None, want=("logprob", "lse"), workspace=None, stream=None):
    """Forward on rows row_idx; outputs are compact [m]."""
    n, v, ld = _rows_view(logits)
    _i32(targets, "targets", n)
    _i32(row_idx, "row_idx")
    m = row_idx.numel()
    lp = _f32(m, logits, logprob) if (logprob is not None or "logprob" in want) else None
    ls = _f32(m, logits, lse) if (lse is not None or "lse" in want) else None
    en = _f32(m, logits, entropy) if (entropy is not None or "entropy" in want) else None
    ws, wsb = _workspace(m, v, logits, workspace)
    _check(_lib.vwc_selected_logprob_fwd_rows(_ptr(logits), _dtype(logits), n, v, ld,
                                              _ptr(targets), _ptr(row_idx), m, float(temperature),
                                              _ptr(lp), _ptr(ls), _ptr(en), _ptr(ws), wsb,
                                              _stream(stream, logits)))
    return lp, ls, en


def entropy(logits, temperature=1.0, out=None, lse=None, workspace=None, stream=None):
    n, v, ld = _rows_view(logits)
    en = _f32(n, logits, out)
    lse = None if lse is None else _f32(n, logits, lse)
    ws, wsb = _workspace(n, v, logits, workspace)
    _check(_lib.vwc_entropy(_ptr(logits), _dtype(logits), n, v, ld, float(temperature), _ptr(en),
                            _ptr(lse), _ptr(ws), wsb, _stream(stream, logits)))
    return en


def entropy_rows(logits, row_idx, temperature=1.0, out=None, lse=None, workspace=None,
                 stream=None):
    n, v, ld = _rows_view(logits)
    _i32(row_idx, "row_idx")
    m = row_idx.numel()
    en = _f32(m, logits, out)
    lse = None if lse is None else _f32(m, logits, lse)
    ws, wsb = _workspace(m, v, logits, workspace)
    _check(_lib.vwc_entropy_rows(_ptr(logits), _dtype(logits), n, v, ld, _ptr(row_idx), m,
                                 float(temperature), _ptr(en), _ptr(lse), _ptr(ws), wsb,
                                 _stream(stream, logits)))
    return en


def _grad_out(logits, rows, grad_logits, grad_dtype):
    if grad_logits is None:
        return torch.empty((rows, logits.size(1)), dtype=grad_dtype or logits.dtype,
                           device=logits.device)
    return grad_logits


def selected_logprob_bwd(logits, targets, lse, grad_logprob, temperature=1.0, grad_logits=None,
                         grad_dtype=None, stream=None):
    """Dense backward: grad_logits[r, j] = g_r ([j == t_r] - p_rj) / tau."""
    n, v, ld = _rows_view(logits)
    _i32(targets, "targets", n)
    _f32_in(lse, n, "lse")
    _f32_in(grad_logprob, n, "grad_logprob")
    g = _grad_out(logits, n, grad_logits, grad_dtype)
    gld = _grad_rows(g, n, v)
    _check(_lib.vwc_selected_logprob_bwd(_ptr(logits), _dtype(logits), n, v, ld, _ptr(targets),
                                         float(temperature), _ptr(lse), _ptr(grad_logprob),
                                         _ptr(g), _dtype(g), gld, _stream(stream, logits)))
    return g


def selected_logprob_fwd_bwd(logits, targets, grad_logprob, temperature=1.0, logprob=None,
                             lse=None, entropy=None, want=("logprob", "lse"), grad_logits=None,
                             grad_dtype=None, workspace=None, stream=None):
    """Forward and backward in one call for a loss weight grad_logprob known up front;
    returns (logprob, lse, entropy, grad_logits), None for outputs not asked for (lse is
    always produced)."""
    n, v, ld = _rows_view(logits)
    _i32(targets, "targets", n)
    _f32_in(grad_logprob, n, "grad_logprob")
    lp = _f32(n, logits, logprob) if (logprob is not None or "logprob" in want) else None
    ls = _f32(n, logits, lse)
    en = _f32(n, logits, entropy) if (entropy is not None or "entropy" in want) else None
    g = _grad_out(logits, n, grad_logits, grad_dtype)
    gld = _grad_rows(g, n, v)
    ws, wsb = _workspace(n, v, logits, workspace)
    _check(_lib.vwc_selected_logprob_fwd_bwd(_ptr(logits), _dtype(logits), n, v, ld,
                                             _ptr(targets), float(temperature),
                                             _ptr(grad_logprob), _ptr(lp), _ptr(ls), _ptr(en),
                                             _ptr(g), _dtype(g), gld, _ptr(ws), wsb,
                                             _stream(stream, logits)))
    return lp, ls, en, g


def logprob_entropy_fwd_bwd(logits, targets, grad_logprob, grad_entropy, temperature=1.0,
                            logprob=None, lse=None, entropy=None, want=("logprob", "lse", "entropy"),
                            grad_logits=None, grad_dtype=None, workspace=None, stream=None):
    """Forward and the logprob + entropy backward in one call for loss weights
    grad_logprob (g, or None: 0) and grad_entropy (h) known up front; returns (logprob,
    lse, entropy, grad_logits), None for logprob when not asked for."""
    n, v, ld = _rows_view(logits)
    if targets is not None:
        _i32(targets, "targets", n)
    if grad_logprob is not None:
        _f32_in(grad_logprob, n, "grad_logprob")
    _f32_in(grad_entropy, n, "grad_entropy")
    lp = _f32(n, logits, logprob) if (logprob is not None or "logprob" in want) else None
    ls = _f32(n, logits, lse)
    en = _f32(n, logits, entropy)
    g = _grad_out(logits, n, grad_logits, grad_dtype)
    gld = _grad_rows(g, n, v)
    ws, wsb = _workspace(n, v, logits, workspace)
    _check(_lib.vwc_logprob_entropy_fwd_bwd(_ptr(logits), _dtype(logits), n, v, ld,
                                            _ptr(targets), float(temperature), _ptr(grad_logprob),
                                            _ptr(grad_entropy), _ptr(lp), _ptr(ls), _ptr(en),
                                            _ptr(g), _dtype(g), gld, _ptr(ws), wsb,
                                            _stream(stream, logits)))
    return lp, ls, en, g


def logprob_entropy_fwd_bwd_rows(logits, targets, row_idx, grad_logprob, grad_entropy,
                                 temperature=1.0, logprob=None, lse=None, entropy=None,
                                 want=("logprob", "lse", "entropy"), grad_logits=None,
                                 grad_dtype=None, layout=VWC_GRAD_COMPACT, workspace=None,
                                 stream=None):
    """The one-call logprob + entropy forward and backward over a row set; weights and
    outputs compact [m]; returns (logprob, lse, entropy, grad_logits)."""
    n, v, ld = _rows_view(logits)
    if targets is not None:
        _i32(targets, "targets", n)
    _i32(row_idx, "row_idx")
    m = row_idx.numel()
    if grad_logprob is not None:
        _f32_in(grad_logprob, m, "grad_logprob")
    _f32_in(grad_entropy, m, "grad_entropy")
    lp = _f32(m, logits, logprob) if (logprob is not None or "logprob" in want) else None
    ls = _f32(m, logits, lse)
    en = _f32(m, logits, entropy)
    rows = m if layout == VWC_GRAD_COMPACT else n
    if grad_logits is None:
        grad_logits = _grad_out(logits, rows, None, grad_dtype)
        if layout == VWC_GRAD_SCATTER:
            grad_logits.zero_()
    gld = _grad_rows(grad_logits, rows, v)
    ws, wsb = _workspace(m, v, logits, workspace)
    _check(_lib.vwc_logprob_entropy_fwd_bwd_rows(_ptr(logits), _dtype(logits), n, v, ld,
                                                 _ptr(targets), _ptr(row_idx), m,
                                                 float(temperature), _ptr(grad_logprob),
                                                 _ptr(grad_entropy), _ptr(lp), _ptr(ls), _ptr(en),
                                                 _ptr(grad_logits), _dtype(grad_logits), gld,
                                                 layout, _ptr(ws), wsb, _stream(stream, logits)))
    return lp, ls, en, grad_logits


def selected_logprob_fwd_bwd_rows(logits, targets, row_idx, grad_logprob, temperature=1.0,
                                  logprob=None, lse=None, entropy=None, want=("logprob", "lse"),
                                  grad_logits=None, grad_dtype=None, layout=VWC_GRAD_COMPACT,
                                  workspace=None, stream=None):
    """The one-call forward + backward over a row set; outputs and grad_logprob compact [m];
    returns (logprob, lse, entropy, grad_logits)."""
    n, v, ld = _rows_view(logits)
    _i32(targets, "targets", n)
    _i32(row_idx, "row_idx")
    m = row_idx.numel()
    _f32_in(grad_logprob, m, "grad_logprob")
    lp = _f32(m, logits, logprob) if (logprob is not None or "logprob" in want) else None
    ls = _f32(m, logits, lse)
    en = _f32(m, logits, entropy) if (entropy is not None or "entropy" in want) else None
    rows = m if layout == VWC_GRAD_COMPACT else n
    if grad_logits is None:
        grad_logits = _grad_out(logits, rows, None, grad_dtype)
        if layout == VWC_GRAD_SCATTER:
            grad_logits.zero_()
    gld = _grad_rows(grad_logits, rows, v)
    ws, wsb = _workspace(m, v, logits, workspace)
    _check(_lib.vwc_selected_logprob_fwd_bwd_rows(_ptr(logits), _dtype(logits), n, v, ld,
                                                  _ptr(targets), _ptr(row_idx), m,
                                                  float(temperature), _ptr(grad_logprob),
                                                  _ptr(lp), _ptr(ls), _ptr(en),
                                                  _ptr(grad_logits), _dtype(grad_logits), gld,
                                                  layout, _ptr(ws), wsb,
                                                  _stream(stream, logits)))
    return lp, ls, en, grad_logits


def selected_logprob_bwd_rows(logits, targets, row_idx, lse, grad_logprob, temperature=1.0,
                              grad_logits=None, grad_dtype=None, layout=VWC_GRAD_COMPACT,
                              stream=None):
    n, v, ld = _rows_view(logits)
    _i32(targets, "targets", n)
    _i32(row_idx, "row_idx")
    m = row_idx.numel()
    _f32_in(lse, m, "lse")
    _f32_in(grad_logprob, m, "grad_logprob")
    rows = m if layout == VWC_GRAD_COMPACT else n
    if grad_logits is None:
        grad_logits = _grad_out(logits, rows, None, grad_dtype)
        if layout == VWC_GRAD_SCATTER:
            grad_logits.zero_()
    gld = _grad_rows(grad_logits, rows, v)
    _check(_lib.vwc_selected_logprob_bwd_rows(_ptr(logits), _dtype(logits), n, v, ld,
                                              _ptr(targets), _ptr(row_idx), m,
                                              float(temperature), _ptr(lse), _ptr(grad_logprob),
                                              _ptr(grad_logits), _dtype(grad_logits), gld,
                                              layout, _stream(stream, logits)))
    return grad_logits


def logprob_entropy_bwd(logits, targets, lse, entropy, grad_logprob=None, grad_entropy=None,
                        temperature=1.0, grad_logits=None, grad_dtype=None, stream=None):
    """Dense backward of sum_r g_r logprob_r + h_r entropy_r (g or h may be None)."""
    n, v, ld = _rows_view(logits)
    if targets is not None:
        _i32(targets, "targets", n)
    for t, name in ((lse, "lse"), (entropy, "entropy"), (grad_logprob, "grad_logprob"),
                    (grad_entropy, "grad_entropy")):
        _f32_in(t, n, name)
    g = _grad_out(logits, n, grad_logits, grad_dtype)
    gld = _grad_rows(g, n, v)
    _check(_lib.vwc_logprob_entropy_bwd(_ptr(logits), _dtype(logits), n, v, ld, _ptr(targets),
                                        float(temperature), _ptr(lse), _ptr(entropy),
                                        _ptr(grad_logprob), _ptr(grad_entropy), _ptr(g), _dtype(g),
                                        gld, _stream(stream, logits)))
    return g


def logprob_entropy_bwd_rows(logits, targets, row_idx, lse, entropy, grad_logprob=None,
                             grad_entropy=None, temperature=1.0, grad_logits=None, grad_dtype=None,
                             layout=VWC_GRAD_COMPACT, stream=None):
    """Compact-row version of logprob_entropy_bwd (lse/entropy/gradients are [m])."""
    n, v, ld = _rows_view(logits)
    if targets is not None:
        _i32(targets, "targets", n)
    _i32(row_idx, "row_idx")
    m = row_idx.numel()
    for t, name in ((lse, "lse"), (entropy, "entropy"), (grad_logprob, "grad_logprob"),
                    (grad_entropy, "grad_entropy")):
        _f32_in(t, m, name)
    rows = m if layout == VWC_GRAD_COMPACT else n
    if grad_logits is None:
        grad_logits = _grad_out(logits, rows, None, grad_dtype)
        if layout == VWC_GRAD_SCATTER:
            grad_logits.zero_()
    gld = _grad_rows(grad_logits, rows, v)
    _check(_lib.vwc_logprob_entropy_bwd_rows(_ptr(logits), _dtype(logits), n, v, ld,
                                             _ptr(targets), _ptr(row_idx), m, float(temperature),
                                             _ptr(lse), _ptr(entropy), _ptr(grad_logprob),
                                             _ptr(grad_entropy), _ptr(grad_logits),
                                             _dtype(grad_logits), gld, layout,
                                             _stream(stream, logits)))
    return grad_logits


def topk_kl_fwd(logits, topk_idx, teacher_logprob, mode=VWC_KL_TAIL, tail_mass_eps=1e-6,
                temperature=1.0, workspace=None, stream=None):
    """Top-k forward KL per row; returns dict of float32 [n_rows] tensors:
    loss, student_mass, teacher_mass, topk_sum, lse."""
    n, v, ld = _rows_view(logits)
    _i32(topk_idx, "topk_idx")
    if topk_idx.dim() != 2 or topk_idx.size(0) != n or teacher_logprob.shape != topk_idx.shape \
            or teacher_logprob.dtype != torch.float32 or not teacher_logprob.is_contiguous():
        raise ValueError("topk_idx int32 and teacher_logprob float32 must both be [n_rows, k]")
    k = topk_idx.size(1)
    out = {name: torch.empty(n, dtype=torch.float32, device=logits.device)
           for name in ("loss", "student_mass", "teacher_mass", "topk_sum", "lse")}
    ws, wsb = _workspace(n, v, logits, workspace)
    _check(_lib.vwc_topk_kl_fwd(_ptr(logits), _dtype(logits), n, v, ld, _ptr(topk_idx),
                                _ptr(teacher_logprob), k, int(mode), float(tail_mass_eps),
                                float(temperature), _ptr(out["loss"]), _ptr(out["student_mass"]),
                                _ptr(out["teacher_mass"]), _ptr(out["topk_sum"]),
                                _ptr(out["lse"]), _ptr(ws), wsb, _stream(stream, logits)))
    return out


def topk_kl_bwd(logits, topk_idx, teacher_logprob, fwd, grad_loss, mode=VWC_KL_TAIL,
                tail_mass_eps=1e-6, temperature=1.0, grad_logits=None, grad_dtype=None,
                stream=None):
    """Gradient of sum_r grad_loss[r] * loss[r] w.r.t. the student logits; `fwd` is the
    dict topk_kl_fwd returned."""
    n, v, ld = _rows_view(logits)
    _i32(topk_idx, "topk_idx")
    if topk_idx.dim() != 2 or topk_idx.size(0) != n or teacher_logprob.shape != topk_idx.shape:
        raise ValueError("topk_idx and teacher_logprob must both be [n_rows, k]")
    _f32_in(teacher_logprob, topk_idx.numel(), "teacher_logprob")
    for name in ("lse", "student_mass", "teacher_mass", "topk_sum"):
        _f32_in(fwd[name], n, name)
    _f32_in(grad_loss, n, "grad_loss")
    g = _grad_out(logits, n, grad_logits, grad_dtype)
    gld = _grad_rows(g, n, v)
    _check(_lib.vwc_topk_kl_bwd(_ptr(logits), _dtype(logits), n, v, ld, _ptr(topk_idx),
                                _ptr(teacher_logprob), topk_idx.size(1), int(mode),
                                float(tail_mass_eps), float(temperature), _ptr(fwd["lse"]),
                                _ptr(fwd["student_mass"]), _ptr(fwd["teacher_mass"]),
                                _ptr(fwd["topk_sum"]), _ptr(grad_loss), _ptr(g), _dtype(g), gld,
                                _stream(stream, logits)))
    return g


def topk_kl_fwd_bwd(logits, topk_idx, teacher_logprob, grad_loss, mode=VWC_KL_TAIL,
                    tail_mass_eps=1e-6, temperature=1.0, grad_logits=None, grad_dtype=None,
                    workspace=None, stream=None):
    """Top-k KL forward and backward in one call for a loss weight grad_loss known up front;
    returns (dict of float32 [n_rows] tensors as topk_kl_fwd, grad_logits)."""
    n, v, ld = _rows_view(logits)
    _i32(topk_idx, "topk_idx")
    if topk_idx.dim() != 2 or topk_idx.size(0) != n or teacher_logprob.shape != topk_idx.shape:
        raise ValueError("topk_idx and teacher_logprob must both be [n_rows, k]")
    _f32_in(teacher_logprob, topk_idx.numel(), "teacher_logprob")
    _f32_in(grad_loss, n, "grad_loss")
    out = {name: torch.empty(n, dtype=torch.float32, device=logits.device)
           for name in ("loss", "student_mass", "teacher_mass", "topk_sum", "lse")}
    g = _grad_out(logits, n, grad_logits, grad_dtype)
    gld = _grad_rows(g, n, v)
    ws, wsb = _workspace(n, v, logits, workspace)
    _check(_lib.vwc_topk_kl_fwd_bwd(_ptr(logits), _dtype(logits), n, v, ld, _ptr(topk_idx),
                                    _ptr(teacher_logprob), topk_idx.size(1), int(mode),
                                    float(tail_mass_eps), float(temperature), _ptr(grad_loss),
                                    _ptr(out["loss"]), _ptr(out["student_mass"]),
                                    _ptr(out["teacher_mass"]), _ptr(out["topk_sum"]),
                                    _ptr(out["lse"]), _ptr(g), _dtype(g), gld, _ptr(ws), wsb,
                                    _stream(stream, logits)))
    return out, g


def topk_kl_fwd_bwd_rows(logits, row_idx, topk_idx, teacher_logprob, grad_loss,
                         mode=VWC_KL_TAIL, tail_mass_eps=1e-6, temperature=1.0, grad_logits=None,
                         grad_dtype=None, layout=VWC_GRAD_COMPACT, workspace=None, stream=None):
    """The one-call top-k KL over the rows row_idx; payload [m, k], grad_loss and outputs [m];
    returns (dict as topk_kl_fwd_rows, grad_logits compact [m, vocab] or scattered)."""
    n, v, ld = _rows_view(logits)
    _i32(row_idx, "row_idx")
    m = row_idx.numel()
    _i32(topk_idx, "topk_idx")
    if topk_idx.dim() != 2 or topk_idx.size(0) != m or teacher_logprob.shape != topk_idx.shape:
        raise ValueError("topk_idx and teacher_logprob must both be [m, k]")
    _f32_in(teacher_logprob, topk_idx.numel(), "teacher_logprob")
    _f32_in(grad_loss, m, "grad_loss")
    out = {name: torch.empty(m, dtype=torch.float32, device=logits.device)
           for name in ("loss", "student_mass", "teacher_mass", "topk_sum", "lse")}
    rows = m if layout == VWC_GRAD_COMPACT else n
    if grad_logits is None:
        grad_logits = _grad_out(logits, rows, None, grad_dtype)
        if layout == VWC_GRAD_SCATTER:
            grad_logits.zero_()
    gld = _grad_rows(grad_logits, rows, v)
    ws, wsb = _workspace(m, v, logits, workspace)
    _check(_lib.vwc_topk_kl_fwd_bwd_rows(_ptr(logits), _dtype(logits), n, v, ld, _ptr(row_idx),
                                         m, _ptr(topk_idx), _ptr(teacher_logprob),
                                         topk_idx.size(1), int(mode), float(tail_mass_eps),
                                         float(temperature), _ptr(grad_loss), _ptr(out["loss"]),
                                         _ptr(out["student_mass"]), _ptr(out["teacher_mass"]),
                                         _ptr(out["topk_sum"]), _ptr(out["lse"]),
                                         _ptr(grad_logits), _dtype(grad_logits), gld, layout,
                                         _ptr(ws), wsb, _stream(stream, logits)))
    return out, grad_logits


def topk_kl_fwd_rows(logits, row_idx, topk_idx, teacher_logprob, mode=VWC_KL_TAIL,
                     tail_mass_eps=1e-6, temperature=1.0, workspace=None, stream=None):
    """Top-k forward KL of the rows row_idx; topk_idx / teacher_logprob are [m, k] (one
    payload per listed row); returns dict of float32 [m] tensors as topk_kl_fwd."""
    n, v, ld = _rows_view(logits)
    _i32(row_idx, "row_idx")
    m = row_idx.numel()
    _i32(topk_idx, "topk_idx")
    if topk_idx.dim() != 2 or topk_idx.size(0) != m or teacher_logprob.shape != topk_idx.shape:
        raise ValueError("topk_idx and teacher_logprob must both be [m, k]")
    _f32_in(teacher_logprob, topk_idx.numel(), "teacher_logprob")
    k = topk_idx.size(1)
    out = {name: torch.empty(m, dtype=torch.float32, device=logits.device)
           for name in ("loss", "student_mass", "teacher_mass", "topk_sum", "lse")}
    ws, wsb = _workspace(m, v, logits, workspace)
    _check(_lib.vwc_topk_kl_fwd_rows(_ptr(logits), _dtype(logits), n, v, ld, _ptr(row_idx), m,
                                     _ptr(topk_idx), _ptr(teacher_logprob), k, int(mode),
                                     float(tail_mass_eps), float(temperature), _ptr(out["loss"]),
                                     _ptr(out["student_mass"]), _ptr(out["teacher_mass"]),
                                     _ptr(out["topk_sum"]), _ptr(out["lse"]), _ptr(ws), wsb,
                                     _stream(stream, logits)))
    return out


def topk_kl_bwd_rows(logits, row_idx, topk_idx, teacher_logprob, fwd, grad_loss,
                     mode=VWC_KL_TAIL, tail_mass_eps=1e-6, temperature=1.0, grad_logits=None,
                     grad_dtype=None, layout=VWC_GRAD_COMPACT, stream=None):
    """Gradient of sum_i grad_loss[i] * loss[i] over the rows row_idx; `fwd` is the dict
    topk_kl_fwd_rows returned.  layout: compact [m, vocab] or scatter into [n_rows, vocab]."""
    n, v, ld = _rows_view(logits)
    _i32(row_idx, "row_idx")
    m = row_idx.numel()
    _i32(topk_idx, "topk_idx")
    if topk_idx.dim() != 2 or topk_idx.size(0) != m or teacher_logprob.shape != topk_idx.shape:
        raise ValueError("topk_idx and teacher_logprob must both be [m, k]")
    _f32_in(teacher_logprob, topk_idx.numel(), "teacher_logprob")
    for name in ("lse", "student_mass", "teacher_mass", "topk_sum"):
        _f32_in(fwd[name], m, name)
    _f32_in(grad_loss, m, "grad_loss")
    rows = m if layout == VWC_GRAD_COMPACT else n
    if grad_logits is None:
        grad_logits = _grad_out(logits, rows, None, grad_dtype)
        if layout == VWC_GRAD_SCATTER:
            grad_logits.zero_()
    gld = _grad_rows(grad_logits, rows, v)
    _check(_lib.vwc_topk_kl_bwd_rows(_ptr(logits), _dtype(logits), n, v, ld, _ptr(row_idx), m,
                                     _ptr(topk_idx), _ptr(teacher_logprob), topk_idx.size(1),
                                     int(mode), float(tail_mass_eps), float(temperature),
                                     _ptr(fwd["lse"]), _ptr(fwd["student_mass"]),
                                     _ptr(fwd["teacher_mass"]), _ptr(fwd["topk_sum"]),
                                     _ptr(grad_loss), _ptr(grad_logits), _dtype(grad_logits), gld,
                                     layout, _stream(stream, logits)))
    return grad_logits


def vocab_partial(logits_slice, v_start, targets=None, row_idx=None, temperature=1.0, out=None,
                  workspace=None, stream=None):
    """Partial (m, s, t, w) of a vocabulary slice; returns a [m, 4] float32 tensor."""
    n, v, ld = _rows_view(logits_slice)
    if targets is not None:
        _i32(targets, "targets", n)
    if row_idx is not None:
        _i32(row_idx, "row_idx")
    m = n if row_idx is None else row_idx.numel()
    if out is None:
        out = torch.empty((m, 4), dtype=torch.float32, device=logits_slice.device)
    _f32_in(out, 4 * m, "out")
    ws, wsb = _workspace(m, v, logits_slice, workspace)
    _check(_lib.vwc_vocab_partial(_ptr(logits_slice), _dtype(logits_slice), n, v, ld, v_start,
                                  _ptr(targets), _ptr(row_idx), m, float(temperature), _ptr(out),
                                  _ptr(ws), wsb, _stream(stream, logits_slice)))
    return out


def partial_combine(parts, temperature=1.0, logprob=None, lse=None, entropy=None,
                    want=("logprob", "lse", "entropy"), stream=None):
    """Merge [k, rows, 4] float32 partials (slice-major) into per-row outputs."""
    if parts.dim() != 3 or parts.size(2) != 4 or parts.dtype != torch.float32 \
            or not parts.is_contiguous():
        raise ValueError("parts must be a contiguous float32 [k, rows, 4] tensor")
    k, rows = parts.size(0), parts.size(1)
    lp = _f32(rows, parts, logprob) if (logprob is not None or "logprob" in want) else None
    ls = _f32(rows, parts, lse) if (lse is not None or "lse" in want) else None
    en = _f32(rows, parts, entropy) if (entropy is not None or "entropy" in want) else None
    _check(_lib.vwc_partial_combine(_ptr(parts), k, rows, float(temperature), _ptr(lp), _ptr(ls),
                                    _ptr(en), _stream(stream, parts)))
    return lp, ls, en


def mask_to_index_workspace_bytes(n: int) -> int:
    return int(_lib.vwc_mask_to_index_workspace_bytes(n))


def mask_to_index(mask, row_idx=None, count=None, workspace=None, one_group=False, stream=None):
    """Ascending int32 ids of the nonzero entries of a uint8/bool mask (device count).
    Long masks take the tiled scan over the whole GPU (vwc_mask_to_index_ws, with a
    workspace allocated here when none is passed); one_group=True forces the
    one-workgroup call (vwc_mask_to_index)."""
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    if mask.dtype != torch.uint8 or not mask.is_contiguous():
        raise TypeError("mask must be a contiguous uint8 or bool tensor")
    n = mask.numel()
    if row_idx is None:
        row_idx = torch.empty(max(n, 1), dtype=torch.int32, device=mask.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=mask.device)
    _i32(row_idx, "row_idx", n)
    _i32(count, "count", 1)
    if one_group:
        _check(_lib.vwc_mask_to_index(_ptr(mask), n, _ptr(row_idx), _ptr(count),
                                      _stream(stream, mask)))
        return row_idx, count
    need = mask_to_index_workspace_bytes(n)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=mask.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.vwc_mask_to_index_ws(_ptr(mask), n, _ptr(row_idx), _ptr(count), _ptr(workspace),
                                     wsb, _stream(stream, mask)))
    return row_idx, count


def lmhead_workspace_bytes(rows: int, vocab: int, d: int) -> int:
    return int(_lib.vwc_lmhead_workspace_bytes(rows, vocab, d))


def lmhead_logprob_fwd(hidden, weight, targets=None, row_idx=None, temperature=1.0,
                       logprob=None, lse=None, entropy=None, want=("logprob", "lse"), d=None,
                       workspace=None, stream=None):
    """Fused LM head: logprob / lse / entropy of hidden[row_idx] @ weight.T without
    materialising the logits.  hidden [n_rows, >= d] and weight [vocab, >= d] are
    bfloat16 with unit column stride; outputs are compact [m] float32."""
    for t, name in ((hidden, "hidden"), (weight, "weight")):
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
    n, kh, ldh = _rows_view(hidden)
    v, kw, ldw = _rows_view(weight)
    d = min(kh, kw) if d is None else int(d)
    if targets is not None:
        _i32(targets, "targets", n)
    if row_idx is not None:
        _i32(row_idx, "row_idx")
    m = n if row_idx is None else row_idx.numel()
    lp = _f32(m, hidden, logprob) if (logprob is not None or "logprob" in want) else None
    ls = _f32(m, hidden, lse) if (lse is not None or "lse" in want) else None
    en = _f32(m, hidden, entropy) if (entropy is not None or "entropy" in want) else None
    need = lmhead_workspace_bytes(m, v, d)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=hidden.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.vwc_lmhead_logprob_fwd(_ptr(hidden), n, ldh, _ptr(weight), v, ldw, d,
                                       _ptr(targets), _ptr(row_idx), m, float(temperature),
                                       _ptr(lp), _ptr(ls), _ptr(en), _ptr(workspace), wsb,
                                       _stream(stream, hidden)))
    return lp, ls, en
