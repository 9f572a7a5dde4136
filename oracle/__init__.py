"""fp64 CPU oracle for selected-token log-probabilities (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it.  It shares no code with the HIP
path; the two meet only in the seeded input generators of ``workloads``.

The arithmetic lives in ``oracle.c`` (plain C, double precision, one row at a
time).  This module is marshalling: numpy arrays in, numpy arrays out.  The one
exception is ``lmhead_blocked``: the LM head's definition in float64 numpy with
the projection of a block of kept rows as one BLAS matrix product, fast enough to
check every kept row of a full-size call.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16 = 0
FP32 = 1
FP64 = 2

_ERRORS = {
    -1: "invalid argument",
    -2: "target out of range",
    -3: "row index out of range",
    -4: "out of memory",
}


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_ERRORS.get(code, code)}")
        self.code = code


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (strict IEEE double, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB points the tests at another build: a deliberately broken copy
        # (mutation checks) or a sanitizer-instrumented one.
        path = os.environ.get("ORACLE_LIB") or _LIB_PATH
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(path)
        p, i64, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
        lib.oracle_forward.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, i64, d, i64, p, p, p]
        lib.oracle_backward.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, i64, d, p, p]
        lib.oracle_backward_entropy.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, i64, d, p,
                                                p, p]
        lib.oracle_topk_kl_forward.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, i64,
                                               ctypes.c_int, d, d, p, p, p]
        lib.oracle_topk_kl_backward.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, i64,
                                                ctypes.c_int, d, d, p, p]
        lib.oracle_slice_partial.argtypes = [p, ctypes.c_int, i64, i64, i64, i64, p, p, i64, d,
                                             p, p, p, p]
        lib.oracle_combine.argtypes = [i64, i64, p, p, p, p, p, p, p]
        lib.oracle_forward_vchunk.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, i64, d, i64,
                                              p, p, p]
        lib.oracle_lmhead_logits.argtypes = [p, i64, i64, p, i64, i64, i64, p, i64, p, p]
        lib.oracle_lmhead_forward.argtypes = [p, i64, i64, p, i64, i64, i64, p, p, i64, d, i64,
                                              p, p, p, p]
        lib.oracle_bf16_rne.argtypes = [d]
        lib.oracle_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_bf16_rne_array.argtypes = [p, p, i64]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        for f in ("oracle_forward", "oracle_backward", "oracle_backward_entropy",
                  "oracle_topk_kl_forward", "oracle_topk_kl_backward",
                  "oracle_slice_partial", "oracle_combine", "oracle_forward_vchunk",
                  "oracle_lmhead_logits", "oracle_lmhead_forward"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float32:
        return FP32
    raise TypeError("logits must be uint16 (bf16 bit patterns) or float32")


def _tau(tau) -> float:
    """The temperature crosses the library boundary as a C float; the oracle works on
    that float widened to double (0.7 -> 0.699999988079071)."""
    return float(np.float32(tau))


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(rc, what)


def _rows_arg(rows, n_rows):
    if rows is None:
        return None, n_rows
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    return rows, rows.shape[0]


def _targets_arg(targets):
    return None if targets is None else np.ascontiguousarray(targets, dtype=np.int32)


def forward(x: np.ndarray, targets, tau: float = 1.0, rows=None, row_chunk: int | None = None,
            want=("logprob", "lse", "entropy"), vocab: int | None = None):
    """Per-row logprob / lse / entropy in float64.

    x: [n_rows, ld] uint16 (bf16 bits) or float32; the first ``vocab`` columns
    (default: all) are the vocabulary.  Returns a dict of [m] float64 arrays.
    """
    x = np.ascontiguousarray(x)
    n_rows, ld = x.shape
    vocab = ld if vocab is None else vocab
    rows, m = _rows_arg(rows, n_rows)
    targets = _targets_arg(targets)
    out = {k: (np.empty(m, np.float64) if k in want else None)
           for k in ("logprob", "lse", "entropy")}
    chunk = max(m, 1) if row_chunk is None else row_chunk
    rc = _load().oracle_forward(_ptr(x), _dtype_code(x), n_rows, vocab, ld, _ptr(targets),
                                _ptr(rows), m, _tau(tau), chunk, _ptr(out["logprob"]),
                                _ptr(out["lse"]), _ptr(out["entropy"]))
    _check(rc, "oracle_forward")
    return {k: v for k, v in out.items() if v is not None}


def forward_vchunk(x: np.ndarray, targets, tau: float, vchunk: int, rows=None,
                   want=("logprob", "lse", "entropy"), vocab: int | None = None):
    """Forward through vocabulary chunks of ``vchunk`` columns merged by the combine."""
    x = np.ascontiguousarray(x)
    n_rows, ld = x.shape
    vocab = ld if vocab is None else vocab
    rows, m = _rows_arg(rows, n_rows)
    targets = _targets_arg(targets)
    out = {k: (np.empty(m, np.float64) if k in want else None)
           for k in ("logprob", "lse", "entropy")}
    rc = _load().oracle_forward_vchunk(_ptr(x), _dtype_code(x), n_rows, vocab, ld, _ptr(targets),
                                       _ptr(rows), m, _tau(tau), vchunk, _ptr(out["logprob"]),
                                       _ptr(out["lse"]), _ptr(out["entropy"]))
    _check(rc, "oracle_forward_vchunk")
    return {k: v for k, v in out.items() if v is not None}


def backward(x: np.ndarray, targets, grad_out, tau: float = 1.0, rows=None,
             vocab: int | None = None) -> np.ndarray:
    """[m, vocab] float64 gradient of grad_out[i] * logprob_i w.r.t. the logits."""
    x = np.ascontiguousarray(x)
    n_rows, ld = x.shape
    vocab = ld if vocab is None else vocab
    rows, m = _rows_arg(rows, n_rows)
    targets = _targets_arg(targets)
    g = np.ascontiguousarray(grad_out, dtype=np.float32)
    if g.shape != (m,):
        raise ValueError("grad_out must have one entry per output row")
    grad = np.empty((m, vocab), np.float64)
    rc = _load().oracle_backward(_ptr(x), _dtype_code(x), n_rows, vocab, ld, _ptr(targets),
                                 _ptr(rows), m, _tau(tau), _ptr(g), _ptr(grad))
    _check(rc, "oracle_backward")
    return grad


def backward_entropy(x: np.ndarray, targets, grad_logprob, grad_entropy, tau: float = 1.0,
                     rows=None, vocab: int | None = None) -> np.ndarray:
    """[m, vocab] float64 gradient of sum_i g_i logprob_i + h_i entropy_i w.r.t. the logits;
    grad_logprob (g) or grad_entropy (h) may be None (zero)."""
    x = np.ascontiguousarray(x)
    n_rows, ld = x.shape
    vocab = ld if vocab is None else vocab
    rows, m = _rows_arg(rows, n_rows)
    targets = _targets_arg(targets)
    g = None if grad_logprob is None else np.ascontiguousarray(grad_logprob, dtype=np.float32)
    h = None if grad_entropy is None else np.ascontiguousarray(grad_entropy, dtype=np.float32)
    for a in (g, h):
        if a is not None and a.shape != (m,):
            raise ValueError("gradients must have one entry per output row")
    grad = np.empty((m, vocab), np.float64)
    rc = _load().oracle_backward_entropy(_ptr(x), _dtype_code(x), n_rows, vocab, ld,
                                         _ptr(targets), _ptr(rows), m, _tau(tau), _ptr(g),
                                         _ptr(h), _ptr(grad))
    _check(rc, "oracle_backward_entropy")
    return grad


KL_TRUNCATED = 0
KL_TAIL = 1


def topk_kl_forward(x: np.ndarray, topk_idx, teacher_logprob, mode: int, tail_eps: float = 1e-6,
                    tau: float = 1.0, vocab: int | None = None):
    """Per-row top-k KL loss, student top-k mass Q and teacher mass P (float64)."""
    x = np.ascontiguousarray(x)
    n_rows, ld = x.shape
    vocab = ld if vocab is None else vocab
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    tlp = np.ascontiguousarray(teacher_logprob, dtype=np.float32)
    k = idx.shape[1]
    loss, q, pm = (np.empty(n_rows, np.float64) for _ in range(3))
    rc = _load().oracle_topk_kl_forward(_ptr(x), _dtype_code(x), n_rows, vocab, ld, _ptr(idx),
                                        _ptr(tlp), k, int(mode), float(tail_eps), _tau(tau),
                                        _ptr(loss), _ptr(q), _ptr(pm))
    _check(rc, "oracle_topk_kl_forward")
    return {"loss": loss, "student_mass": q, "teacher_mass": pm}


def topk_kl_backward(x: np.ndarray, topk_idx, teacher_logprob, mode: int, grad_loss,
                     tail_eps: float = 1e-6, tau: float = 1.0, vocab: int | None = None):
    """[n_rows, vocab] float64 gradient of sum_i g_i L_i w.r.t. the student logits."""
    x = np.ascontiguousarray(x)
    n_rows, ld = x.shape
    vocab = ld if vocab is None else vocab
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    tlp = np.ascontiguousarray(teacher_logprob, dtype=np.float32)
    g = np.ascontiguousarray(grad_loss, dtype=np.float32)
    grad = np.empty((n_rows, vocab), np.float64)
    rc = _load().oracle_topk_kl_backward(_ptr(x), _dtype_code(x), n_rows, vocab, ld, _ptr(idx),
                                         _ptr(tlp), idx.shape[1], int(mode), float(tail_eps),
                                         _tau(tau), _ptr(g), _ptr(grad))
    _check(rc, "oracle_topk_kl_backward")
    return grad


def slice_partial(x: np.ndarray, v_start: int, v_local: int, targets, tau: float, rows=None):
    """(m, s, w, t) float64 partial of columns [v_start, v_start + v_local) of x."""
    x = np.ascontiguousarray(x)
    n_rows, ld = x.shape
    if v_start < 0 or v_start + v_local > ld:
        raise ValueError("slice outside the row")
    rows, m = _rows_arg(rows, n_rows)
    targets = _targets_arg(targets)
    pm, ps, pw = (np.empty(m, np.float64) for _ in range(3))
    pt = np.empty(m, np.float64) if targets is not None else None
    base = x.ctypes.data + v_start * x.itemsize
    rc = _load().oracle_slice_partial(ctypes.c_void_p(base), _dtype_code(x), n_rows, v_local, ld,
                                      v_start, _ptr(targets), _ptr(rows), m, _tau(tau),
                                      _ptr(pm), _ptr(ps), _ptr(pw), _ptr(pt))
    _check(rc, "oracle_slice_partial")
    return pm, ps, pw, pt


def combine(pm, ps, pw, pt):
    """Merge [k, m] float64 partial arrays; returns dict of logprob/lse/entropy."""
    pm, ps, pw = (np.ascontiguousarray(a, dtype=np.float64) for a in (pm, ps, pw))
    k, m = pm.shape
    pt = None if pt is None else np.ascontiguousarray(pt, dtype=np.float64)
    lp = np.empty(m, np.float64) if pt is not None else None
    lse, ent = np.empty(m, np.float64), np.empty(m, np.float64)
    rc = _load().oracle_combine(k, m, _ptr(pm), _ptr(ps), _ptr(pw), _ptr(pt), _ptr(lp),
                                _ptr(lse), _ptr(ent))
    _check(rc, "oracle_combine")
    out = {"lse": lse, "entropy": ent}
    if lp is not None:
        out["logprob"] = lp
    return out


def bf16_rne(v) -> np.ndarray:
    """Round float64 values to bf16 (ties to even); returns uint16 bit patterns."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_bf16_rne_array(_ptr(v), _ptr(out), v.size)
    return out


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> int:
    """Run later oracle calls on n threads; returns the previous count."""
    prev = num_threads()
    _load().oracle_set_num_threads(int(n))
    return prev


def _lmhead_operands(hidden, weight, d):
    hidden = np.ascontiguousarray(hidden)
    weight = np.ascontiguousarray(weight)
    if hidden.dtype != np.uint16 or weight.dtype != np.uint16:
        raise TypeError("hidden and weight must be uint16 (bf16 bit patterns)")
    n_rows, ldh = hidden.shape
    vocab, ldw = weight.shape
    d = min(ldh, ldw) if d is None else d
    return hidden, weight, n_rows, ldh, vocab, ldw, d


def lmhead_logits(hidden, weight, d: int | None = None, rows=None, want_abs: bool = False):
    """float64 [m, vocab] logits x = hidden[rows, :d] @ weight[:, :d].T (and, with
    want_abs, the matching sums of |products|)."""
    hidden, weight, n_rows, ldh, vocab, ldw, d = _lmhead_operands(hidden, weight, d)
    rows, m = _rows_arg(rows, n_rows)
    x = np.empty((m, vocab), np.float64)
    a = np.empty((m, vocab), np.float64) if want_abs else None
    rc = _load().oracle_lmhead_logits(_ptr(hidden), n_rows, ldh, _ptr(weight), vocab, ldw, d,
                                      _ptr(rows), m, _ptr(x), _ptr(a))
    _check(rc, "oracle_lmhead_logits")
    return (x, a) if want_abs else x


def lmhead_forward(hidden, weight, targets, tau: float = 1.0, rows=None, d: int | None = None,
                   want=("logprob", "lse", "entropy"), row_chunk: int = 16,
                   err_scale: bool = False):
    """Per-row logprob / lse / entropy of the LM head over hidden[rows] in float64.

    hidden: uint16 [n_rows, ldh]; weight: uint16 [vocab, ldw]; the first d
    columns of each are the hidden dimension.  With err_scale, the dict also
    holds (A_t + max_j A_j) / tau per row (see oracle.h)."""
    hidden, weight, n_rows, ldh, vocab, ldw, d = _lmhead_operands(hidden, weight, d)
    rows, m = _rows_arg(rows, n_rows)
    targets = _targets_arg(targets)
    out = {k: (np.empty(m, np.float64) if k in want else None)
           for k in ("logprob", "lse", "entropy")}
    es = np.empty(m, np.float64) if err_scale else None
    rc = _load().oracle_lmhead_forward(_ptr(hidden), n_rows, ldh, _ptr(weight), vocab, ldw, d,
                                       _ptr(targets), _ptr(rows), m, _tau(tau), row_chunk,
                                       _ptr(out["logprob"]), _ptr(out["lse"]),
                                       _ptr(out["entropy"]), _ptr(es))
    _check(rc, "oracle_lmhead_forward")
    res = {k: v for k, v in out.items() if v is not None}
    if err_scale:
        res["err_scale"] = es
    return res
