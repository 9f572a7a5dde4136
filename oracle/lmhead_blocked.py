"""fp64 LM-head oracle for every kept row of a full-size call (TEST INFRASTRUCTURE).

Only the tests may import this module; the product path never does.  It shares no
code with the HIP path, nor with ``oracle.c``: it decodes the bf16 operands itself.

What it computes is the fused LM head's definition ("[Bug] Training/log-prob forward
materializes full-vocab fp32 logits ..." maintainer comment: project only the kept
rows; "[RL][Performance] Avoid full-vocabulary TP gather for selected-token
logprobs", "Proposed solution": the selected log-probability is the negative
token cross entropy): for a kept hidden row h and the weight W stored one row per
vocabulary entry, the logits x_j = sum_k h_k W_jk, then with z = x / tau

    lse = log sum_j exp(z_j),   logprob = z_t - lse,   entropy = lse - sum_j p_j z_j.

The one step taken from a library is the projection of a block of kept rows,
a float64 matrix product (numpy's BLAS), so that every one of thousands of rows can
be checked in about a minute; ``oracle.c`` sums each logit in a fixed order and is
far slower.  Everything else is the definition above, in float64, block by block.
The error-scale output (A_t + max_j A_j) / tau, with A_j = sum_k |h_k W_jk|, is
formed the same way from |h| and |W|.
"""
from __future__ import annotations

import numpy as np


def _decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (the 16 bits are the high half of a float32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def lmhead_forward_blocked(hidden, weight, targets, tau: float = 1.0, rows=None,
                           d: int | None = None, block: int = 256, err_scale: bool = False):
    """Per-kept-row logprob / lse / entropy (float64 [m]) of the LM head.

    hidden: uint16 [n_rows, ldh] and weight: uint16 [vocab, ldw] (bf16 bit patterns;
    the first d columns of each are the hidden dimension); targets: int [n_rows],
    indexed by row id; rows: the kept row ids (None: all rows), in output order.
    tau is taken as the C float the library receives, widened to double.  With
    err_scale the dict also holds (A_t + max_j A_j) / tau per row."""
    hidden = np.asarray(hidden)
    weight = np.asarray(weight)
    if hidden.dtype != np.uint16 or weight.dtype != np.uint16:
        raise TypeError("hidden and weight must be uint16 (bf16 bit patterns)")
    n_rows, ldh = hidden.shape
    vocab, ldw = weight.shape
    d = min(ldh, ldw) if d is None else int(d)
    if not 0 < d <= min(ldh, ldw):
        raise ValueError("need 0 < d <= ldh and d <= ldw")
    rows = np.arange(n_rows, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= n_rows):
        raise IndexError("row id outside the hidden rows")
    t = np.asarray(targets, np.int64)[rows]
    if t.size and (t.min() < 0 or t.max() >= vocab):
        raise IndexError("target outside the vocabulary")
    tau = float(np.float32(tau))
    w = _decode_bf16(weight[:, :d])
    wabs = np.abs(w) if err_scale else None
    m = rows.size
    out = {k: np.empty(m, np.float64) for k in ("logprob", "lse", "entropy")}
    if err_scale:
        out["err_scale"] = np.empty(m, np.float64)
    for b0 in range(0, m, block):
        sel = slice(b0, min(b0 + block, m))
        h = _decode_bf16(hidden[rows[sel], :d])
        z = (h @ w.T) / tau                        # the block's logits over tau
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        s = e.sum(axis=1)
        lse = zmax[:, 0] + np.log(s)
        at = np.arange(z.shape[0])
        out["lse"][sel] = lse
        out["logprob"][sel] = z[at, t[sel]] - lse
        out["entropy"][sel] = lse - (e * z).sum(axis=1) / s
        if err_scale:
            a = np.abs(h) @ wabs.T
            out["err_scale"][sel] = (a[at, t[sel]] + a.max(axis=1)) / tau
    return out
