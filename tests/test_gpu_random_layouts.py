"""A seeded sweep over random shapes and layouts against the fp64 oracle.

Each case draws a dtype, a vocabulary width on a log scale (64 to 300000, so
every segment count and both merge shapes appear), a row stride (often
padded), an element offset of the first row (rows off 16 bytes), a few rows
and a temperature.  Checked: the forward, the backward into a buffer of the
logits' layout and into a contiguous one (the two may take different paths),
a two-slice split of the vocabulary at a random column through the merge,
and a row set with a duplicate.  Bars as in the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import vocab_wide_cross_amd as vwc
import workloads as W
from gpu_util import (DEV, assert_bf16_grad, assert_close_scalar, grad_bits, like_layout,
                      place_rows)

pytestmark = pytest.mark.gpu


def _cases(count=48, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(count):
        dtype = "bf16" if rng.random() < 0.6 else "fp32"
        vocab = int(np.exp(rng.uniform(np.log(64), np.log(300000))))
        ld = vocab + int(rng.integers(1, 9)) if rng.random() < 0.5 else vocab
        off = int(rng.integers(0, 8 if dtype == "bf16" else 4))
        n = int(rng.integers(1, 7))
        tau = float(rng.choice([1.0, 0.7, 1.3]))
        cut = int(rng.integers(1, vocab))
        out.append((c, dtype, vocab, ld, off, n, tau, cut))
    return out


def _np(t):
    return t.detach().cpu().numpy()


def _check_grad(got, ref, what):
    if got.dtype == torch.bfloat16:
        assert_bf16_grad(grad_bits(got), ref, what, oracle)
    else:
        err = np.abs(_np(got).astype(np.float64) - ref).max()
        assert err <= 1e-6, f"{what}: fp32 gradient error {err:.3g}"


@pytest.mark.parametrize("case", _cases(),
                         ids=lambda c: f"{c[0]}-{c[1]}-V{c[2]}-ld{c[3]}-off{c[4]}-n{c[5]}")
def test_random_layout(case):
    c, dtype, vocab, ld, off, n, tau, cut = case
    name = "spiked_bf16_8192x248320" if dtype == "bf16" else "tiny_fp32_64x2048"
    w = W.scaled(name, n, vocab, seed=5000 + c, tau=tau)
    x = W.logits_rows(w, np.arange(n), ld=ld)
    t, g = W.targets(w), W.grad_out(w)
    _, xv = place_rows(x, off)
    xd = xv[:, :vocab]
    td, gd = torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)

    lp, lse, ent = vwc.selected_logprob_fwd(xd, td, w.tau, want=("logprob", "lse", "entropy"))
    ref = oracle.forward(x, t, tau=w.tau, vocab=vocab)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], k)

    gref = oracle.backward(x, t, g, tau=w.tau, vocab=vocab)
    gsame = like_layout(xv)[:, :vocab]
    vwc.selected_logprob_bwd(xd, td, lse, gd, w.tau, grad_logits=gsame)
    _check_grad(gsame, gref, "gradient in the logits' layout")
    gdense = vwc.selected_logprob_bwd(xd, td, lse, gd, w.tau)
    _check_grad(gdense, gref, "contiguous gradient")

    parts = torch.stack([vwc.vocab_partial(xd[:, :cut], 0, targets=td, temperature=w.tau),
                         vwc.vocab_partial(xd[:, cut:], cut, targets=td, temperature=w.tau)])
    slp, slse, sent = vwc.partial_combine(parts, w.tau)
    for k, v in (("logprob", slp), ("lse", slse), ("entropy", sent)):
        assert_close_scalar(_np(v), ref[k], f"split at {cut}: {k}")

    rows = np.array([n - 1, 0, n - 1], dtype=np.int32)
    rlp, rlse, _ = vwc.selected_logprob_fwd_rows(xd, td, torch.from_numpy(rows).to(DEV), w.tau)
    assert_close_scalar(_np(rlp), ref["logprob"][rows], "row set logprob")
    assert_close_scalar(_np(rlse), ref["lse"][rows], "row set lse")
