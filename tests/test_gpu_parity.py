"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small shapes cover every row (several row segments, ragged tails, the
rows that do not start on 16 bytes, edge cases).  Bars: logprob /
lse / entropy abs err <= 5e-5; fp32 gradient abs err <= 1e-6; bf16 gradient
within one bf16 step of the oracle rounded to bf16; the computed row set equal
to the oracle's, bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import vocab_wide_cross_amd as vwc
import workloads as W
from gpu_util import (DEV, assert_bf16_grad, assert_close_scalar, grad_bits, log,
                      to_dev_logits)

pytestmark = pytest.mark.gpu


def _host(w):
    return W.all_logits(w), W.targets(w), W.grad_out(w)


def _np(t):
    return t.cpu().numpy()


# ------------------------------------------------------------------ forward / backward, dense


@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_tiny_fp32_forward_backward(tau):
    w = W.get("tiny_fp32_64x2048")
    x, t, g = _host(w)
    log(f"tiny fp32 tau={tau}")
    xd, td, gd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd(xd, td, tau, want=("logprob", "lse", "entropy"))
    grad = vwc.selected_logprob_bwd(xd, td, lse, gd, tau)
    ref = oracle.forward(x, t, tau=tau)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], k)
    gref = oracle.backward(x, t, g, tau=tau)
    err = np.abs(_np(grad).astype(np.float64) - gref).max()
    assert err <= 1e-6, f"fp32 grad err {err}"


@pytest.mark.parametrize("vocab", [1, 7, 8, 9, 2048, 20011, 65537, 151936])
def test_bf16_forward_backward_shapes(vocab):
    """One segment (V <= 65536), several segments (65537: 2, 151936: 3), a ragged
    tail after the last 16-byte vector, and rows shorter than one vector."""
    n = 40 if vocab > 60000 else 96
    w = W.scaled("spiked_bf16_8192x248320", n, vocab)
    x, t, g = _host(w)
    log(f"bf16 [{n}, {vocab}]")
    xd, td, gd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    grad = vwc.selected_logprob_bwd(xd, td, lse, gd)
    ref = oracle.forward(x, t)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], f"{k} V={vocab}")
    gref = oracle.backward(x, t, g)
    if vocab == 1:
        # The exact gradient is 0 and lse = x / tau.  The forward folds the one
        # term as 2^r with r = x c - fl(x c), the rounding residual of its shift,
        # through the hardware's approximate exp2 (about 1 ulp), and undoes r in
        # fp64; so the sum is 1 + e with |e| <= about 2^-22 and the saved lse may
        # sit up to 2|e| from x / tau.  The backward's -expm1(x/tau - lse) turns
        # that into |grad| <= |g| / tau * 2^-21, give or take the exp2's last
        # bit, which is why the check allows twice that.
        gg = _np(grad.float())[:, 0].astype(np.float64)
        assert np.all(np.abs(gg) <= np.abs(g) * 2.0 ** -20)
    else:
        assert_bf16_grad(grad_bits(grad), gref, f"grad V={vocab}", oracle)
    zero = g == 0.0
    gb = grad_bits(grad)
    assert np.all(gb[zero] == 0), "rows with zero grad_out must be +0.0"


@pytest.mark.parametrize("dtype,vocab", [("bf16", 1048579), ("bf16", 2097155), ("fp32", 4194311)])
def test_very_wide_rows(dtype, vocab):
    """Rows far wider than any vocabulary on the pages, with a ragged tail: 17 or 33
    bf16 (2 or 4 MiB rows) or 129 fp32 (16 MiB rows) forward segments of at most
    128 KiB, merged by the combine kernel; the backward in 33, 65 or 257 pieces of
    at most 64 KiB.  At 2097155 bf16 columns the 1 KiB rounding of the segment
    boundaries leaves the backward's last piece with no whole vector, only the
    row's three tail elements.  The one call runs the two calls (the rows do not
    fit on chip) with their bits."""
    n = 3
    base = "spiked_bf16_8192x248320" if dtype == "bf16" else "tiny_fp32_64x2048"
    w = W.scaled(base, n, vocab)
    x, t, g = _host(w)
    log(f"{dtype} [{n}, {vocab}]")
    xd, td, gd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    grad = vwc.selected_logprob_bwd(xd, td, lse, gd)
    ref = oracle.forward(x, t)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], f"{k} V={vocab}")
    gref = oracle.backward(x, t, g)
    if dtype == "bf16":
        assert_bf16_grad(grad_bits(grad), gref, f"grad V={vocab}", oracle)
    else:
        err = np.abs(_np(grad).astype(np.float64) - gref).max()
        assert err <= 1e-6, f"fp32 grad err {err}"
    olp, olse, _, ograd = vwc.selected_logprob_fwd_bwd(xd, td, gd)
    assert torch.equal(olp, lp) and torch.equal(olse, lse)
    bits = (lambda a: a.view(torch.int16)) if dtype == "bf16" else (lambda a: a.view(torch.int32))
    assert torch.equal(bits(ograd), bits(grad))


def test_confident_target_gradient_limited_by_saved_lse():
    """Rows whose target holds nearly all the mass (1 - p_t down to 1e-9).  The
    target column g/tau (1 - p_t) is computed from the saved fp32 lse, so its
    error is bounded by |g|/tau times lse's rounding; every other column stays
    within one bf16 step of the oracle."""
    V, n = 4096, 32
    rng = np.random.default_rng(11)
    x = rng.standard_normal((n, V)).astype(np.float32)
    t = rng.integers(0, V, n).astype(np.int32)
    x[np.arange(n), t] = np.linspace(8.0, 30.0, n).astype(np.float32)
    g = rng.uniform(-1, 1, n).astype(np.float32)
    xd, td, gd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    for tau in (1.0, 0.7):
        _, lse, _ = vwc.selected_logprob_fwd(xd, td, tau)
        g32 = _np(vwc.selected_logprob_bwd(xd, td, lse, gd, tau, grad_dtype=torch.float32))
        gref = oracle.backward(x, t, g, tau=tau)
        ref_lse = oracle.forward(x, t, tau=tau)["lse"]
        tau32 = float(np.float32(tau))
        bound = np.abs(g) / tau32 * (2 * np.spacing(np.abs(ref_lse).astype(np.float32)) + 2.0 ** -22)
        err_t = np.abs(g32[np.arange(n), t] - gref[np.arange(n), t])
        assert np.all(err_t <= bound), (err_t / bound).max()
        other = np.ones_like(g32, bool)
        other[np.arange(n), t] = False
        assert np.abs(g32[other] - gref[other]).max() <= 1e-6


def test_fp32_grad_from_bf16_and_bf16_grad_from_fp32():
    w = W.scaled("spiked_bf16_8192x248320", 32, 5003)
    x, t, g = _host(w)
    xd, td, gd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    _, lse, _ = vwc.selected_logprob_fwd(xd, td)
    g32 = vwc.selected_logprob_bwd(xd, td, lse, gd, grad_dtype=torch.float32)
    gref = oracle.backward(x, t, g)
    # lse is an fp32 input here, so p carries its rounding: 1e-6 absolute still holds
    assert np.abs(_np(g32).astype(np.float64) - gref).max() <= 1e-6
    wf = W.scaled("tiny_fp32_64x2048", 32, 5003)
    xf, tf, gf = _host(wf)
    xfd, tfd, gfd = to_dev_logits(xf), torch.from_numpy(tf).to(DEV), torch.from_numpy(gf).to(DEV)
    _, lsef, _ = vwc.selected_logprob_fwd(xfd, tfd)
    gb = vwc.selected_logprob_bwd(xfd, tfd, lsef, gfd, grad_dtype=torch.bfloat16)
    assert_bf16_grad(grad_bits(gb), oracle.backward(xf, tf, gf), "fp32->bf16 grad", oracle)


@pytest.mark.parametrize("vocab,ld", [(20011, 20011), (20011, 20013), (4096, 4100), (70001, 70003)])
def test_unaligned_rows_odd_stride(vocab, ld):
    """Rows that do not start on 16 bytes (odd ld): the forward streams vectors from
    each row's first 16-byte boundary; the backward, whose gradient rows here have
    another stride (another phase), goes element by element."""
    w = W.scaled("spiked_bf16_8192x248320", 24, vocab)
    x = W.logits_rows(w, np.arange(w.n_rows), ld=ld)
    t, g = W.targets(w), W.grad_out(w)
    xd = to_dev_logits(x)[:, :vocab]
    td, gd = torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    grad = torch.zeros((w.n_rows, ld + 1), dtype=torch.bfloat16, device=DEV)[:, :vocab]
    vwc.selected_logprob_bwd(xd, td, lse, gd, grad_logits=grad)
    ref = oracle.forward(x, t, vocab=vocab)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], k)
    gref = oracle.backward(x, t, g, vocab=vocab)
    assert_bf16_grad(grad_bits(grad), gref, "unaligned grad", oracle)


# ------------------------------------------------------------------ row sets


def test_mask_to_index_matches_nonzero():
    rng = np.random.default_rng(7)
    for n in (0, 1, 5, 16383, 16384, 16385, 32768, 100003):
        for p in (0.0, 0.25, 0.5, 1.0):
            mask = (rng.random(n) < p).astype(np.uint8)
            if n > 3 and p == 0.5:
                mask[rng.integers(0, n, 3)] = 7  # any nonzero byte counts
            md = torch.from_numpy(mask).to(DEV)
            idx, cnt = vwc.mask_to_index(md)
            c = int(cnt.item())
            want = np.flatnonzero(mask).astype(np.int32)
            assert c == want.size
            assert np.array_equal(_np(idx[:c]), want)
    # a mask that does not start on 16 bytes takes the byte-by-byte path
    mask = (rng.random(40001) < 0.3).astype(np.uint8)
    md = torch.from_numpy(mask).to(DEV)[1:]
    idx, cnt = vwc.mask_to_index(md)
    c = int(cnt.item())
    assert np.array_equal(_np(idx[:c]), np.flatnonzero(mask[1:]).astype(np.int32))
    # packed workload mask: the response spans
    w = W.get("packed_bf16_32768x248320")
    m = W.loss_mask(w)
    idx, cnt = vwc.mask_to_index(torch.from_numpy(m).to(DEV))
    c = int(cnt.item())
    assert c == 8192 and np.array_equal(_np(idx[:c]), W.row_index(w))


@pytest.mark.parametrize("n", [65537, 160000, 160003, 1 << 20, 1000003])
def test_long_mask_to_index_tiled_and_one_group(n):
    """Long masks (packed and context-parallel sequences): the tiled scan over the
    whole GPU and the one-workgroup scan both give numpy's nonzero, bit for bit,
    for sparse, dense, full and empty masks and a mask that starts off 16 bytes."""
    rng = np.random.default_rng(n)
    for p in (0.0, 0.01, 0.5, 1.0):
        mask = (rng.random(n + 1) < p).astype(np.uint8)
        mask[rng.integers(0, n, 3)] = 9 if p > 0 else 0
        want = np.flatnonzero(mask[:n]).astype(np.int32)
        md = torch.from_numpy(mask).to(DEV)
        for view in (md[:n], md[1:]):  # the second starts off 16 bytes
            w = want if view.data_ptr() == md.data_ptr() else \
                np.flatnonzero(mask[1:]).astype(np.int32)
            for one_group in (False, True):
                idx, cnt = vwc.mask_to_index(view, one_group=one_group)
                c = int(cnt.item())
                assert c == w.size, (p, one_group, c, w.size)
                assert np.array_equal(_np(idx[:c]), w), (p, one_group)
    log(f"mask_to_index n={n}: tiled and one-group scans equal nonzero()")


def test_long_mask_to_index_graph_replays():
    """The tiled scan (three launches and a workspace) captured once and replayed
    on new masks gives the eager ids every time."""
    n = 1 << 20
    mask = torch.zeros(n, dtype=torch.uint8, device=DEV)
    idx = torch.empty(n, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(vwc.mask_to_index_workspace_bytes(n), dtype=torch.uint8, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(9)
    mask.copy_((torch.rand(n, device=DEV, generator=gen) < 0.3).to(torch.uint8))
    vwc.mask_to_index(mask, idx, cnt, workspace=ws)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vwc.mask_to_index(mask, idx, cnt, workspace=ws)
    for rep in range(3):
        mask.copy_((torch.rand(n, device=DEV, generator=gen) < 0.1 + 0.3 * rep).to(torch.uint8))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = np.flatnonzero(_np(mask)).astype(np.int32)
        c = int(cnt.item())
        assert c == want.size and np.array_equal(_np(idx[:c]), want), rep


def test_compact_rows_forward_and_entropy():
    w = W.scaled("masked_bf16_4096x151936", 160, 151936)
    x, t, _ = _host(w)
    idx = W.row_index(w)
    log(f"compact rows: {idx.size} of {w.n_rows}")
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    idd = torch.from_numpy(idx).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd_rows(xd, td, idd, want=("logprob", "lse", "entropy"))
    ref = oracle.forward(x, t, rows=idx)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], k)
    # compact == dense at those rows, bit for bit
    dlp, dlse, dent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    for a, b in ((lp, dlp), (lse, dlse), (ent, dent)):
        assert torch.equal(a, b[idd])
    ent2 = vwc.entropy_rows(xd, idd)
    assert torch.equal(ent2, ent)
    assert torch.equal(vwc.entropy(xd), dent)


def test_compact_backward_compact_and_scatter():
    w = W.scaled("packed_bf16_32768x248320", 256, 30011)
    x, t, g = _host(w)
    idx = W.row_index(w)
    assert idx.size == 8 * w.response_len
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    idd = torch.from_numpy(idx).to(DEV)
    gc = torch.from_numpy(g[idx]).to(DEV)
    lp, lse, _ = vwc.selected_logprob_fwd_rows(xd, td, idd)
    comp = vwc.selected_logprob_bwd_rows(xd, td, idd, lse, gc, layout=vwc.VWC_GRAD_COMPACT)
    scat = torch.full((w.n_rows, w.vocab), 3.0, dtype=torch.bfloat16, device=DEV)
    vwc.selected_logprob_bwd_rows(xd, td, idd, lse, gc, grad_logits=scat,
                                  layout=vwc.VWC_GRAD_SCATTER)
    gref = oracle.backward(x, t, g[idx], rows=idx)
    assert_bf16_grad(grad_bits(comp), gref, "compact grad", oracle)
    assert torch.equal(scat[idd], comp)
    others = np.setdiff1d(np.arange(w.n_rows), idx)
    assert torch.all(scat[torch.from_numpy(others).to(DEV)] == 3.0), "scatter touched other rows"
    # dense backward restricted to the rows equals the compact one bit for bit
    gd_full = np.zeros(w.n_rows, np.float32)
    gd_full[idx] = g[idx]
    _, dlse, _ = vwc.selected_logprob_fwd(xd, td)
    dense = vwc.selected_logprob_bwd(xd, td, dlse, torch.from_numpy(gd_full).to(DEV))
    assert torch.equal(dense[idd], comp)
    assert torch.all(dense[torch.from_numpy(others).to(DEV)].view(torch.int16) == 0)


def test_empty_row_sets_are_noops():
    x = torch.randn(4, 64, device=DEV).to(torch.bfloat16)
    t = torch.zeros(4, dtype=torch.int32, device=DEV)
    e = torch.empty(0, dtype=torch.int32, device=DEV)
    lp, lse, _ = vwc.selected_logprob_fwd_rows(x, t, e)
    assert lp.numel() == 0 and lse.numel() == 0
    g = vwc.selected_logprob_bwd_rows(x, t, e, lse, lp)
    assert g.shape == (0, 64)
    z = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    lp0, _, _ = vwc.selected_logprob_fwd(z, torch.empty(0, dtype=torch.int32, device=DEV))
    assert lp0.numel() == 0


@pytest.mark.parametrize("vocab", [70001, 248320])
def test_row_chunks_are_bitwise_identical(vocab):
    """Covering the rows in chunks of 1 / 7 / 64 / 4096 gives the same bits, through
    row lists and through dense calls on row slices, forward and backward (rows of
    2 segments merged in-block, and of 4 merged by a second launch)."""
    w = W.scaled("spiked_bf16_8192x248320", 200, vocab)
    x, t, g = _host(w)
    xd, td, gd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    full, flse, fent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    fgrad = vwc.selected_logprob_bwd(xd, td, flse, gd)
    for chunk in (1, 7, 64, 4096):
        parts, ents, dense = [], [], []
        for r0 in range(0, w.n_rows, chunk):
            r1 = min(r0 + chunk, w.n_rows)
            rows = torch.arange(r0, r1, dtype=torch.int32, device=DEV)
            lp, _, en = vwc.selected_logprob_fwd_rows(xd, td, rows, want=("logprob", "entropy"))
            parts.append(lp)
            ents.append(en)
            dlp, dlse, _ = vwc.selected_logprob_fwd(xd[r0:r1], td[r0:r1])
            dense.append(dlp)
            if chunk == 64:
                gr = vwc.selected_logprob_bwd(xd[r0:r1], td[r0:r1], dlse, gd[r0:r1])
                assert torch.equal(gr.view(torch.int16), fgrad[r0:r1].view(torch.int16))
        assert torch.equal(torch.cat(parts), full) and torch.equal(torch.cat(ents), fent)
        assert torch.equal(torch.cat(dense), full)


def test_run_to_run_deterministic():
    w = W.scaled("spiked_bf16_8192x248320", 64, 151936)
    x, t, g = _host(w)
    xd, td, gd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    a = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    b = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    ga = vwc.selected_logprob_bwd(xd, td, a[1], gd)
    gb = vwc.selected_logprob_bwd(xd, td, a[1], gd)
    assert torch.equal(ga.view(torch.int16), gb.view(torch.int16))


def test_concurrent_streams_give_sequential_bits():
    """The library holds no state between calls: forward, backward and the one call
    issued on two streams at once, on different inputs (4-segment rows that use
    the workspace), give the bits of the same calls made one after another."""
    outs = []
    cases = []
    for seed, n in ((1, 96), (2, 80)):
        w = W.scaled("spiked_bf16_8192x248320", n, 248320 + seed)
        x, t, g = _host(w)
        cases.append((to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)))

    def work(xd, td, gd, stream):
        lp, lse, ent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"),
                                                stream=stream)
        grad = vwc.selected_logprob_bwd(xd, td, lse, gd, stream=stream)
        one = vwc.selected_logprob_fwd_bwd(xd, td, gd, stream=stream)
        return (lp, lse, ent, grad, one[0], one[1], one[3])

    seq = [work(*c, torch.cuda.current_stream()) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for c, st in zip(cases, streams):
            with torch.cuda.stream(st):
                outs.append(work(*c, st))
    torch.cuda.synchronize()
    for k, o in enumerate(outs):
        ref = seq[k % 2]
        for a, b in zip(o, ref):
            va = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
            vb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
            assert torch.equal(va, vb)


# ------------------------------------------------------------------ split vocabulary


def _split(xd, td, tau, v_local, k, rows=None):
    parts = []
    for q in range(k):
        sl = xd[:, q * v_local:(q + 1) * v_local]
        parts.append(vwc.vocab_partial(sl, q * v_local, td, rows, tau))
    return torch.stack(parts)


def test_split_vocab_matches_single_pass_and_oracle():
    w = W.scaled("extreme_fp32_16384x248320", 48, 4 * 6208)
    x, t, _ = _host(w)
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    parts = _split(xd, td, w.tau, 6208, 4)
    lp, lse, ent = vwc.partial_combine(parts, w.tau)
    slp, slse, sent = vwc.selected_logprob_fwd(xd, td, w.tau, want=("logprob", "lse", "entropy"))
    ref = oracle.forward(x, t, tau=w.tau)
    for k, v, s in (("logprob", lp, slp), ("lse", lse, slse), ("entropy", ent, sent)):
        ulps = 0 if k == "entropy" else 4
        assert_close_scalar(_np(v), ref[k], f"split {k}", ulps=ulps)
        assert_close_scalar(_np(s), ref[k], f"single {k}", ulps=ulps)
    # each slice partial against the oracle's slice partial (reference-free form)
    for q in range(4):
        pm, ps, pw, pt = oracle.slice_partial(x, q * 6208, 6208, t, w.tau)
        got = _np(parts[q]).astype(np.float64)
        tau = float(np.float32(w.tau))
        assert_close_scalar(got[:, 0] / tau + np.log(got[:, 1]), pm + np.log(ps), "slice lse",
                            ulps=4)
        assert_close_scalar(np.log(got[:, 1]) - got[:, 3] / got[:, 1], np.log(ps) - pw / ps,
                            "slice entropy")
        own = np.isfinite(pt)
        assert np.array_equal(np.isfinite(got[:, 2]), own)
        assert np.array_equal(got[own, 2] / tau, pt[own])


def test_split_vocab_rows_and_unowned_targets():
    w = W.scaled("extreme_fp32_16384x248320", 40, 3 * 2000)
    x, t, _ = _host(w)
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    rows = torch.tensor([3, 0, 39, 17], dtype=torch.int32, device=DEV)
    parts = _split(xd, td, 1.0, 2000, 3, rows)
    lp, lse, ent = vwc.partial_combine(parts, 1.0)
    ref = oracle.forward(x, t, rows=_np(rows))
    assert_close_scalar(_np(lp), ref["logprob"], "rows split lp", ulps=4)
    # only two of three slices: targets in the third are owned by none -> -inf
    lp2, _, _ = vwc.partial_combine(parts[:2].contiguous(), 1.0)
    own = _np(td[rows.long()]) < 4000
    assert np.all(np.isneginf(_np(lp2)[~own])) and np.all(np.isfinite(_np(lp2)[own]))


# ------------------------------------------------------------------ edge values


@pytest.mark.parametrize("vocab", [1000, 100000, 151936, 248320])
def test_out_of_range_targets_and_rows_give_nan(vocab):
    """One segment, two and three (merged inside the row's workgroup), four (a
    workgroup per segment and a merge launch)."""
    w = W.scaled("spiked_bf16_8192x248320", 8, vocab)
    x, t, _ = _host(w)
    t[2], t[5] = -1, vocab
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    lp, lse, _ = vwc.selected_logprob_fwd(xd, td)
    lpn = _np(lp)
    assert np.isnan(lpn[2]) and np.isnan(lpn[5])
    ok = np.ones(8, bool)
    ok[[2, 5]] = False
    ref = oracle.forward(x[ok], t[ok])
    assert_close_scalar(lpn[ok], ref["logprob"], "lp")
    assert np.all(np.isfinite(_np(lse)))
    rows = torch.tensor([0, 8, -3, 1], dtype=torch.int32, device=DEV)
    t[2], t[5] = 0, 0
    td = torch.from_numpy(t).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd_rows(xd, td, rows, want=("logprob", "lse", "entropy"))
    for v in (lp, lse, ent):
        a = _np(v)
        assert np.isnan(a[1]) and np.isnan(a[2]) and np.isfinite(a[0]) and np.isfinite(a[3])
    ref = oracle.forward(x, t, rows=np.array([0, 1]))
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v)[[0, 3]], ref[k], k)
    part = _np(vwc.vocab_partial(xd, 0, td, rows))
    assert np.isnan(part[[1, 2]][:, 1:]).all() and np.isfinite(part[[0, 3]]).all()


def test_masked_minus_inf_logits():
    """-inf logits (masked vocabulary entries) carry zero probability: finite
    logprob, lse, entropy and gradient."""
    w = W.scaled("tiny_fp32_64x2048", 16, 3001)
    x, t, g = _host(w)
    rng = np.random.default_rng(3)
    mask = rng.random(x.shape) < 0.3
    mask[np.arange(16), t] = False
    mask[:, :300] = True            # whole leading chunks of -inf
    mask[np.arange(16), t] = False
    x = x.copy()
    x[mask] = -np.inf
    xd, td, gd = to_dev_logits(x), torch.from_numpy(t).to(DEV), torch.from_numpy(g).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    grad = vwc.selected_logprob_bwd(xd, td, lse, gd)
    ref = oracle.forward(x, t)
    for k, v in (("logprob", lp), ("lse", lse), ("entropy", ent)):
        assert_close_scalar(_np(v), ref[k], k)
    gref = oracle.backward(x, t, g)
    assert np.abs(_np(grad).astype(np.float64) - gref).max() <= 1e-6
    # the entropy gradient: exactly 0 at the -inf columns (0 log 0 = 0)
    h = np.random.default_rng(4).uniform(-1, 1, 16).astype(np.float32)
    both = _np(vwc.logprob_entropy_bwd(xd, td, lse, ent, gd, torch.from_numpy(h).to(DEV)))
    assert np.all(both[mask] == 0.0) and np.all(np.isfinite(both))
    eref = oracle.backward_entropy(x, t, g, h)
    assert np.abs(both.astype(np.float64) - eref).max() <= 1e-6
    # split vocabulary: the slice [0, 300) is -inf (but for a target there) and
    # adds nothing
    cuts = [0, 300, 1700, 3001]
    parts = torch.stack([vwc.vocab_partial(xd[:, a:b], a, td, None) for a, b in
                         zip(cuts[:-1], cuts[1:])])
    empty = t >= 300
    assert empty.any() and np.all(_np(parts[0])[empty, 1] == 0.0)
    lp2, lse2, ent2 = vwc.partial_combine(parts, 1.0, want=("logprob", "lse", "entropy"))
    for k, v in (("logprob", lp2), ("lse", lse2), ("entropy", ent2)):
        assert_close_scalar(_np(v), ref[k], f"split {k}")


def test_nan_logit_poisons_only_its_row():
    w = W.scaled("spiked_bf16_8192x248320", 6, 5000)
    x, t, _ = _host(w)
    x = x.copy()
    x[4, 1234] = 0x7FC0  # bf16 NaN
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    for v in (lp, lse, ent):
        a = _np(v)
        assert np.isnan(a[4]) and np.all(np.isfinite(np.delete(a, 4)))


def test_dominant_logit_and_uniform_rows():
    V = 151936
    x = np.zeros((3, V), np.float32)
    x[1, 777] = 1000.0
    x[2] = -5.5
    t = np.array([5, 777, 9], np.int32)
    xd, td = to_dev_logits(x), torch.from_numpy(t).to(DEV)
    lp, lse, ent = vwc.selected_logprob_fwd(xd, td, want=("logprob", "lse", "entropy"))
    assert abs(_np(lp)[0] + math.log(V)) < 5e-5 and abs(_np(ent)[0] - math.log(V)) < 5e-5
    assert abs(_np(lp)[1]) < 5e-5 and abs(_np(ent)[1]) < 5e-5
    assert abs(_np(lp)[2] + math.log(V)) < 5e-5
