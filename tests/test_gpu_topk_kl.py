"""GPU parity of the truncated and tail-aware top-k KL against the fp64 oracle.

Forward outputs (loss, student/teacher top-k mass, raw top-k sum): abs err <= 5e-5.
Gradients: fp32 within 1e-6; bf16 within one bf16 step of the rounded oracle, or,
where a coefficient cancels (q_j - p_j inside the payload, alpha = P - p_tail Q /
(1 - Q) outside), within the error that the forward's fp32 lse, P and Q carry
into it (first-order bound from their measured deviations) plus one spacing.
"""
import numpy as np
import pytest
import torch

import oracle
import vocab_wide_cross_amd as vwc
import workloads as W
from gpu_util import DEV, assert_close_scalar, grad_bits, log, to_dev_logits, upload_workload
from helpers import bf16_ulp_distance

pytestmark = pytest.mark.gpu

MODES = [vwc.VWC_KL_TRUNCATED, vwc.VWC_KL_TAIL]


def _np(t):
    return t.cpu().numpy()


def _dev(w, x, idx, tlp):
    return to_dev_logits(x), torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV)


def check_fwd(fwd, x, idx, tlp, mode, tau, eps=1e-6):
    ref = oracle.topk_kl_forward(x, idx, tlp, mode, tail_eps=eps, tau=tau)
    assert_close_scalar(_np(fwd["loss"]), ref["loss"], "loss")
    assert_close_scalar(_np(fwd["student_mass"]), ref["student_mass"], "student_mass")
    assert_close_scalar(_np(fwd["teacher_mass"]), ref["teacher_mass"], "teacher_mass")
    return ref


def grad_bound(x, idx, tlp, mode, tau, fwd, ref_fwd, g, eps=1e-6):
    """Per-element allowance from the forward's fp32 deviations (first order)."""
    tau32 = float(np.float32(tau))
    o = oracle.forward(x, None, tau=tau, want=("lse",))
    xf = (W.bf16_bits_to_float32(x) if x.dtype == np.uint16 else x).astype(np.float64)
    q = np.exp(xf / tau32 - o["lse"][:, None])
    dl = np.abs(_np(fwd["lse"]).astype(np.float64) - o["lse"])
    P, Q = ref_fwd["teacher_mass"], ref_fwd["student_mass"]
    dP = np.abs(_np(fwd["teacher_mass"]).astype(np.float64) - P)
    dQ = np.abs(_np(fwd["student_mass"]).astype(np.float64) - Q)
    pt = np.maximum(0.0, 1.0 - P)
    if mode == vwc.VWC_KL_TAIL:
        qt = np.maximum(1.0 - Q, eps)
        d_alpha = (dP + pt * dQ / qt) / qt
        alpha = P - pt * Q / qt
    else:
        d_alpha = dP
        alpha = P
    e = (d_alpha + (np.abs(alpha) + 2) * dl + 1e-6)[:, None] + np.zeros_like(q)
    return np.abs(g / tau32)[:, None] * q * 2 * e


def check_bf16_grad(got_bits, ref, bound):
    steps = bf16_ulp_distance(got_bits, oracle.bf16_rne(ref))
    got = W.bf16_bits_to_float32(got_bits).astype(np.float64)
    ok = (steps <= 1) | (np.abs(got - ref) <= bound + np.abs(ref) * 2.0 ** -7 + 2.0 ** -133)
    assert ok.all(), f"{(~ok).sum()} elements beyond the bar"
    return int((steps > 1).sum())


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_topk_kl_fp32_tiny(mode, tau):
    """The verl PR's small test shape: b=2, s=96 (192 rows), V=2048, K=32, fp32."""
    w = W.get("distill_fp32_192x2048_k32")
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    g = np.random.default_rng(1).uniform(-1, 1, w.n_rows).astype(np.float32)
    xd, idd, tld = _dev(w, x, idx, tlp)
    fwd = vwc.topk_kl_fwd(xd, idd, tld, mode, temperature=tau)
    check_fwd(fwd, x, idx, tlp, mode, tau)
    grad = vwc.topk_kl_bwd(xd, idd, tld, fwd, torch.from_numpy(g).to(DEV), mode, temperature=tau)
    ref = oracle.topk_kl_backward(x, idx, tlp, mode, g, tau=tau)
    assert np.abs(_np(grad).astype(np.float64) - ref).max() <= 1e-6


@pytest.mark.parametrize("mode", MODES)
def test_topk_kl_bf16_multi_segment(mode):
    w = W.scaled("distill_bf16_4096x248320_k128", 24, 151936)
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    g = np.random.default_rng(2).uniform(-1, 1, w.n_rows).astype(np.float32)
    g[3] = 0.0
    xd, idd, tld = _dev(w, x, idx, tlp)
    fwd = vwc.topk_kl_fwd(xd, idd, tld, mode)
    ref_fwd = check_fwd(fwd, x, idx, tlp, mode, 1.0)
    grad = vwc.topk_kl_bwd(xd, idd, tld, fwd, torch.from_numpy(g).to(DEV), mode)
    ref = oracle.topk_kl_backward(x, idx, tlp, mode, g)
    n = check_bf16_grad(grad_bits(grad), ref, grad_bound(x, idx, tlp, mode, 1.0, fwd, ref_fwd, g))
    log(f"top-k KL bf16 mode={mode}: {n} elements beyond one bf16 step (within the bar)")
    assert np.all(grad_bits(grad)[3] == 0)


def test_topk_kl_clamp_guard_and_bad_index():
    """Q > P clamps the truncated loss (row gradient +0.0); 1 - Q < eps turns off
    the tail term's gradient; an out-of-range payload column gives NaN."""
    V, K = 4096, 8
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, V)).astype(np.float32)
    idx = np.stack([rng.choice(V, K, replace=False) for _ in range(4)]).astype(np.int32)
    tlp = np.log(np.full((4, K), 0.5 / K)).astype(np.float32)
    x[0, idx[0]] = 12.0      # Q ~ 1 - 1e-3 > P: truncated clamp
    x[1, idx[1]] = 40.0      # 1 - Q < eps: guard active
    g = np.ones(4, np.float32)
    xd, idd, tld = to_dev_logits(x), torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV)
    gd = torch.from_numpy(g).to(DEV)
    for mode in MODES:
        fwd = vwc.topk_kl_fwd(xd, idd, tld, mode)
        check_fwd(fwd, x, idx, tlp, mode, 1.0)
        grad = vwc.topk_kl_bwd(xd, idd, tld, fwd, gd, mode)
        ref = oracle.topk_kl_backward(x, idx, tlp, mode, g)
        assert np.abs(_np(grad).astype(np.float64) - ref).max() <= 1e-6
        if mode == vwc.VWC_KL_TRUNCATED:
            assert _np(fwd["loss"])[0] == 0.0
            gz = _np(grad[0]).view(np.uint32)
            assert np.all(gz == 0)
    bad = idx.copy()
    bad[2, 3] = V
    fwd = vwc.topk_kl_fwd(xd, torch.from_numpy(bad).to(DEV), tld, vwc.VWC_KL_TAIL)
    loss = _np(fwd["loss"])
    assert np.isnan(loss[2]) and np.all(np.isfinite(np.delete(loss, 2)))


def check_all_rows(fwd, grad, xh, idx, tlp, mode, tau, g, what, block=128):
    """Every row's forward outputs and bf16 gradient against the oracle, in blocks
    of rows (the oracle's gradient of a block is [block, V] fp64).  Returns the
    number of elements beyond one bf16 step (all within the bar)."""
    n_beyond = 0
    for r0 in range(0, xh.shape[0], block):
        rows = np.arange(r0, min(r0 + block, xh.shape[0]))
        ri = torch.from_numpy(rows).to(DEV)
        sub = {k: v[ri] for k, v in fwd.items()}
        ref_fwd = check_fwd(sub, xh[rows], idx[rows], tlp[rows], mode, tau)
        ref = oracle.topk_kl_backward(xh[rows], idx[rows], tlp[rows], mode, g[rows], tau=tau)
        n_beyond += check_bf16_grad(grad_bits(grad[ri]), ref,
                                    grad_bound(xh[rows], idx[rows], tlp[rows], mode, tau, sub,
                                               ref_fwd, g[rows]))
    log(f"{what} mode={mode}: all {xh.shape[0]} rows checked, {n_beyond} elements beyond one "
        f"bf16 step (within the bar)")
    return n_beyond


@pytest.mark.timeout(900)
def test_topk_kl_full_size_k128():
    """The page's distillation dimensions: N=4096, V=248320 bf16, K=128; every row
    against the oracle, for both objectives."""
    w = W.get("distill_bf16_4096x248320_k128")
    x, xh = upload_workload(w, keep_rows=True)
    idx, tlp = W.topk_payload(w)
    g = np.random.default_rng(5).uniform(-1, 1, w.n_rows).astype(np.float32)
    idd, tld, gd = (torch.from_numpy(a).to(DEV) for a in (idx, tlp, g))
    for mode in MODES:
        fwd = vwc.topk_kl_fwd(x, idd, tld, mode)
        grad = vwc.topk_kl_bwd(x, idd, tld, fwd, gd, mode)
        torch.cuda.synchronize()
        check_all_rows(fwd, grad, xh, idx, tlp, mode, 1.0, g, "top-k KL full size")
        assert torch.all(torch.isfinite(fwd["loss"]))
        if mode == vwc.VWC_KL_TAIL:
            assert torch.all(fwd["loss"] >= -5e-5)
        del grad
    del x
    torch.cuda.empty_cache()


def _bf16_round(a):
    """float32 -> bf16 bits (round to nearest even) for building test logits."""
    return oracle.bf16_rne(a.astype(np.float64))


def _payload_columns(V, N, seg_col, k, rng):
    """Columns that land on unit and segment edges: the first unit, a whole unit,
    both sides of the first segment boundary, the last whole unit and the tail
    past it; then distinct random columns up to k."""
    tail0 = (V // N) * N
    edge = [0, 1, N - 1, seg_col - 1, seg_col, seg_col + 1, tail0 - 1, V - 1, V - 2]
    edge += list(range(4 * N, 5 * N))  # one whole unit
    cols = list(dict.fromkeys(c for c in edge if 0 <= c < V))
    rest = rng.permutation(np.setdiff1d(np.arange(V), cols))[: k - len(cols)]
    return np.concatenate([cols, rest]).astype(np.int32)[:k]


# (logits dtype, grad dtype, vocab, k, ld padding): the fused pass (rows on 16
# bytes, k <= 256) with payload columns in the tail, on segment edges and filling
# a unit, for each dtype pair; and the two cases that keep the separate payload
# launch (k above the fused table's 256, rows not on 16 bytes).  The row stride
# is the vocabulary rounded up to 8 (plus the padding); the columns past the
# vocabulary hold NaN, in the logits and in the gradient buffer.
LAYOUTS = [
    ("bf16", "bf16", 151939, 64, 0),
    ("bf16", "fp32", 151939, 40, 0),
    ("fp32", "fp32", 70001, 32, 0),
    ("fp32", "bf16", 70001, 32, 0),
    ("bf16", "bf16", 151939, 300, 0),
    ("bf16", "bf16", 151939, 64, 1),
]


@pytest.mark.parametrize("layout", LAYOUTS, ids=[f"{a}-{b}-V{c}-k{d}-pad{e}" for a, b, c, d, e in LAYOUTS])
@pytest.mark.parametrize("mode", MODES)
def test_topk_kl_payload_layouts(layout, mode):
    dt, gdt, V, K, pad = layout
    n = 6
    N = 8 if dt == "bf16" else 4
    e = 2 if dt == "bf16" else 4
    ld = (V + 7) // 8 * 8 + pad
    nseg = -(-(V * e) // (256 * 1024))
    seg_col = -(-(V // N) // nseg) * N  # first column of segment 1
    rng = np.random.default_rng(31 + K + pad)
    idx = np.stack([_payload_columns(V, N, seg_col, K, rng) for _ in range(n)])
    w_ = rng.exponential(size=(n, K))
    mass = rng.uniform(0.5, 0.98, size=(n, 1))
    tlp = np.log(mass * w_ / w_.sum(1, keepdims=True)).astype(np.float32)
    xf = np.full((n, ld), np.nan, np.float32)
    xf[:, :V] = rng.standard_normal((n, V)) * 2.0
    for r in range(n):  # student close to the teacher on the payload: cancellation
        xf[r, idx[r]] = tlp[r] + 9.0 + rng.normal(0, 0.05, K).astype(np.float32)
    x = _bf16_round(xf) if dt == "bf16" else xf
    xv = np.ascontiguousarray(x[:, :V])
    g = rng.uniform(-1, 1, n).astype(np.float32)
    g[1] = 0.0
    log(f"top-k KL payload layout {layout} mode={mode}")
    xd = to_dev_logits(x)[:, :V]
    idd, tld = torch.from_numpy(idx).to(DEV), torch.from_numpy(tlp).to(DEV)
    fwd = vwc.topk_kl_fwd(xd, idd, tld, mode)
    ref_fwd = check_fwd(fwd, xv, idx, tlp, mode, 1.0)
    gdtype = torch.bfloat16 if gdt == "bf16" else torch.float32
    gbuf = torch.full((n, ld), float("nan"), dtype=gdtype, device=DEV)
    grad = vwc.topk_kl_bwd(xd, idd, tld, fwd, torch.from_numpy(g).to(DEV), mode,
                           grad_logits=gbuf[:, :V])
    ref = oracle.topk_kl_backward(xv, idx, tlp, mode, g)
    if gdt == "fp32":
        err = np.abs(_np(grad).astype(np.float64) - ref).max()
        assert err <= 1e-6, f"fp32 grad err {err}"
    else:
        bound = grad_bound(xv, idx, tlp, mode, 1.0, fwd, ref_fwd, g)
        nb = check_bf16_grad(grad_bits(grad.contiguous()), ref, bound)
        log(f"  {nb} elements beyond one bf16 step (within the bar)")
    assert np.all(_np(grad[1].float()) == 0.0)
    assert torch.isnan(gbuf[:, V:].float()).all()  # nothing written past the vocabulary


@pytest.mark.parametrize("k,pad", [(128, 0), (300, 0), (64, 1)],
                         ids=["single-pass", "fix-up k300", "fix-up unaligned"])
@pytest.mark.parametrize("mode", MODES)
def test_topk_kl_rows_equal_dense_rows(k, pad, mode):
    """The row-set calls give each listed row the dense call's bits: forward
    outputs, and gradients in the compact and the scatter layouts (the fused
    payload pass and both fix-up cases); bad row ids give NaN and no gradient."""
    w = W.scaled("distill_bf16_4096x248320_k128", 16, 151936, topk=k)
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    g = np.random.default_rng(8).uniform(-1, 1, w.n_rows).astype(np.float32)
    g[5] = 0.0
    ld = 151936 + 8 * pad + pad
    xh = np.zeros((w.n_rows, ld), np.uint16)
    xh[:, :151936] = x
    xd = to_dev_logits(xh)[:, :151936]
    idd, tld, gd = (torch.from_numpy(a).to(DEV) for a in (idx, tlp, g))
    dense = vwc.topk_kl_fwd(xd, idd, tld, mode)
    dgrad = vwc.topk_kl_bwd(xd, idd, tld, dense, gd, mode)
    rows = np.array([15, 0, 5, 9, 3], np.int32)
    rl = torch.from_numpy(rows).to(DEV).long()
    rd = torch.from_numpy(rows).to(DEV)
    sub = vwc.topk_kl_fwd_rows(xd, rd, idd[rl].contiguous(), tld[rl].contiguous(), mode)
    for key in dense:
        assert torch.equal(sub[key], dense[key][rl]), key
    comp = vwc.topk_kl_bwd_rows(xd, rd, idd[rl].contiguous(), tld[rl].contiguous(), sub,
                                gd[rl].contiguous(), mode)
    assert torch.equal(comp.view(torch.int16), dgrad[rl].view(torch.int16))
    scat = torch.full_like(xd, float("nan"))
    vwc.topk_kl_bwd_rows(xd, rd, idd[rl].contiguous(), tld[rl].contiguous(), sub,
                         gd[rl].contiguous(), mode, grad_logits=scat,
                         layout=vwc.VWC_GRAD_SCATTER)
    assert torch.equal(scat[rl].view(torch.int16), dgrad[rl].view(torch.int16))
    others = np.setdiff1d(np.arange(w.n_rows), rows)
    assert torch.isnan(scat[others].float()).all()  # rows outside the list untouched
    # a bad row id: NaN outputs, no gradient written
    bad = torch.tensor([2, -1, 16], dtype=torch.int32, device=DEV)
    bl = torch.tensor([2, 0, 0], device=DEV).long()
    sb = vwc.topk_kl_fwd_rows(xd, bad, idd[bl].contiguous(), tld[bl].contiguous(), mode)
    assert torch.isnan(sb["loss"][1:]).all() and torch.isfinite(sb["loss"][0])
    cg = torch.full((3, 151936), 7.0, dtype=torch.bfloat16, device=DEV)
    vwc.topk_kl_bwd_rows(xd, bad, idd[bl].contiguous(), tld[bl].contiguous(), sb,
                         torch.ones(3, device=DEV), mode, grad_logits=cg)
    assert (cg[1:].float() == 7.0).all()
