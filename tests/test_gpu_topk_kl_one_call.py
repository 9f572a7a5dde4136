"""GPU parity of the one-call top-k KL forward + backward (vwc_topk_kl_fwd_bwd).

Forward outputs against the fp64 oracle to the top-k forward's bar (abs 5e-5); the
gradient to the top-k backward's bars (fp32 within 1e-6, bf16 within one step or the
first-order allowance where coefficients cancel), and equal bit for bit to what the
separate backward writes from the one call's own lse, student_mass, teacher_mass and
topk_sum, also in place.  Layouts: the on-chip pass with payload columns in the tail,
on unit edges and filling a unit, fp32 and bf16, both objectives, two temperatures;
the two-call fallback (k above 256, rows off 16 bytes, another gradient dtype).
"""
import numpy as np
import pytest
import torch

import oracle
import vocab_wide_cross_amd as vwc
import workloads as W
from gpu_util import DEV, grad_bits, log, to_dev_logits, upload_workload
from test_gpu_topk_kl import (MODES, _bf16_round, _payload_columns, check_all_rows, check_bf16_grad,
                              check_fwd, grad_bound)

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy()


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_one_call_fp32_tiny(mode, tau):
    """The verl PR's small shape: 192 rows, V = 2048, K = 32, fp32."""
    w = W.get("distill_fp32_192x2048_k32")
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    g = np.random.default_rng(11).uniform(-1, 1, w.n_rows).astype(np.float32)
    g[7] = 0.0
    xd, idd, tld, gd = (to_dev_logits(x), torch.from_numpy(idx).to(DEV),
                        torch.from_numpy(tlp).to(DEV), torch.from_numpy(g).to(DEV))
    fwd, grad = vwc.topk_kl_fwd_bwd(xd, idd, tld, gd, mode, temperature=tau)
    check_fwd(fwd, x, idx, tlp, mode, tau)
    ref = oracle.topk_kl_backward(x, idx, tlp, mode, g, tau=tau)
    assert np.abs(_np(grad).astype(np.float64) - ref).max() <= 1e-6
    sep = vwc.topk_kl_bwd(xd, idd, tld, fwd, gd, mode, temperature=tau)
    assert torch.equal(_bits(grad), _bits(sep))
    assert torch.all(grad[7] == 0)
    # in place: the gradient replaces the logits, same bits
    xin = to_dev_logits(x)
    fwd2, gin = vwc.topk_kl_fwd_bwd(xin, idd, tld, gd, mode, temperature=tau, grad_logits=xin)
    assert gin.data_ptr() == xin.data_ptr()
    for key in fwd:
        assert torch.equal(fwd2[key], fwd[key]), key
    assert torch.equal(_bits(gin), _bits(grad))


# (dtype, vocab, k): rows with a tail past the whole vectors and payload columns on
# it, on unit edges and filling a unit; k up to the on-chip limit of 256.
LAYOUTS = [("bf16", 151939, 64), ("bf16", 151939, 256), ("fp32", 70001, 32)]


@pytest.mark.parametrize("layout", LAYOUTS, ids=[f"{a}-V{b}-k{c}" for a, b, c in LAYOUTS])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_one_call_payload_layouts(layout, mode, tau):
    dt, V, K = layout
    n = 6
    N = 8 if dt == "bf16" else 4
    ld = (V + 7) // 8 * 8
    rng = np.random.default_rng(41 + K)
    idx = np.stack([_payload_columns(V, N, 64 * N, K, rng) for _ in range(n)])
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
    log(f"one-call top-k KL layout {layout} mode={mode} tau={tau}")
    xd = to_dev_logits(x)[:, :V]
    idd, tld, gd = (torch.from_numpy(a).to(DEV) for a in (idx, tlp, g))
    gdtype = torch.bfloat16 if dt == "bf16" else torch.float32
    gbuf = torch.full((n, ld), float("nan"), dtype=gdtype, device=DEV)
    fwd, grad = vwc.topk_kl_fwd_bwd(xd, idd, tld, gd, mode, temperature=tau,
                                    grad_logits=gbuf[:, :V])
    ref_fwd = check_fwd(fwd, xv, idx, tlp, mode, tau)
    ref = oracle.topk_kl_backward(xv, idx, tlp, mode, g, tau=tau)
    if dt == "fp32":
        err = np.abs(_np(grad).astype(np.float64) - ref).max()
        assert err <= 1e-6, f"fp32 grad err {err}"
    else:
        nb = check_bf16_grad(grad_bits(grad.contiguous()), ref,
                             grad_bound(xv, idx, tlp, mode, tau, fwd, ref_fwd, g))
        log(f"  {nb} elements beyond one bf16 step (within the bar)")
    sbuf = torch.full((n, ld), float("nan"), dtype=gdtype, device=DEV)
    sep = vwc.topk_kl_bwd(xd, idd, tld, fwd, gd, mode, temperature=tau, grad_logits=sbuf[:, :V])
    assert torch.equal(_bits(grad), _bits(sep))
    assert np.all(_np(grad[1].float()) == 0.0)
    assert torch.isnan(gbuf[:, V:].float()).all()  # nothing written past the vocabulary


def test_one_call_clamp_guard_and_bad_index():
    """Q > P clamps the truncated loss (row gradient +0.0); 1 - Q < eps turns off the
    tail term's gradient; an out-of-range payload column gives NaN outputs; each as
    the separate calls give them from the one call's outputs."""
    V, K = 4096, 8
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, V)).astype(np.float32)
    idx = np.stack([rng.choice(V, K, replace=False) for _ in range(4)]).astype(np.int32)
    tlp = np.log(np.full((4, K), 0.5 / K)).astype(np.float32)
    x[0, idx[0]] = 12.0
    x[1, idx[1]] = 40.0
    idx[2, 3] = V  # outside the row
    g = np.ones(4, np.float32)
    xd, idd, tld, gd = (to_dev_logits(x), torch.from_numpy(idx).to(DEV),
                        torch.from_numpy(tlp).to(DEV), torch.from_numpy(g).to(DEV))
    good = np.array([0, 1, 3])
    for mode in MODES:
        fwd, grad = vwc.topk_kl_fwd_bwd(xd, idd, tld, gd, mode)
        assert np.isnan(_np(fwd["loss"])[2]) and np.isnan(_np(fwd["teacher_mass"])[2])
        sub = {k: v[good] for k, v in fwd.items()}
        check_fwd(sub, x[good], idx[good], tlp[good], mode, 1.0)
        ref = oracle.topk_kl_backward(x[good], idx[good], tlp[good], mode, g[good])
        assert np.abs(_np(grad[good]).astype(np.float64) - ref).max() <= 1e-6
        sep = vwc.topk_kl_bwd(xd, idd, tld, fwd, gd, mode)
        a, b = _np(grad), _np(sep)
        assert np.array_equal(np.isnan(a), np.isnan(b))
        assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])
        if mode == vwc.VWC_KL_TRUNCATED:
            assert _np(fwd["loss"])[0] == 0.0 and np.all(a[0] == 0.0)


@pytest.mark.parametrize("case", ["k300", "unaligned", "fp32-grad"])
def test_one_call_falls_back_to_two_calls(case):
    """Outside the on-chip pass the call runs the separate forward and backward:
    the same bits as calling them."""
    V = 151936
    k = 300 if case == "k300" else 64
    w = W.scaled("distill_bf16_4096x248320_k128", 8, V, topk=k)
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    g = np.random.default_rng(9).uniform(-1, 1, w.n_rows).astype(np.float32)
    pad = 1 if case == "unaligned" else 0
    xh = np.zeros((w.n_rows, V + pad), np.uint16)
    xh[:, :V] = x
    xd = to_dev_logits(xh)[:, :V]
    idd, tld, gd = (torch.from_numpy(a).to(DEV) for a in (idx, tlp, g))
    gdt = torch.float32 if case == "fp32-grad" else None
    mode = vwc.VWC_KL_TAIL
    fwd, grad = vwc.topk_kl_fwd_bwd(xd, idd, tld, gd, mode, grad_dtype=gdt)
    f2 = vwc.topk_kl_fwd(xd, idd, tld, mode)
    for key in fwd:
        assert torch.equal(fwd[key], f2[key]), key
    sep = vwc.topk_kl_bwd(xd, idd, tld, f2, gd, mode, grad_dtype=gdt)
    assert torch.equal(_bits(grad), _bits(sep))


@pytest.mark.timeout(900)
def test_one_call_full_size_k128():
    """The page's distillation dimensions (4096 x 248320 bf16, K = 128), in the launch
    the bench times: every row's gradient equals the separate backward's from the one
    call's outputs, and every row meets the oracle's bars, for both objectives."""
    w = W.get("distill_bf16_4096x248320_k128")
    x, xh = upload_workload(w, keep_rows=True)
    idx, tlp = W.topk_payload(w)
    g = np.random.default_rng(5).uniform(-1, 1, w.n_rows).astype(np.float32)
    g[100] = 0.0
    idd, tld, gd = (torch.from_numpy(a).to(DEV) for a in (idx, tlp, g))
    for mode in MODES:
        fwd, grad = vwc.topk_kl_fwd_bwd(x, idd, tld, gd, mode)
        sep = vwc.topk_kl_bwd(x, idd, tld, fwd, gd, mode)
        assert torch.equal(_bits(grad), _bits(sep))
        del sep
        check_all_rows(fwd, grad, xh, idx, tlp, mode, 1.0, g, "one-call top-k KL full size")
        assert torch.all(grad[100] == 0)
        del grad
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", MODES)
def test_one_call_rows_equal_dense_rows(mode):
    """The row-set one call gives each listed row the dense one call's bits (outputs
    and gradient, compact and scatter layouts); bad row ids give NaN outputs and no
    gradient."""
    w = W.scaled("distill_bf16_4096x248320_k128", 16, 151936)
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    g = np.random.default_rng(8).uniform(-1, 1, w.n_rows).astype(np.float32)
    g[5] = 0.0
    xd = to_dev_logits(x)
    idd, tld, gd = (torch.from_numpy(a).to(DEV) for a in (idx, tlp, g))
    dense, dgrad = vwc.topk_kl_fwd_bwd(xd, idd, tld, gd, mode)
    rows = np.array([15, 0, 5, 9, 3], np.int32)
    rl = torch.from_numpy(rows).to(DEV).long()
    rd = torch.from_numpy(rows).to(DEV)
    pay = (idd[rl].contiguous(), tld[rl].contiguous())
    sub, comp = vwc.topk_kl_fwd_bwd_rows(xd, rd, *pay, gd[rl].contiguous(), mode)
    for key in dense:
        assert torch.equal(sub[key], dense[key][rl]), key
    assert torch.equal(_bits(comp), _bits(dgrad[rl]))
    scat = torch.full_like(xd, float("nan"))
    vwc.topk_kl_fwd_bwd_rows(xd, rd, *pay, gd[rl].contiguous(), mode, grad_logits=scat,
                             layout=vwc.VWC_GRAD_SCATTER)
    assert torch.equal(_bits(scat[rl]), _bits(dgrad[rl]))
    others = np.setdiff1d(np.arange(w.n_rows), rows)
    assert torch.isnan(scat[others].float()).all()  # rows outside the list untouched
    bad = torch.tensor([2, -1, 16], dtype=torch.int32, device=DEV)
    bl = torch.tensor([2, 0, 0], device=DEV).long()
    cg = torch.full((3, 151936), 7.0, dtype=torch.bfloat16, device=DEV)
    sb, _ = vwc.topk_kl_fwd_bwd_rows(xd, bad, idd[bl].contiguous(), tld[bl].contiguous(),
                                     gd[bl].contiguous(), mode, grad_logits=cg)
    assert torch.isnan(sb["loss"][1:]).all() and torch.isnan(sb["lse"][1:]).all()
    assert torch.isfinite(sb["loss"][0])
    assert torch.equal(_bits(cg[0]), _bits(dgrad[2]))
    assert torch.all(cg[1:].float() == 7.0)  # no gradient written for bad ids


@pytest.mark.parametrize("k", [64, 300], ids=["on-chip", "two-call"])
def test_one_call_without_loss_output(k):
    """The loss output may be null (the C ABI allows it): the other outputs and the
    gradient are those of the call that writes the loss, in the on-chip pass and in
    the two-call fallback."""
    from vocab_wide_cross_amd import _binding as B
    w = W.scaled("distill_bf16_4096x248320_k128", 6, 151936, topk=k)
    x = W.all_logits(w)
    idx, tlp = W.topk_payload(w)
    g = np.random.default_rng(17).uniform(-1, 1, w.n_rows).astype(np.float32)
    xd = to_dev_logits(x)
    idd, tld, gd = (torch.from_numpy(a).to(DEV) for a in (idx, tlp, g))
    ref, rgrad = vwc.topk_kl_fwd_bwd(xd, idd, tld, gd, vwc.VWC_KL_TAIL, temperature=0.7)
    n, V = w.n_rows, w.vocab
    out = {key: torch.full((n,), 7.0, device=DEV)
           for key in ("student_mass", "teacher_mass", "topk_sum", "lse")}
    grad = torch.full_like(xd, 3.0)
    ws, wsb = B._workspace(n, V, xd, None)
    st = B._lib.vwc_topk_kl_fwd_bwd(
        B._ptr(xd), B._dtype(xd), n, V, V, B._ptr(idd), B._ptr(tld), k, vwc.VWC_KL_TAIL, 1e-6,
        0.7, B._ptr(gd), None, B._ptr(out["student_mass"]), B._ptr(out["teacher_mass"]),
        B._ptr(out["topk_sum"]), B._ptr(out["lse"]), B._ptr(grad), B._dtype(grad), V,
        B._ptr(ws), wsb, B._stream(None, xd))
    assert st == 0, B._lib.vwc_last_error().decode()
    torch.cuda.synchronize()
    for key, v in out.items():
        assert torch.equal(v, ref[key]), key
    assert torch.equal(_bits(grad), _bits(rgrad))


@pytest.mark.parametrize("mode", MODES)
def test_one_call_rows_at_every_16_byte_phase(mode):
    """Rows at an odd stride (151941 bf16) start at all eight 16-byte phases.  With a
    gradient of the same layout (a buffer of that stride, or in place) the on-chip
    pass runs with head elements before the first whole vector; payload columns in
    the head and the tail are stored by the threads that own those elements.  The
    result meets the oracle's bars and equals, bit for bit, the separate backward
    from the call's own outputs."""
    V, K, n = 151939, 64, 9
    ld = V + 2
    rng = np.random.default_rng(77)
    idx = np.stack([_payload_columns(V, 8, 64 * 8, K, rng) for _ in range(n)])
    w_ = rng.exponential(size=(n, K))
    mass = rng.uniform(0.5, 0.98, size=(n, 1))
    tlp = np.log(mass * w_ / w_.sum(1, keepdims=True)).astype(np.float32)
    xf = np.full((n, ld), np.nan, np.float32)
    xf[:, :V] = rng.standard_normal((n, V)) * 2.0
    for r in range(n):
        xf[r, idx[r]] = tlp[r] + 9.0 + rng.normal(0, 0.05, K).astype(np.float32)
    x = _bf16_round(xf)
    xv = np.ascontiguousarray(x[:, :V])
    g = rng.uniform(-1, 1, n).astype(np.float32)
    g[2] = 0.0
    xd = to_dev_logits(x)[:, :V]
    assert xd.stride(0) == ld
    idd, tld, gd = (torch.from_numpy(a).to(DEV) for a in (idx, tlp, g))
    gbuf = torch.full((n, ld), float("nan"), dtype=torch.bfloat16, device=DEV)
    fwd, grad = vwc.topk_kl_fwd_bwd(xd, idd, tld, gd, mode, grad_logits=gbuf[:, :V])
    ref_fwd = check_fwd(fwd, xv, idx, tlp, mode, 1.0)
    ref = oracle.topk_kl_backward(xv, idx, tlp, mode, g)
    check_bf16_grad(grad_bits(grad.contiguous()), ref,
                    grad_bound(xv, idx, tlp, mode, 1.0, fwd, ref_fwd, g))
    sbuf = torch.full((n, ld), float("nan"), dtype=torch.bfloat16, device=DEV)
    sep = vwc.topk_kl_bwd(xd, idd, tld, fwd, gd, mode, grad_logits=sbuf[:, :V])
    assert torch.equal(_bits(grad), _bits(sep))
    assert torch.isnan(gbuf[:, V:].float()).all()
    assert torch.all(grad[2] == 0)
    xin = to_dev_logits(x)[:, :V]
    fwd2, gin = vwc.topk_kl_fwd_bwd(xin, idd, tld, gd, mode, grad_logits=xin)
    for key in fwd:
        assert torch.equal(fwd2[key], fwd[key]), key
    assert torch.equal(_bits(gin), _bits(grad))


@pytest.mark.parametrize("mode", MODES)
def test_one_call_special_values(mode):
    """-inf logits off the payload (masked entries, a whole leading stretch of them)
    and a NaN logit in one row: outputs as the separate forward gives them (NaN in
    the same places), the gradient the separate backward's bits from the call's own
    outputs, and the oracle's values on the finite rows."""
    V, K, n = 3001, 16, 12
    rng = np.random.default_rng(23)
    x = rng.standard_normal((n, V)).astype(np.float32)
    idx = np.stack([rng.choice(np.arange(400, V), K, replace=False) for _ in range(n)]).astype(np.int32)
    tlp = np.log(np.full((n, K), 0.6 / K)).astype(np.float32)
    mask = rng.random(x.shape) < 0.3
    mask[:, :300] = True
    for r in range(n):
        mask[r, idx[r]] = False
    x[mask] = -np.inf
    x[5, 2000] = np.nan
    g = rng.uniform(-1, 1, n).astype(np.float32)
    xd, idd, tld, gd = (torch.from_numpy(a).to(DEV) for a in (x, idx, tlp, g))
    fwd, grad = vwc.topk_kl_fwd_bwd(xd, idd, tld, gd, mode, temperature=0.7)
    sf = vwc.topk_kl_fwd(xd, idd, tld, mode, temperature=0.7)
    for key in fwd:
        a, b = _np(fwd[key]).astype(np.float64), _np(sf[key]).astype(np.float64)
        assert np.array_equal(np.isnan(a), np.isnan(b)), key
        ok = ~np.isnan(a)
        assert np.abs(a[ok] - b[ok]).max() <= 1e-4, key
    assert np.isnan(_np(fwd["lse"])[5])
    sep = vwc.topk_kl_bwd(xd, idd, tld, fwd, gd, mode, temperature=0.7)
    a, b = _np(grad), _np(sep)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])
    rows = np.array([r for r in range(n) if r != 5])
    check_fwd({k: v[torch.from_numpy(rows).to(DEV)] for k, v in fwd.items()}, x[rows], idx[rows],
              tlp[rows], mode, 0.7)
    ref = oracle.topk_kl_backward(x[rows], idx[rows], tlp[rows], mode, g[rows], tau=0.7)
    assert np.abs(a[rows].astype(np.float64) - ref).max() <= 1e-6
    assert np.all(a[rows][mask[rows]] == 0.0)  # masked entries: probability 0
