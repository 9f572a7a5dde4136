"""Pins for the fp64 oracle, each against something other than the oracle itself:
library routines (torch fp64 cross_entropy, log_softmax autograd, Categorical
entropy), closed forms, invariants, brute force and central finite differences.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a wrong
sign or index, tau applied on one side only, a transposed partial) fails at least
one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def tiny():
    w = W.get("tiny_fp32_64x2048")
    return w, W.all_logits(w), W.targets(w), W.grad_out(w)


# ----------------------------------------------------------------------------- logprob


@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_logprob_is_minus_cross_entropy(tiny, tau):
    """log_softmax(x/tau)[t] == -cross_entropy(x/tau, t): the identity the Megatron
    issue builds on ("Avoid full-vocabulary TP gather ...", "Proposed solution")."""
    _, x, t, _ = tiny
    o = oracle.forward(x, t, tau=tau)
    z = torch.from_numpy(x).double() / float(np.float32(tau))
    ce = torch.nn.functional.cross_entropy(z, torch.from_numpy(t).long(), reduction="none")
    np.testing.assert_allclose(o["logprob"], -ce.numpy(), rtol=0, atol=1e-12)
    lse = torch.logsumexp(z, dim=1).numpy()
    np.testing.assert_allclose(o["lse"], lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["masked_bf16_4096x151936", "spiked_bf16_8192x248320",
                                  "packed_bf16_32768x248320", "extreme_fp32_16384x248320"])
def test_logprob_identity_sampled_rows(name):
    """Same identity on a few rows of every full-size workload (bf16 decode included)."""
    w = W.get(name)
    rows = np.array([0, 1, w.n_rows // 2, w.n_rows - 1])
    x = W.logits_rows(w, rows)
    t = W.targets(w)[rows]
    o = oracle.forward(x, t, tau=w.tau)
    xf = W.bf16_bits_to_float32(x) if w.dtype == "bf16" else x
    z = torch.from_numpy(xf).double() / float(np.float32(w.tau))
    ce = torch.nn.functional.cross_entropy(z, torch.from_numpy(t).long(), reduction="none")
    # |lp| reaches 1.4e4 in the extreme workload: compare relative to the magnitude.
    np.testing.assert_allclose(o["logprob"], -ce.numpy(), rtol=1e-13, atol=1e-12)


def test_logprob_brute_force(tiny):
    """Naive softmax without the max shift (safe for N(0,1) logits), pure numpy."""
    _, x, t, _ = tiny
    o = oracle.forward(x, t)
    e = np.exp(x.astype(np.float64))
    naive = np.log(e[np.arange(x.shape[0]), t] / e.sum(axis=1))
    np.testing.assert_allclose(o["logprob"], naive, rtol=0, atol=1e-12)


def test_logprob_normalizes(tiny):
    """sum_t exp(logprob(t)) == 1 for every row (all V targets of 3 rows)."""
    _, x, _, _ = tiny
    V = x.shape[1]
    for r in (0, 17, 63):
        xr = np.repeat(x[r:r + 1], V, axis=0)
        o = oracle.forward(xr, np.arange(V, dtype=np.int32), want=("logprob",))
        assert abs(np.exp(o["logprob"]).sum() - 1.0) < 1e-12


def test_uniform_logits():
    for V in (1, 2, 7, 2048, 151936):
        x = np.full((1, V), 0.25, np.float32)
        o = oracle.forward(x, np.array([V - 1], np.int32), tau=0.7)
        assert abs(o["logprob"][0] + math.log(V)) < 1e-12
        assert abs(o["entropy"][0] - math.log(V)) < 1e-12 * max(1.0, math.log(V))


def test_shift_invariance():
    """lp(x + c) == lp(x) with exactly representable shifted logits."""
    rng = np.random.default_rng(5)
    x = (rng.integers(-256, 256, size=(8, 1000)) / 64.0).astype(np.float32)
    t = rng.integers(0, 1000, size=8).astype(np.int32)
    a = oracle.forward(x, t)
    b = oracle.forward((x + np.float32(5.0)).astype(np.float32), t)
    np.testing.assert_allclose(a["logprob"], b["logprob"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a["entropy"], b["entropy"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["lse"] - a["lse"], 5.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("tau", [0.5, 2.0, 0.25])
def test_temperature_is_logit_scaling(tiny, tau):
    """lp(x, tau) == lp(x / tau, 1) for power-of-two tau (x / tau exact in fp32).
    Pins that tau divides both the target logit and the log-sum-exp."""
    _, x, t, _ = tiny
    a = oracle.forward(x, t, tau=tau)
    b = oracle.forward((x / np.float32(tau)).astype(np.float32), t, tau=1.0)
    for k in ("logprob", "lse", "entropy"):
        np.testing.assert_allclose(a[k], b[k], rtol=0, atol=1e-12)


def test_golden_closed_forms():
    path = os.path.join(GOLDEN, "closed_forms.txt")
    env = {"log": math.log, "log1p": math.log1p, "exp": math.exp}
    n = 0
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, xs, t, tau, lp_expr, h_expr, _src = [s.strip() for s in line.split("|")]
        x = np.array([[float(v) for v in xs.split(",")]], np.float32)
        o = oracle.forward(x, np.array([int(t)], np.int32), tau=float(tau))
        assert abs(o["logprob"][0] - eval(lp_expr, env)) < 1e-14, name
        assert abs(o["entropy"][0] - eval(h_expr, env)) < 1e-14, name
        n += 1
    assert n >= 6


def test_golden_uniform_payload_mass():
    """Printed example: a uniform payload has top-k log-probs of -log V and top-k mass
    K / V = 2.11e-4 (verl PR, tail-aware top-k KL text, VeOmni notes)."""
    vals = {}
    for line in open(os.path.join(GOLDEN, "uniform_payload_mass.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = [s.strip() for s in line.split("=")]
            vals[k] = float(v)
    V, K = int(vals["vocab"]), int(vals["k"])
    x = np.zeros((K, V), np.float32)
    t = np.linspace(0, V - 1, K).astype(np.int32)
    o = oracle.forward(x, t, want=("logprob",))
    assert np.all(np.abs(o["logprob"] + math.log(V)) < 1e-12)
    mass = float(np.exp(o["logprob"]).sum())
    assert float(f"{mass:.{int(vals['printed_digits']) - 1}e}") == vals["printed_mass"]


# ----------------------------------------------------------------------------- entropy


def test_entropy_brute_force_and_library(tiny):
    _, x, t, _ = tiny
    for tau in (1.0, 0.7):
        o = oracle.forward(x, t, tau=tau)
        z = x.astype(np.float64) / float(np.float32(tau))
        p = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
        brute = -(p * np.log(p)).sum(axis=1)
        np.testing.assert_allclose(o["entropy"], brute, rtol=0, atol=1e-12)
        cat = torch.distributions.Categorical(logits=torch.from_numpy(z)).entropy().numpy()
        np.testing.assert_allclose(o["entropy"], cat, rtol=0, atol=1e-12)


def _minus_inf_rows(seed=21, n=6, V=777):
    """Rows with -inf entries (masked vocabulary), one row with whole runs of them."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, V)).astype(np.float32) * 2
    mask = rng.random((n, V)) < 0.3
    mask[1, :400] = True
    t = rng.integers(0, V, n).astype(np.int32)
    mask[np.arange(n), t] = False
    x[mask] = -np.inf
    return x, t, mask


def test_entropy_with_minus_inf_entries():
    """A -inf logit has probability 0 and adds 0 log 0 = 0 to the entropy: the
    oracle equals torch fp64 Categorical (which clamps -inf logits) and itself on
    the row with those columns removed; logprob and lse are unchanged too."""
    x, t, mask = _minus_inf_rows()
    for tau in (1.0, 0.7):
        o = oracle.forward(x, t, tau=tau)
        z = torch.from_numpy(x).double() / float(np.float32(tau))
        cat = torch.distributions.Categorical(logits=z).entropy().numpy()
        np.testing.assert_allclose(o["entropy"], cat, rtol=0, atol=1e-12)
        for r in range(x.shape[0]):
            keep = ~mask[r]
            tr = np.array([int(keep[:t[r]].sum())], np.int32)
            ref = oracle.forward(x[r:r + 1, keep], tr, tau=tau)
            for k in ("logprob", "lse", "entropy"):
                assert abs(o[k][r] - ref[k][0]) <= 1e-12, (r, k)


def test_entropy_grad_with_minus_inf_entries():
    """d(g lp + h H)/dx with -inf logits: exactly 0 at those columns and, at the
    others, the gradient of the row with them removed; torch fp64 autograd of
    log_softmax and Categorical entropy agrees."""
    x, t, mask = _minus_inf_rows(22)
    rng = np.random.default_rng(23)
    g = rng.uniform(-1, 1, x.shape[0]).astype(np.float32)
    h = rng.uniform(-1, 1, x.shape[0]).astype(np.float32)
    tau = 0.7
    gr = oracle.backward_entropy(x, t, g, h, tau=tau)
    assert np.all(gr[mask] == 0.0) and np.all(np.isfinite(gr))
    for r in range(x.shape[0]):
        keep = ~mask[r]
        tr = np.array([int(keep[:t[r]].sum())], np.int32)
        ref = oracle.backward_entropy(x[r:r + 1, keep], tr, g[r:r + 1], h[r:r + 1], tau=tau)
        np.testing.assert_allclose(gr[r, keep], ref[0], rtol=0, atol=1e-14)
    xt = torch.from_numpy(x).double().requires_grad_(True)
    z = xt / float(np.float32(tau))
    lp = torch.log_softmax(z, dim=1)[torch.arange(x.shape[0]), torch.from_numpy(t).long()]
    H = torch.distributions.Categorical(logits=z).entropy()
    (lp * torch.from_numpy(g).double() + H * torch.from_numpy(h).double()).sum().backward()
    np.testing.assert_allclose(gr, xt.grad.numpy(), rtol=0, atol=1e-14)


def test_slice_of_minus_inf_adds_nothing():
    """A vocabulary slice whose logits are all -inf has sum 0 and adds nothing to
    the merge: slicing reproduces the single pass, entropy included."""
    x, t, _ = _minus_inf_rows(24, V=600)
    x[:, 200:400] = -np.inf
    t = np.where((t >= 200) & (t < 400), t - 200, t).astype(np.int32)
    o = oracle.forward(x, t, tau=0.7)
    for vchunk in (200, 100, 7):
        v = oracle.forward_vchunk(x, t, 0.7, vchunk)
        for k in ("logprob", "lse", "entropy"):
            np.testing.assert_allclose(v[k], o[k], rtol=1e-12, atol=1e-12)


def test_entropy_one_dominant_entry():
    x = np.zeros((1, 4096), np.float32)
    x[0, 123] = 1000.0
    o = oracle.forward(x, np.array([123], np.int32))
    assert abs(o["logprob"][0]) < 1e-300 or o["logprob"][0] == 0.0
    assert 0.0 <= o["entropy"][0] < 1e-300 or o["entropy"][0] == 0.0


def test_extreme_workload_closed_form():
    """In the +-1e4 workload every non-extreme term underflows next to the +1e4
    entries, so H = ln c and lp = -ln c at a +1e4 target, else (x_t - 1e4)/tau - ln c,
    where c counts the +1e4 entries of the row."""
    w = W.get("extreme_fp32_16384x248320")
    rows = np.array([3, 4096])
    x = W.logits_rows(w, rows)
    t = W.targets(w)[rows]
    t[1] = int(np.flatnonzero(x[1] == np.float32(1e4))[0])  # one row with a +1e4 target
    o = oracle.forward(x, t, tau=w.tau)
    tau = float(np.float32(w.tau))
    for i in range(2):
        c = int((x[i] == np.float32(1e4)).sum())
        assert 1000 < c < 1500
        assert abs(o["entropy"][i] - math.log(c)) < 1e-9
        xt = float(x[i, t[i]])
        want = -math.log(c) if xt == 1e4 else (xt - 1e4) / tau - math.log(c)
        assert abs(o["logprob"][i] - want) < 1e-9 * max(1.0, abs(want))


# ----------------------------------------------------------------------------- gradient


def test_grad_rows_sum_to_zero(tiny):
    _, x, t, g = tiny
    for tau in (1.0, 0.7):
        gr = oracle.backward(x, t, g, tau=tau)
        assert np.abs(gr.sum(axis=1)).max() < x.shape[1] * 1e-16 * 4


def test_grad_matches_torch_autograd(tiny):
    _, x, t, g = tiny
    for tau in (1.0, 0.7):
        gr = oracle.backward(x, t, g, tau=tau)
        xt = torch.from_numpy(x).double().requires_grad_(True)
        lp = torch.log_softmax(xt / float(np.float32(tau)), dim=1)
        lp = lp[torch.arange(x.shape[0]), torch.from_numpy(t).long()]
        (lp * torch.from_numpy(g).double()).sum().backward()
        np.testing.assert_allclose(gr, xt.grad.numpy(), rtol=0, atol=1e-14)


@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_grad_central_finite_differences(tiny, tau):
    """d lp_r / d x_rj by central differences of the oracle's own forward, on the
    target column and a spread of other columns of 3 rows."""
    _, x, t, _ = tiny
    V = x.shape[1]
    h = 2.0 ** -10
    for r in (0, 31, 63):
        cols = np.unique(np.concatenate([[t[r]], np.linspace(0, V - 1, 24).astype(int)]))
        plus = np.repeat(x[r:r + 1], len(cols), axis=0)
        minus = plus.copy()
        plus[np.arange(len(cols)), cols] += np.float32(h)
        minus[np.arange(len(cols)), cols] -= np.float32(h)
        step = (plus[np.arange(len(cols)), cols].astype(np.float64)
                - minus[np.arange(len(cols)), cols].astype(np.float64))
        tt = np.full(len(cols), t[r], np.int32)
        lp_p = oracle.forward(plus, tt, tau=tau, want=("logprob",))["logprob"]
        lp_m = oracle.forward(minus, tt, tau=tau, want=("logprob",))["logprob"]
        fd = (lp_p - lp_m) / step
        gr = oracle.backward(x[r:r + 1], t[r:r + 1], np.ones(1, np.float32), tau=tau)[0]
        np.testing.assert_allclose(gr[cols], fd, rtol=0, atol=1e-8)


def test_grad_zero_rows_are_positive_zero(tiny):
    """Rows whose incoming gradient is 0 get exactly +0.0 ("Avoid full-vocabulary TP
    gather ...", "Prototype correctness": masked positions have exactly zero gradient)."""
    _, x, t, g = tiny
    g = g.copy()
    g[::3] = 0.0
    g[1] = -0.0
    gr = oracle.backward(x, t, g)
    z = (g == 0.0)
    assert np.all(gr[z] == 0.0) and not np.any(np.signbit(gr[z]))
    assert np.all(np.abs(gr[~z]).max(axis=1) > 0)


# ----------------------------------------------------------------------------- split-V


@pytest.mark.parametrize("vchunk", [1, 2, 3, 5, 7, 8, 64, 1000, 4096])
def test_vocab_chunks_match_single_pass(tiny, vchunk):
    """Vocabulary chunks merged by the shard combine reproduce the single pass
    (chunk sizes of the verl PR's small test: 7, 64, 4096)."""
    _, x, t, _ = tiny
    for tau in (1.0, 0.7):
        a = oracle.forward(x, t, tau=tau)
        b = oracle.forward_vchunk(x, t, tau=tau, vchunk=vchunk)
        for k in ("logprob", "lse", "entropy"):
            np.testing.assert_allclose(b[k], a[k], rtol=1e-12, atol=1e-12)


def test_split4_extreme_rows():
    """The 4 x 62080 slicing of the extreme fp32 workload against the single pass."""
    w = W.get("extreme_fp32_16384x248320")
    rows = np.array([0, 9999])
    x = W.logits_rows(w, rows)
    t = W.targets(w)[rows]
    a = oracle.forward(x, t, tau=w.tau)
    parts = [oracle.slice_partial(x, q * 62080, 62080, t, w.tau) for q in range(4)]
    pm, ps, pw, pt = (np.stack([p[i] for p in parts]) for i in range(4))
    # exactly one slice owns each target
    assert np.all((pt > -np.inf).sum(axis=0) == 1)
    b = oracle.combine(pm, ps, pw, pt)
    for k in ("logprob", "lse", "entropy"):
        np.testing.assert_allclose(b[k], a[k], rtol=1e-12, atol=1e-12)


def test_unowned_target_is_visible():
    x = np.zeros((1, 16), np.float32)
    pm, ps, pw, pt = oracle.slice_partial(x, 0, 8, np.array([12], np.int32), 1.0)
    assert pt[0] == -np.inf
    o = oracle.combine(pm[None], ps[None], pw[None], pt[None])
    assert o["logprob"][0] == -np.inf


# ----------------------------------------------------------------------------- chunks / rows


def test_row_chunks_bitwise(tiny):
    """Row chunking changes nothing, bit for bit: the chunk sizes of the NeMo-RL
    PR's tests (1, 2, 3, 5, 7, 8, 64) and of the verl PR's (7, 64, 4096)."""
    _, x, t, _ = tiny
    a = oracle.forward(x, t, row_chunk=4096)
    for c in (1, 2, 3, 5, 7, 8, 64):
        b = oracle.forward(x, t, row_chunk=c)
        for k in a:
            assert np.array_equal(a[k], b[k])


def test_default_chunk_with_a_residual():
    """1024 + 7 rows through the default chunk of 1024: the residual chunk of 7
    gives the rows' single-row values, bit for bit (forward and gradient)."""
    w = W.scaled("tiny_fp32_64x2048", 1031, 257)
    x, t, g = W.all_logits(w), W.targets(w), W.grad_out(w)
    a = oracle.forward(x, t, row_chunk=1024)
    for r in (0, 1023, 1024, 1030):
        b = oracle.forward(x[r:r + 1], t[r:r + 1], row_chunk=1)
        for k in a:
            assert a[k][r] == b[k][0]
    gr = oracle.backward(x, t, g)
    g1 = oracle.backward(x[1024:], t[1024:], g[1024:])
    assert np.array_equal(gr[1024:], g1)


def test_compact_rows_equal_dense_rows():
    w = W.scaled("masked_bf16_4096x151936", 96, 3001)
    x = W.all_logits(w)
    t = W.targets(w)
    idx = W.row_index(w)
    assert np.array_equal(idx, np.nonzero(W.loss_mask(w))[0])
    d = oracle.forward(x, t)
    c = oracle.forward(x, t, rows=idx)
    for k in d:
        assert np.array_equal(d[k][idx], c[k])


def test_errors():
    x = np.zeros((2, 8), np.float32)
    t = np.array([0, 9], np.int32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.forward(x, t)
    assert e.value.code == -2
    with pytest.raises(oracle.OracleError):
        oracle.forward(x, np.array([0, 1], np.int32), row_chunk=0)
    with pytest.raises(oracle.OracleError):
        oracle.forward(x, np.array([0, 1], np.int32), row_chunk=-3)
    with pytest.raises(oracle.OracleError):
        oracle.forward(x, np.array([0, 1], np.int32), tau=0.0)
    with pytest.raises(oracle.OracleError) as e:
        oracle.forward(x, np.array([0, 1], np.int32), rows=np.array([0, 2], np.int32))
    assert e.value.code == -3
    # zero-length row sets are a no-op
    o = oracle.forward(x, np.array([0, 1], np.int32), rows=np.zeros(0, np.int32))
    assert o["logprob"].shape == (0,)


# ----------------------------------------------------------------------------- bf16 rounding


def test_bf16_rne_against_torch():
    """fp64 -> bf16 RNE equals torch's fp32 -> bf16 for fp32-representable values."""
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-40, 38, 100000),
                        [0.0, -0.0, 1e-45, -1e-45, 3.4e38, -3.4e38, np.inf, -np.inf]])
    v32 = v.astype(np.float32)
    want = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne(v32.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_rne_ties_and_double_rounding():
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,                   # tie -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 0x3F82,               # tie -> even (1 + 2^-6)
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,      # above the tie: no double rounding
        -(1.0 + 2.0 ** -8 + 2.0 ** -30): 0xBF81,
        2.0 ** -133: 0x0001,                       # smallest bf16 subnormal
        2.0 ** -134: 0x0000,                       # tie with zero -> even (0)
        3 * 2.0 ** -134: 0x0002,                   # tie 1.5 ulp -> even (2 ulp)
        (2 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,      # tie at the top -> overflow
        float("nan"): 0x7FC0,
    }
    for v, want in cases.items():
        assert oracle.bf16_rne(np.array([v]))[0] == want, (v, hex(want))


# ----------------------------------------------------------------------------- entropy gradient


def test_entropy_grad_matches_torch_autograd(tiny):
    """d(g lp + h H)/dx against torch fp64 autograd of log_softmax and Categorical entropy."""
    _, x, t, g = tiny
    h = np.random.default_rng(4).uniform(-1, 1, x.shape[0]).astype(np.float32)
    for tau in (1.0, 0.7):
        gr = oracle.backward_entropy(x, t, g, h, tau=tau)
        xt = torch.from_numpy(x).double().requires_grad_(True)
        z = xt / float(np.float32(tau))
        lp = torch.log_softmax(z, dim=1)[torch.arange(x.shape[0]), torch.from_numpy(t).long()]
        H = torch.distributions.Categorical(logits=z).entropy()
        (lp * torch.from_numpy(g).double() + H * torch.from_numpy(h).double()).sum().backward()
        np.testing.assert_allclose(gr, xt.grad.numpy(), rtol=0, atol=1e-14)


@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_entropy_grad_central_finite_differences(tiny, tau):
    """dH_r/dx_rj by central differences of the oracle's own forward entropy."""
    _, x, t, _ = tiny
    V = x.shape[1]
    h = 2.0 ** -10
    for r in (2, 40):
        cols = np.linspace(0, V - 1, 24).astype(int)
        plus = np.repeat(x[r:r + 1], len(cols), axis=0)
        minus = plus.copy()
        plus[np.arange(len(cols)), cols] += np.float32(h)
        minus[np.arange(len(cols)), cols] -= np.float32(h)
        step = (plus[np.arange(len(cols)), cols].astype(np.float64)
                - minus[np.arange(len(cols)), cols].astype(np.float64))
        tt = np.full(len(cols), t[r], np.int32)
        hp = oracle.forward(plus, tt, tau=tau, want=("entropy",))["entropy"]
        hm = oracle.forward(minus, tt, tau=tau, want=("entropy",))["entropy"]
        fd = (hp - hm) / step
        gr = oracle.backward_entropy(x[r:r + 1], None, None, np.ones(1, np.float32), tau=tau)[0]
        np.testing.assert_allclose(gr[cols], fd, rtol=0, atol=1e-8)


def test_entropy_grad_rows_sum_to_zero_and_reduce_to_logprob_grad(tiny):
    _, x, t, g = tiny
    h = np.random.default_rng(9).uniform(-1, 1, x.shape[0]).astype(np.float32)
    both = oracle.backward_entropy(x, t, g, h, tau=0.7)
    assert np.abs(both.sum(axis=1)).max() < x.shape[1] * 1e-16 * 8
    only_lp = oracle.backward_entropy(x, t, g, None, tau=0.7)
    np.testing.assert_array_equal(only_lp, oracle.backward(x, t, g, tau=0.7))
    zero = oracle.backward_entropy(x, t, np.zeros_like(g), np.zeros_like(h))
    assert np.all(zero == 0.0) and not np.any(np.signbit(zero))
    # uniform rows have zero entropy gradient (H is at its maximum)
    u = np.full((2, 64), 0.5, np.float32)
    gu = oracle.backward_entropy(u, None, None, np.ones(2, np.float32))
    assert np.abs(gu).max() < 1e-15


# ----------------------------------------------------------------------------- top-k KL
# Source: "[megatron] feat: add memory-efficient chunked top-k KL computation", commit
# text of the tail-aware top-k KL change ("What does this PR do?", "Design & Code Changes").


@pytest.fixture(scope="module")
def distill():
    w = W.get("distill_fp32_192x2048_k32")
    x = W.all_logits(w)[:48]
    idx, tlp = W.topk_payload_rows(w, np.arange(48))
    return x, idx, tlp


def _torch_kl(x, idx, tlp, mode, eps, tau):
    """The loss written independently in torch (fp64): log_softmax + gather."""
    xt = torch.from_numpy(x).double().requires_grad_(True)
    logq = torch.log_softmax(xt / float(np.float32(tau)), dim=1)
    lq = logq.gather(1, torch.from_numpy(idx).long())
    a = torch.from_numpy(tlp).double()
    p = a.exp()
    L = (p * (a - lq)).sum(1)
    if mode == oracle.KL_TRUNCATED:
        L = L.clamp_min(0.0)
    else:
        P, Q = p.sum(1), lq.exp().sum(1)
        pt, qt = 1 - P, (1 - Q).clamp_min(eps)
        L = L + torch.where(pt > 0, pt * (pt.log() - qt.log()), torch.zeros_like(pt))
    return xt, L


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_topk_kl_matches_torch_autograd(distill, mode, tau):
    x, idx, tlp = distill
    g = np.random.default_rng(2).uniform(-1, 1, x.shape[0]).astype(np.float32)
    o = oracle.topk_kl_forward(x, idx, tlp, mode, tau=tau)
    gr = oracle.topk_kl_backward(x, idx, tlp, mode, g, tau=tau)
    xt, L = _torch_kl(x, idx, tlp, mode, 1e-6, tau)
    np.testing.assert_allclose(o["loss"], L.detach().numpy(), rtol=0, atol=1e-12)
    (L * torch.from_numpy(g).double()).sum().backward()
    np.testing.assert_allclose(gr, xt.grad.numpy(), rtol=0, atol=1e-14)


def test_topk_kl_tail_gradient_closed_form(distill):
    """The page's analytic gradient: q_j - p_j inside the teacher top-k,
    q_j (P - Q) / (1 - Q) outside."""
    x, idx, tlp = distill
    g = np.ones(x.shape[0], np.float32)
    gr = oracle.topk_kl_backward(x, idx, tlp, oracle.KL_TAIL, g)
    o = oracle.topk_kl_forward(x, idx, tlp, oracle.KL_TAIL)
    z = x.astype(np.float64)
    q = np.exp(z - z.max(1, keepdims=True))
    q /= q.sum(1, keepdims=True)
    P, Q = o["teacher_mass"], o["student_mass"]
    want = q * ((P - Q) / (1 - Q))[:, None]
    rows = np.arange(x.shape[0])[:, None]
    want[rows, idx] = q[rows, idx] - np.exp(tlp.astype(np.float64))
    np.testing.assert_allclose(gr, want, rtol=0, atol=1e-14)


def test_topk_kl_finite_differences(distill):
    x, idx, tlp = distill
    V = x.shape[1]
    hh = 2.0 ** -10
    for mode in (0, 1):
        r = 5
        cols = np.unique(np.concatenate([idx[r, :4], np.linspace(0, V - 1, 12).astype(int)]))
        plus = np.repeat(x[r:r + 1], len(cols), axis=0)
        minus = plus.copy()
        plus[np.arange(len(cols)), cols] += np.float32(hh)
        minus[np.arange(len(cols)), cols] -= np.float32(hh)
        step = (plus[np.arange(len(cols)), cols].astype(np.float64)
                - minus[np.arange(len(cols)), cols].astype(np.float64))
        rep = lambda a: np.repeat(a[r:r + 1], len(cols), axis=0)
        lp = oracle.topk_kl_forward(plus, rep(idx), rep(tlp), mode)["loss"]
        lm = oracle.topk_kl_forward(minus, rep(idx), rep(tlp), mode)["loss"]
        gr = oracle.topk_kl_backward(x[r:r + 1], idx[r:r + 1], tlp[r:r + 1], mode,
                                     np.ones(1, np.float32))[0]
        np.testing.assert_allclose(gr[cols], (lp - lm) / step, rtol=0, atol=1e-8)


def test_topk_kl_full_vocabulary_and_lower_bound():
    """With K = V the tail-aware loss is the full forward KL; with K < V it is a
    non-negative lower bound of it, growing with K."""
    rng = np.random.default_rng(3)
    V = 512
    x = rng.standard_normal((6, V)).astype(np.float32)
    w = rng.exponential(size=(6, V)) ** 3
    pfull = w / w.sum(1, keepdims=True)
    z = x.astype(np.float64)
    logq = z - z.max(1, keepdims=True)
    logq -= np.log(np.exp(logq).sum(1, keepdims=True))
    kl_full = (pfull * (np.log(pfull) - logq)).sum(1)
    prev = np.zeros(6)
    for K in (8, 32, 128, V):
        order = np.argsort(-pfull, axis=1)[:, :K]
        tlp = np.log(np.take_along_axis(pfull, order, 1)).astype(np.float32)
        o = oracle.topk_kl_forward(x, order.astype(np.int32), tlp, oracle.KL_TAIL)
        assert np.all(o["loss"] >= -1e-12)
        assert np.all(o["loss"] <= kl_full + 1e-6)
        assert np.all(o["loss"] >= prev - 1e-6)  # more categories: the bound tightens
        prev = o["loss"]
    # K = V: equal to the full KL up to the fp32 rounding of the payload log-probs
    np.testing.assert_allclose(prev, kl_full, rtol=0, atol=1e-5)


def test_topk_kl_truncated_clamp_and_tail_guard():
    """A student that puts more top-k mass than the teacher (Q > P) makes the
    truncated sum negative: clamped to 0 with zero gradient.  A student with
    1 - Q below eps turns the tail term's gradient off."""
    V, K = 256, 8
    idx = np.arange(K, dtype=np.int32)[None].repeat(2, 0)
    tlp = np.log(np.full((2, K), 0.5 / K)).astype(np.float32)     # P = 0.5
    x = np.zeros((2, V), np.float32)
    x[0, :K] = 6.0                                                # Q ~ 0.93 > P
    x[1, :K] = 40.0                                               # 1 - Q ~ 1e-15 < eps
    tr = oracle.topk_kl_forward(x, idx, tlp, oracle.KL_TRUNCATED)
    assert tr["loss"][0] == 0.0 and tr["student_mass"][0] > 0.5
    gtr = oracle.topk_kl_backward(x, idx, tlp, oracle.KL_TRUNCATED, np.ones(2, np.float32))
    assert np.all(gtr[0] == 0.0)
    tl = oracle.topk_kl_forward(x, idx, tlp, oracle.KL_TAIL, tail_eps=1e-6)
    assert np.all(tl["loss"] > 0)
    gtl = oracle.topk_kl_backward(x, idx, tlp, oracle.KL_TAIL, np.ones(2, np.float32),
                                  tail_eps=1e-6)
    # guard active on row 1: the gradient is the truncated one, q_j P - p_j [j in T]
    z = x[1].astype(np.float64)
    q = np.exp(z - z.max())
    q /= q.sum()
    want = q * 0.5
    want[:K] -= 0.5 / K
    np.testing.assert_allclose(gtl[1], want, rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------- LM head
#
# The fused LM head ("[Bug] Training/log-prob forward materializes full-vocab fp32
# logits ...", maintainer comment: project only the loss-mask rows of the final
# hidden state; "[RL][Performance] Avoid full-vocabulary TP gather ...",
# "Alternatives considered": a fused LM-head / cross-entropy kernel): logits
# x = hidden @ weight^T, then the same logprob / lse / entropy.


def _bf16(a):
    return W.float32_to_bf16_bits(np.asarray(a, dtype=np.float32))


@pytest.fixture(scope="module")
def lm_tiny():
    w = W.get("lmhead_bf16_300x2000_d320")
    wt = W.lmhead_weight(w)
    return w, W.lmhead_hidden(w, weight=wt), wt, W.targets(w)


@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_lmhead_matches_torch_fp64(lm_tiny, tau):
    """torch fp64 matmul of the decoded operands, then torch's cross_entropy,
    logsumexp and Categorical entropy."""
    _, h, wt, t = lm_tiny
    rows = np.array([0, 5, 17, 255, 256, 299], np.int32)
    o = oracle.lmhead_forward(h, wt, t, tau=tau, rows=rows)
    hf = torch.from_numpy(W.bf16_bits_to_float32(h[rows])).double()
    wf = torch.from_numpy(W.bf16_bits_to_float32(wt)).double()
    z = (hf @ wf.T) / float(np.float32(tau))
    ce = torch.nn.functional.cross_entropy(z, torch.from_numpy(t[rows]).long(), reduction="none")
    np.testing.assert_allclose(o["logprob"], -ce.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(o["lse"], torch.logsumexp(z, 1).numpy(), rtol=0, atol=1e-11)
    ent = torch.distributions.Categorical(logits=z).entropy().numpy()
    np.testing.assert_allclose(o["entropy"], ent, rtol=0, atol=1e-11)


def test_lmhead_logits_exact_sums(lm_tiny):
    """Each logit equals the exactly rounded sum of its bf16 products (math.fsum)."""
    _, h, wt, _ = lm_tiny
    x = oracle.lmhead_logits(h[:3], wt[:40])
    hf = W.bf16_bits_to_float32(h[:3]).astype(np.float64)
    wf = W.bf16_bits_to_float32(wt[:40]).astype(np.float64)
    for i in range(3):
        for j in range(40):
            exact = math.fsum(hf[i] * wf[j])
            assert abs(x[i, j] - exact) <= 1e-12 * max(1.0, abs(exact))


def test_lmhead_onehot_hidden_reads_weight_column():
    """A hidden row c * e_k projects onto column k of the weight: the result equals
    the plain forward on the logits c * weight[:, k] (catches a transposed weight or
    a wrong hidden row)."""
    rng = np.random.default_rng(11)
    vocab, d = 37, 12
    wt = _bf16(rng.standard_normal((vocab, d)))
    ks = np.array([3, 0, 11, 7])
    h = np.zeros((4, d), np.float32)
    h[np.arange(4), ks] = [2.0, 0.5, 1.0, 4.0]
    t = np.array([5, 36, 0, 19], np.int32)
    o = oracle.lmhead_forward(_bf16(h), wt, t, tau=0.7)
    cols = W.bf16_bits_to_float32(wt)[:, ks].T * np.array([[2.0], [0.5], [1.0], [4.0]],
                                                           np.float32)
    ref = oracle.forward(cols.astype(np.float32), t, tau=0.7)
    for k in ("logprob", "lse", "entropy"):
        np.testing.assert_allclose(o[k], ref[k], rtol=0, atol=1e-13)


def test_lmhead_zero_weight_is_uniform():
    """All logits zero: logprob = -ln V, lse = ln V, entropy = ln V (to the rounding
    of a 1000-term double sum)."""
    vocab, d = 1000, 64
    h = _bf16(np.random.default_rng(2).standard_normal((5, d)))
    o = oracle.lmhead_forward(h, np.zeros((vocab, d), np.uint16), np.arange(5, dtype=np.int32))
    np.testing.assert_allclose(o["logprob"], -math.log(vocab), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o["lse"], math.log(vocab), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o["entropy"], math.log(vocab), rtol=0, atol=1e-12)


def test_lmhead_two_entries_closed_form():
    """V = 2: with D = (x_1 - x_0) / tau, logprob of entry 0 is -log(1 + e^D), of entry
    1 is -log(1 + e^-D), and the entropy is the binary entropy of sigmoid(D)."""
    rng = np.random.default_rng(5)
    d, tau = 24, 0.7
    wt = _bf16(rng.standard_normal((2, d)))
    h = _bf16(rng.standard_normal((6, d)))
    t = np.array([0, 1, 0, 1, 0, 1], np.int32)
    o = oracle.lmhead_forward(h, wt, t, tau=tau)
    hf = W.bf16_bits_to_float32(h).astype(np.float64)
    wf = W.bf16_bits_to_float32(wt).astype(np.float64)
    tf = float(np.float32(tau))
    for i in range(6):
        D = (math.fsum(hf[i] * wf[1]) - math.fsum(hf[i] * wf[0])) / tf
        lp = -math.log1p(math.exp(D)) if t[i] == 0 else -math.log1p(math.exp(-D))
        p1 = 1.0 / (1.0 + math.exp(-D))
        ent = -(p1 * math.log(p1) + (1 - p1) * math.log(1 - p1))
        x0 = math.fsum(hf[i] * wf[0]) / tf
        assert abs(o["logprob"][i] - lp) <= 1e-13
        assert abs(o["lse"][i] - (x0 + math.log1p(math.exp(D)))) <= 1e-13
        assert abs(o["entropy"][i] - ent) <= 1e-13


def test_lmhead_shift_invariance():
    """Adding one vector u to every weight row moves every logit by h . u: logprob
    and entropy stay, lse moves by (h . u) / tau.  Small integers keep the bf16
    operands and their sums exact."""
    rng = np.random.default_rng(8)
    vocab, d, tau = 300, 16, 0.7
    wi = rng.integers(-8, 9, size=(vocab, d)).astype(np.float32)
    u = rng.integers(-4, 5, size=d).astype(np.float32)
    hi = (rng.integers(-8, 9, size=(7, d)) / 8.0).astype(np.float32)
    t = rng.integers(0, vocab, size=7).astype(np.int32)
    a = oracle.lmhead_forward(_bf16(hi), _bf16(wi), t, tau=tau)
    b = oracle.lmhead_forward(_bf16(hi), _bf16(wi + u), t, tau=tau)
    shift = np.array([math.fsum(hi[i].astype(np.float64) * u) for i in range(7)])
    tf = float(np.float32(tau))
    np.testing.assert_allclose(b["logprob"], a["logprob"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["entropy"], a["entropy"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b["lse"] - a["lse"], shift / tf, rtol=0, atol=1e-12)


def test_lmhead_compact_rows_and_padding(lm_tiny):
    """A row subset gives the dense result at those rows, and columns past d (here
    NaN) are never read."""
    w, h, wt, t = lm_tiny
    rows = np.array([299, 3, 3, 128, 0], np.int32)
    dense = oracle.lmhead_forward(h, wt, t)
    hp = np.full((h.shape[0], w.hidden + 24), 0x7FC0, np.uint16)
    hp[:, : w.hidden] = h
    wp = np.full((wt.shape[0], w.hidden + 8), 0x7FC0, np.uint16)
    wp[:, : w.hidden] = wt
    comp = oracle.lmhead_forward(hp, wp, t, rows=rows, d=w.hidden)
    for k in ("logprob", "lse", "entropy"):
        np.testing.assert_array_equal(comp[k], dense[k][rows])


def test_lmhead_err_scale():
    """With every product positive, A_j equals the logit itself: err_scale is
    (x_t + max_j x_j) / tau."""
    rng = np.random.default_rng(3)
    vocab, d, tau = 50, 8, 0.7
    wt = _bf16(rng.uniform(0.1, 1.0, (vocab, d)))
    h = _bf16(rng.uniform(0.1, 1.0, (4, d)))
    t = np.array([1, 2, 3, 49], np.int32)
    o = oracle.lmhead_forward(h, wt, t, tau=tau, err_scale=True)
    x = oracle.lmhead_logits(h, wt)
    tf = float(np.float32(tau))
    np.testing.assert_allclose(o["err_scale"], (x[np.arange(4), t] + x.max(1)) / tf,
                               rtol=1e-14, atol=0)


def test_lmhead_rejects_bad_arguments(lm_tiny):
    _, h, wt, t = lm_tiny
    with pytest.raises(oracle.OracleError):
        oracle.lmhead_forward(h, wt, np.full_like(t, 2000))
    with pytest.raises(oracle.OracleError):
        oracle.lmhead_forward(h, wt, t, rows=np.array([300], np.int32))
    with pytest.raises(oracle.OracleError):
        oracle.lmhead_forward(h, wt, t, d=321)


# The blocked LM-head oracle (a float64 BLAS product per block of kept rows, then
# the definition) that lets the full-size GPU test check every kept row.


@pytest.mark.parametrize("tau", [1.0, 0.7])
@pytest.mark.parametrize("block", [1, 7, 256])
def test_lmhead_blocked_matches_torch_fp64(lm_tiny, tau, block):
    """torch fp64 matmul of the decoded operands, cross_entropy, logsumexp and
    Categorical entropy; any block size."""
    from oracle.lmhead_blocked import lmhead_forward_blocked
    _, h, wt, t = lm_tiny
    rows = np.array([0, 5, 17, 255, 256, 299, 5], np.int64)
    o = lmhead_forward_blocked(h, wt, t, tau=tau, rows=rows, block=block)
    hf = torch.from_numpy(W.bf16_bits_to_float32(h[rows])).double()
    wf = torch.from_numpy(W.bf16_bits_to_float32(wt)).double()
    z = (hf @ wf.T) / float(np.float32(tau))
    ce = torch.nn.functional.cross_entropy(z, torch.from_numpy(t[rows]).long(), reduction="none")
    np.testing.assert_allclose(o["logprob"], -ce.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(o["lse"], torch.logsumexp(z, 1).numpy(), rtol=0, atol=1e-11)
    ent = torch.distributions.Categorical(logits=z).entropy().numpy()
    np.testing.assert_allclose(o["entropy"], ent, rtol=0, atol=1e-11)


@pytest.mark.parametrize("lattice", [False, True])
def test_lmhead_blocked_matches_the_c_oracle(lattice):
    """Every row and the error scale agree with oracle.c's fixed-order sums (ragged
    hidden size, NaN padding past d, rows in any order with repeats)."""
    from oracle.lmhead_blocked import lmhead_forward_blocked
    w = W.scaled("lmhead_bf16_300x2000_d320", 300, 2000, lattice=lattice)
    wt = W.lmhead_weight(w)
    h = W.lmhead_hidden(w, weight=wt)
    t = W.targets(w)
    d = w.hidden - 3
    hp = np.full((h.shape[0], w.hidden + 5), 0x7FC0, np.uint16)
    hp[:, :d] = h[:, :d]
    wp = np.full((wt.shape[0], w.hidden + 8), 0x7FC0, np.uint16)
    wp[:, :d] = wt[:, :d]
    rows = np.concatenate([np.arange(299, -1, -1), [7, 7]])
    a = lmhead_forward_blocked(hp, wp, t, tau=0.7, rows=rows, d=d, block=64, err_scale=True)
    b = oracle.lmhead_forward(hp, wp, t, tau=0.7, rows=rows.astype(np.int32), d=d,
                              err_scale=True)
    for k in ("logprob", "lse", "entropy", "err_scale"):
        np.testing.assert_allclose(a[k], b[k], rtol=1e-12, atol=1e-11)


def test_lmhead_blocked_closed_form_and_bad_arguments():
    """Two vocabulary entries: lse = log(e^a + e^b) (the two-entry closed form), and
    row ids or targets outside their ranges are refused."""
    from oracle.lmhead_blocked import lmhead_forward_blocked
    h = _bf16(np.array([[1.0, 2.0], [0.5, -1.0]]))
    wt = _bf16(np.array([[1.0, 0.0], [0.0, 1.0]]))
    t = np.array([1, 0], np.int32)
    o = lmhead_forward_blocked(h, wt, t)
    x = np.array([[1.0, 2.0], [0.5, -1.0]])
    lse = np.log(np.exp(x).sum(1))
    np.testing.assert_allclose(o["lse"], lse, rtol=0, atol=1e-15)
    np.testing.assert_allclose(o["logprob"], x[np.arange(2), t] - lse, rtol=0, atol=1e-15)
    p = np.exp(x - lse[:, None])
    np.testing.assert_allclose(o["entropy"], -(p * np.log(p)).sum(1), rtol=0, atol=1e-15)
    with pytest.raises(IndexError):
        lmhead_forward_blocked(h, wt, np.array([2, 0], np.int32))
    with pytest.raises(IndexError):
        lmhead_forward_blocked(h, wt, t, rows=np.array([2]))
    with pytest.raises(ValueError):
        lmhead_forward_blocked(h, wt, t, d=3)
