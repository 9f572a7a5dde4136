"""Every call under HIP graph capture: a serving or training loop can record
the whole path once and replay it.

The library makes no allocation, host synchronization or memset of its own, so
a captured sequence must replay with the same bits as eager calls on the same
inputs.  Each graph is replayed several times with new inputs written eagerly
between the replays (and the eager reference run in between too), and every
replay is compared bit for bit with the eager result.  Shapes cover one-segment
rows, rows merged inside their workgroup, rows that take the workspace and the
merge launch, fp32 and ragged widths.
"""
import pytest
import torch

import vocab_wide_cross_amd as vwc
from gpu_util import DEV, log

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _same(a, b):
    return torch.equal(_bits(a.contiguous()), _bits(b.contiguous()))


def _capture(run):
    """Warm up on a side stream, then record run() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run()
    return graph, outs


def _check_replays(graph, outs, run, refill):
    for rep in range(REPLAYS):
        refill(rep)
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        ref = run()  # eager, same inputs
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, ref)):
            assert _same(a, b), f"replay {rep}: output {k} differs from the eager call"


@pytest.mark.parametrize("dtype,n,vocab", [("bf16", 384, 151936), ("bf16", 192, 248320),
                                           ("fp32", 64, 2048), ("fp32", 96, 70001)])
def test_logprob_path_replays_bitwise(dtype, n, vocab):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device=DEV).manual_seed(vocab + n)
    x = torch.empty(n, vocab, dtype=tdt, device=DEV)
    t = torch.empty(n, dtype=torch.int32, device=DEV)
    go = torch.empty(n, dtype=torch.float32, device=DEV)
    ho = torch.empty(n, dtype=torch.float32, device=DEV)
    mask = torch.empty(n, dtype=torch.uint8, device=DEV)
    idx = torch.arange(1, n, 3, dtype=torch.int32, device=DEV)  # fixed row set
    # the row-id list is written up to the device count only: one buffer for the
    # graph and the eager calls, so the entries past the count compare equal
    row_ids = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    count = torch.empty(1, dtype=torch.int32, device=DEV)
    go_r = torch.empty(idx.numel(), dtype=torch.float32, device=DEV)

    def refill(rep):
        x.copy_((torch.randn(n, vocab, device=DEV, generator=gen) * 3.0).to(tdt))
        t.copy_(torch.randint(0, vocab, (n,), device=DEV, generator=gen, dtype=torch.int32))
        go.copy_(torch.randn(n, device=DEV, generator=gen))
        go[::5] = 0.0
        ho.copy_(torch.rand(n, device=DEV, generator=gen) * 2 - 1)
        go_r.copy_(torch.randn(idx.numel(), device=DEV, generator=gen))
        mask.copy_((torch.rand(n, device=DEV, generator=gen) < 0.5).to(torch.uint8))

    def run():
        lp, lse, ent = vwc.selected_logprob_fwd(x, t, want=("logprob", "lse", "entropy"))
        g = vwc.logprob_entropy_bwd(x, t, lse, ent, grad_logprob=go, grad_entropy=ho)
        lp_r, lse_r, ent_r = vwc.selected_logprob_fwd_rows(x, t, idx,
                                                           want=("logprob", "lse", "entropy"))
        g_r = vwc.selected_logprob_bwd_rows(x, t, idx, lse_r, go_r)
        g_s = vwc.selected_logprob_bwd_rows(x, t, idx, lse_r, go_r,
                                            layout=vwc.VWC_GRAD_SCATTER)
        h = vwc.entropy(x)
        vwc.mask_to_index(mask, row_idx=row_ids, count=count)
        f_lp, f_lse, _, f_g = vwc.selected_logprob_fwd_bwd(x, t, go)
        e_lp, e_lse, e_ent, e_g = vwc.logprob_entropy_fwd_bwd(x, t, go, ho)
        return [lp, lse, ent, g, lp_r, lse_r, ent_r, g_r, g_s, h, row_ids, count, f_lp, f_lse, f_g,
                e_lp, e_lse, e_ent, e_g]

    refill(-1)
    graph, outs = _capture(run)
    log(f"{dtype} [{n}, {vocab}]: captured {len(outs)} outputs")
    _check_replays(graph, outs, run, refill)


def test_split_vocabulary_and_topk_kl_replay_bitwise():
    n, vocab, k, parts = 128, 248320, 64, 4
    tdt = torch.bfloat16
    gen = torch.Generator(device=DEV).manual_seed(5)
    x = torch.empty(n, vocab, dtype=tdt, device=DEV)
    t = torch.empty(n, dtype=torch.int32, device=DEV)
    gl = torch.empty(n, dtype=torch.float32, device=DEV)
    cols = torch.stack([torch.randperm(vocab, device=DEV, generator=gen)[:k] for _ in range(n)])
    cols = cols.to(torch.int32).contiguous()
    tlp = torch.empty(n, k, dtype=torch.float32, device=DEV)
    w = vocab // parts

    def refill(rep):
        x.copy_((torch.randn(n, vocab, device=DEV, generator=gen) * 3.0).to(tdt))
        t.copy_(torch.randint(0, vocab, (n,), device=DEV, generator=gen, dtype=torch.int32))
        gl.copy_(torch.randn(n, device=DEV, generator=gen))
        tlp.copy_(torch.log_softmax(torch.randn(n, k, device=DEV, generator=gen), dim=1) - 0.2)

    stacked = torch.empty(parts, n, 4, dtype=torch.float32, device=DEV)

    def run():
        for q in range(parts):
            vwc.vocab_partial(x[:, q * w:(q + 1) * w], q * w, targets=t, out=stacked[q])
        lp, lse, ent = vwc.partial_combine(stacked)
        outs = [stacked, lp, lse, ent]
        for mode in (vwc.VWC_KL_TRUNCATED, vwc.VWC_KL_TAIL):
            f = vwc.topk_kl_fwd(x, cols, tlp, mode=mode)
            g = vwc.topk_kl_bwd(x, cols, tlp, f, gl, mode=mode)
            outs += [f["loss"], f["lse"], g]
            f1, g1 = vwc.topk_kl_fwd_bwd(x, cols, tlp, gl, mode=mode)  # the one call
            outs += [f1["loss"], f1["teacher_mass"], f1["lse"], g1]
        return outs

    refill(-1)
    graph, outs = _capture(run)
    _check_replays(graph, outs, run, refill)


def test_lmhead_replays_bitwise():
    n, vocab, d = 300, 2000, 320
    gen = torch.Generator(device=DEV).manual_seed(9)
    hidden = torch.empty(n, d, dtype=torch.bfloat16, device=DEV)
    weight = torch.empty(vocab, d, dtype=torch.bfloat16, device=DEV)
    t = torch.empty(n, dtype=torch.int32, device=DEV)
    idx = torch.arange(0, n, 2, dtype=torch.int32, device=DEV)

    def refill(rep):
        hidden.copy_(torch.randn(n, d, device=DEV, generator=gen).to(torch.bfloat16))
        weight.copy_((torch.randn(vocab, d, device=DEV, generator=gen) * 0.05).to(torch.bfloat16))
        t.copy_(torch.randint(0, vocab, (n,), device=DEV, generator=gen, dtype=torch.int32))

    def run():
        a = vwc.lmhead_logprob_fwd(hidden, weight, t, want=("logprob", "lse", "entropy"))
        b = vwc.lmhead_logprob_fwd(hidden, weight, t, row_idx=idx, want=("logprob", "lse"))
        return [a[0], a[1], a[2], b[0], b[1]]

    refill(-1)
    graph, outs = _capture(run)
    _check_replays(graph, outs, run, refill)
