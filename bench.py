"""Benchmark: selected-token log-probabilities + entropy + backward on one MI355X.

One step = the hot path over one batch of seeded synthetic logits already
resident in HBM: the forward (logprob and lse of every row, one read of the
logits) and the backward with softmax recompute (bf16 gradient of every row;
rows whose incoming gradient is 0 are written as +0.0 without reading their
logits).  The forward that also returns the entropy (same single read) is timed
on its own as `fwd_entropy`; `--entropy-in-step` puts it in the step instead.

Default workload: bf16 logits [8192, 248320] ~ N(0, 3^2) with a +8 spike in
10% of rows, uniform targets, grad_out ~ U(-1, 1) set to 0 on 30% of rows.

Prints ONE JSON line.  `roofline` is for the dominant kernel (the backward):
algorithmic bytes per launch / its average duration from HIP events recorded
on the stream it runs on.  `cpu_baseline` times the fp64 CPU oracle (the
test-infrastructure reference, untuned) on a bounded sample of rows.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
DEFAULT_WORKLOAD = "spiked_bf16_8192x248320"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="the default is the measured step; the other workloads report their "
                         "own passes (compact rows, split vocabulary) in the same format")
    ap.add_argument("--entropy-in-step", action="store_true",
                    help="the step's forward also writes the entropy")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of the logits' size (for counter scaling)")
    ap.add_argument("--row-sweep", action="store_true",
                    help="loss-mask workloads: also time the compact forward on leading parts of "
                         "the row list (64 rows up to all), with a straight-line fit of time "
                         "against rows")
    ap.add_argument("--lmhead-order", default="",
                    help="LM-head workloads, for counter runs: instead of timing, run one call per "
                         "letter in this order, E with the entropy output, L without (e.g. ELLELEEL)")
    return ap.parse_args()


def alg_bytes(n_rows, vocab, esize, gsize, live_rows, entropy):
    """Algorithmic HBM bytes of one forward and one backward launch."""
    out_f = 4 * (3 if entropy else 2)
    fwd = n_rows * (vocab * esize + 4 + out_f)
    # every row: read g (4 B) and write V gradients; live rows also read logits,
    # the target and lse.
    bwd = n_rows * (4 + vocab * gsize) + live_rows * (vocab * esize + 8)
    return fwd, bwd


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, seconds):
    """Time the fp64 oracle (forward + gradient) over rows of the same workload:
    passes over all rows, in blocks of 128, until `seconds` of oracle time."""
    import numpy as np

    import oracle
    import workloads as W

    t_all = W.targets(w)
    g_all = W.grad_out(w)
    x = np.empty((w.n_rows, w.vocab), dtype=w.np_dtype)

    def sink(r0, blk):
        x[r0:r0 + blk.shape[0]] = blk

    W.fill_logits(w, sink, block_rows=256)

    def run(seconds, block):
        rows_done, elapsed = 0, 0.0
        while elapsed < seconds:
            for r0 in range(0, w.n_rows, block):
                rows = np.arange(r0, min(r0 + block, w.n_rows))
                t0 = time.perf_counter()
                oracle.forward(x[rows], t_all[rows])
                oracle.backward(x[rows], t_all[rows], g_all[rows])
                elapsed += time.perf_counter() - t0
                rows_done += rows.size
                if elapsed >= seconds:
                    break
        return rows_done, elapsed

    rows_done, elapsed = run(seconds, 128)
    # Input bytes the oracle consumes per row: the logits row (read by the
    # forward and again by the gradient, counted once) plus target and g.
    row_bytes = w.vocab * w.esize + 8
    out = {"value": rows_done / elapsed, "unit": "tokens/s", "cores": oracle.num_threads(),
           "kind": "oracle", "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
           "input_gbs": rows_done * row_bytes / elapsed / 1e9,
           "sample": f"{rows_done} rows of {w.name} in order, cycling over all {w.n_rows} rows "
                     f"(fwd logprob+lse+entropy and the fp64 gradient of each row), "
                     f"{elapsed:.1f} s of oracle time"}
    out.update(single_core(lambda sec: run(sec, 8), seconds))
    return out


def single_core(run, seconds):
    """The same oracle work on one thread, for a shorter time."""
    import oracle

    prev = oracle.set_num_threads(1)
    try:
        done, el = run(max(2.0, seconds / 3))
    finally:
        oracle.set_num_threads(prev)
    return {"value_1core": done / el, "sample_1core": f"{done} rows on 1 thread, {el:.1f} s"}


# Sources that fix a kernel's code or launch geometry (segment sizes, block
# shapes, the host's segment choice, the lane arithmetic).
TRAFFIC_SOURCES = {
    "vwc_kernels.hip": ["vwc_kernels.hip", "vwc_internal.h", "vwc_lane.h", "vwc_api.cpp"],
    "vwc_lmhead.hip": ["vwc_lmhead.hip", "vwc_internal.h", "vwc_lane.h", "vwc_api.cpp"],
}


def code_digest(paths):
    """SHA-256 over C/HIP sources with their comments and whitespace removed: it
    changes with the code, not with its comments."""
    import hashlib
    import re

    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = re.sub(r"\s+", " ", text).strip()
        h.update(text.encode() + b"\0")
    return h.hexdigest()


def traffic_digest(source="vwc_kernels.hip"):
    csrc = os.path.join(ROOT, "vocab_wide_cross_amd", "csrc")
    return code_digest([os.path.join(csrc, f) for f in TRAFFIC_SOURCES[source]])


def recorded_traffic(kernel_key, workload=DEFAULT_WORKLOAD, source="vwc_kernels.hip"):
    """Per-launch HBM bytes measured by rocprofv3 counters (see profiles/), valid only
    while the kernel code and launch geometry are the ones they were measured on."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        rec = json.load(open(path))
        digest = traffic_digest(source)
    except OSError:
        return None
    if rec.get("kernel_code_digest") != digest:
        return None
    total = 0
    for k in kernel_key:
        if k not in rec["per_launch_bytes"]:
            return None
        total += rec["per_launch_bytes"][k]["total"]
    return total


def ms_stats(samples):
    """Mean, median and minimum of per-step event times (ms)."""
    v = sorted(samples)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"ms": sum(v) / n, "ms_median": med, "ms_min": v[0]}


def time_passes(passes, steps, warmup, stream):
    """Run the passes in order `steps` times; per-pass event times (ms, one list
    per pass) from HIP events recorded on `stream`, and the wall-clock ms of one
    step."""
    import torch

    for _ in range(warmup):
        for _, fn, _ in passes:
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(passes) + 1)]
          for _ in range(steps)]
    wall0 = time.perf_counter()
    for k in range(steps):
        ev[k][0].record(stream)
        for j, (_, fn, _) in enumerate(passes):
            fn()
            ev[k][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3 / steps
    ms = [[e[j].elapsed_time(e[j + 1]) for e in ev] for j in range(len(passes))]
    return ms, wall


def row_sweep(args, w, x, t, idx, stream):
    """The compact forward (logprob, lse, entropy) on the first m entries of the
    row list, for m from 64 up to all of them, and a least-squares line through
    the points of 512 rows and more: its slope is the streaming rate, its
    intercept the time a launch spends outside steady streaming (start-up and
    the drain of its last rows)."""
    import torch

    import vocab_wide_cross_amd as vwc

    M = int(idx.numel())
    e = 2 if w.dtype == "bf16" else 4
    sizes = sorted({m for m in (64, 128, 256, 512, 768, 1024, 1536, 2048, 3072, 4096) if m < M}
                   | {M})
    lp, lse, ent = (torch.empty(M, device=x.device) for _ in range(3))
    ws = torch.empty(max(vwc.workspace_bytes(M, w.vocab, x.dtype), 1), dtype=torch.uint8,
                     device=x.device)
    passes = [(f"fwd_rows[{m}]",
               (lambda m=m: vwc.selected_logprob_fwd_rows(
                   x, t, idx[:m], w.tau, logprob=lp[:m], lse=lse[:m], entropy=ent[:m],
                   workspace=ws, stream=stream)), m * (w.vocab * e + 20)) for m in sizes]
    samples, _ = time_passes(passes, args.steps, args.warmup, stream)
    pts = []
    for (name, _, b), smp, m in zip(passes, samples, sizes):
        st = ms_stats(smp)
        pts.append({"rows": m, **st, "frac": b / (st["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS})
    fit = [p for p in pts if p["rows"] >= 512]
    out = {"points": pts}
    if len(fit) >= 2:
        slope, icpt = fit_line([p["rows"] for p in fit], [p["ms"] for p in fit])
        row_bytes = w.vocab * e + 20
        out["fit"] = {"intercept_us": icpt * 1e3, "us_per_row": slope * 1e3,
                      "streaming_frac": row_bytes / (slope * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return out


def fit_line(xs, ys):
    """Least-squares slope and intercept of ys against xs (at least two distinct xs)."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    slope = sum((a - mx) * (b - my) for a, b in zip(xs, ys)) / sum((a - mx) ** 2 for a in xs)
    return slope, my - slope * mx


def bench_other(args, w, x):
    """The other workloads' passes: compacted rows (loss-mask index list),
    packed compact forward + backward, split-vocabulary partials + merge."""
    import numpy as np
    import torch

    import vocab_wide_cross_amd as vwc
    import workloads as W

    dev = x.device
    stream = torch.cuda.current_stream(dev)
    N, V, e = w.n_rows, w.vocab, (2 if w.dtype == "bf16" else 4)
    t = torch.from_numpy(W.targets(w)).to(dev)
    g_all = W.grad_out(w)
    passes = []
    rows = N
    if w.mask != "none":
        mask = torch.from_numpy(W.loss_mask(w)).to(dev)
        idx_buf, cnt = vwc.mask_to_index(mask)
        M = int(cnt.item())
        idx = idx_buf[:M]
        rows = M
        passes.append(("mask_to_index", lambda: vwc.mask_to_index(mask, idx_buf, cnt, stream=stream),
                       N + 4 * M + 4))
        lp = torch.empty(M, device=dev)
        lse = torch.empty(M, device=dev)
        ent = torch.empty(M, device=dev)
        ws = torch.empty(max(vwc.workspace_bytes(M, V, x.dtype), 1), dtype=torch.uint8, device=dev)
        passes.append(("fwd_rows(logprob,lse,entropy)",
                       lambda: vwc.selected_logprob_fwd_rows(x, t, idx, w.tau, logprob=lp, lse=lse,
                                                             entropy=ent, workspace=ws,
                                                             stream=stream),
                       M * (V * e + 20)))
        if w.mask == "packed":
            gc = torch.from_numpy(g_all[W.row_index(w)]).to(dev)
            hc = torch.from_numpy(np.random.default_rng(8).uniform(-1, 1, M)
                                  .astype(np.float32)).to(dev)
            grad = torch.empty((M, V), dtype=x.dtype, device=dev)
            passes.append(("bwd_rows(compact)",
                           lambda: vwc.selected_logprob_bwd_rows(x, t, idx, lse, gc, w.tau,
                                                                 grad_logits=grad,
                                                                 layout=vwc.VWC_GRAD_COMPACT,
                                                                 stream=stream),
                           M * (2 * V * e + 16)))
            passes.append(("bwd_rows(logprob+entropy grads, compact)",
                           lambda: vwc.logprob_entropy_bwd_rows(x, t, idx, lse, ent, gc, hc,
                                                                w.tau, grad_logits=grad,
                                                                layout=vwc.VWC_GRAD_COMPACT,
                                                                stream=stream),
                           M * (2 * V * e + 24)))
    elif w.topk > 0:
        idx_h, tlp_h = W.topk_payload(w)
        idx = torch.from_numpy(idx_h).to(dev)
        tlp = torch.from_numpy(tlp_h).to(dev)
        K = w.topk
        g = torch.from_numpy(g_all).to(dev)
        ws = torch.empty(max(vwc.workspace_bytes(N, V, x.dtype), 1), dtype=torch.uint8,
                         device=dev)
        fwd = vwc.topk_kl_fwd(x, idx, tlp, vwc.VWC_KL_TAIL, workspace=ws)
        grad = torch.empty_like(x)
        passes.append(("topk_kl_fwd(tail, K=%d)" % K,
                       lambda: vwc._binding._lib.vwc_topk_kl_fwd(
                           vwc._binding._ptr(x), vwc._binding._dtype(x), N, V, V,
                           vwc._binding._ptr(idx), vwc._binding._ptr(tlp), K, vwc.VWC_KL_TAIL,
                           1e-6, float(w.tau), vwc._binding._ptr(fwd["loss"]),
                           vwc._binding._ptr(fwd["student_mass"]),
                           vwc._binding._ptr(fwd["teacher_mass"]),
                           vwc._binding._ptr(fwd["topk_sum"]), vwc._binding._ptr(fwd["lse"]),
                           vwc._binding._ptr(ws), ws.numel(), vwc._binding._stream(stream, x)),
                       N * (V * e + K * (8 + e) + 20)))
        passes.append(("topk_kl_bwd(tail, K=%d)" % K,
                       lambda: vwc.topk_kl_bwd(x, idx, tlp, fwd, g, vwc.VWC_KL_TAIL,
                                               grad_logits=grad, stream=stream),
                       N * (2 * V * e + K * (8 + 2 * e) + 20)))
        # The same forward + backward as one call (the loss weight known up front):
        # one read of the logits and the payload, one write of the gradient.
        passes.append(("topk_kl_fwd_bwd(tail, K=%d, one call)" % K,
                       lambda: vwc.topk_kl_fwd_bwd(x, idx, tlp, g, vwc.VWC_KL_TAIL,
                                                   temperature=float(w.tau), grad_logits=grad,
                                                   workspace=ws, stream=stream),
                       N * (2 * V * e + K * (8 + e) + 24)))
    elif w.n_slices > 1:
        k, vl = w.n_slices, V // w.n_slices
        parts = torch.empty((k, N, 4), dtype=torch.float32, device=dev)
        ws = torch.empty(max(vwc.workspace_bytes(N, vl, x.dtype), 1), dtype=torch.uint8,
                         device=dev)
        for q in range(k):
            passes.append((f"vocab_partial[{q}]",
                           (lambda q=q: vwc.vocab_partial(x[:, q * vl:(q + 1) * vl], q * vl, t,
                                                          None, w.tau, out=parts[q], workspace=ws,
                                                          stream=stream)),
                           N * (vl * e + 4 + 16)))
        lp = torch.empty(N, device=dev)
        lse = torch.empty(N, device=dev)
        ent = torch.empty(N, device=dev)
        passes.append(("partial_combine",
                       lambda: vwc.partial_combine(parts, w.tau, lp, lse, ent, stream=stream),
                       N * (k * 16 + 12)))
    else:
        g = torch.from_numpy(g_all).to(dev)
        lp = torch.empty(N, device=dev)
        lse = torch.empty(N, device=dev)
        ent = torch.empty(N, device=dev)
        grad = torch.empty_like(x)
        passes.append(("fwd(logprob,lse,entropy)",
                       lambda: vwc.selected_logprob_fwd(x, t, w.tau, logprob=lp, lse=lse,
                                                        entropy=ent, stream=stream),
                       N * (V * e + 16)))
        passes.append(("bwd", lambda: vwc.selected_logprob_bwd(x, t, lse, g, w.tau,
                                                               grad_logits=grad, stream=stream),
                       N * (2 * V * e + 12)))
    samples, wall = time_passes(passes, args.steps, args.warmup, stream)
    per_pass = []
    ms = []
    for (name, _, b), smp in zip(passes, samples):
        st = ms_stats(smp)
        m = st["ms"]
        ms.append(m)
        per_pass.append({"pass": name, **st, "bytes_alg": b,
                         "gbs_alg": b / (m * 1e-3) / 1e9,
                         "frac": b / (m * 1e-3) / 1e9 / HBM_PEAK_GBS})
    total_b = sum(p[2] for p in passes)
    total_ms = sum(ms)
    out = {
        "metric": f"rows/s of the {w.name} passes", "value": rows / (wall * 1e-3),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {"workload": w.name, "rows": N, "rows_computed": rows, "vocab": V,
                   "temperature": w.tau},
        "passes": per_pass,
        "all_passes": {"ms": total_ms, "gbs_alg": total_b / (total_ms * 1e-3) / 1e9,
                       "frac": total_b / (total_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
    }
    if args.row_sweep and w.mask != "none":
        out["row_sweep"] = row_sweep(args, w, x, t, idx, stream)
    if w.n_slices > 1:
        sl, sls, sen = (torch.empty(N, device=dev) for _ in range(3))
        wsf = torch.empty(max(vwc.workspace_bytes(N, V, x.dtype), 1), dtype=torch.uint8,
                          device=dev)
        smp1, _ = time_passes([("single", lambda: vwc.selected_logprob_fwd(
            x, t, w.tau, logprob=sl, lse=sls, entropy=sen, workspace=wsf, stream=stream), 0)],
            args.steps, args.warmup, stream)
        st1 = ms_stats(smp1[0])
        b1 = N * (V * e + 16)
        out["single_pass_fwd"] = {**st1, "gbs_alg": b1 / (st1["ms"] * 1e-3) / 1e9,
                                  "frac": b1 / (st1["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return out


def lmhead_cpu_baseline(w, h, wt, tg, rows, seconds):
    """The fp64 oracle on kept rows of the same inputs, one row at a time (its own
    OpenMP over vocabulary columns), until `seconds` have passed."""
    import numpy as np

    import oracle

    sel = np.random.default_rng(11).permutation(rows.size)

    def run(seconds):
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds and done < sel.size:
            r = rows[sel[done: done + 1]]
            oracle.lmhead_forward(h, wt, tg, rows=r)
            done += 1
        return done, time.perf_counter() - t0

    done, el = run(seconds)
    out = {"value": done / el, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
           "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
           # operand bytes one kept row needs: its hidden row and the whole weight
           "input_gbs": done * (w.hidden * 2 + w.vocab * w.hidden * 2) / el / 1e9,
           "sample": f"{done} kept rows of {w.name} in random order (fp64 projection of each "
                     f"row against all {w.vocab} weight rows, then logprob+lse+entropy), "
                     f"{el:.1f} s of oracle time"}
    out.update(single_core(run, seconds))
    return out


def bench_lmhead(args, w):
    """Fused LM head: logprob / lse (and entropy) of the kept hidden rows without
    logits.  Timed beside it, as context: torch's bf16 GEMM (hipBLASLt) writing the
    bf16 logits followed by this library's forward over them."""
    import numpy as np
    import torch

    import vocab_wide_cross_amd as vwc
    import workloads as W

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    t0 = time.time()
    wt_h = W.lmhead_weight(w)
    h_h = W.lmhead_hidden(w, weight=wt_h)
    tg_h = W.targets(w)
    rows_h = W.row_index(w)
    wt = torch.from_numpy(wt_h.view(np.int16)).to(dev).view(torch.bfloat16)
    h = torch.from_numpy(h_h.view(np.int16)).to(dev).view(torch.bfloat16)
    tg = torch.from_numpy(tg_h).to(dev)
    rows = torch.from_numpy(rows_h).to(dev)
    M, V, d = rows_h.size, w.vocab, w.hidden
    ws = torch.empty(vwc.lmhead_workspace_bytes(M, V, d), dtype=torch.uint8, device=dev)
    lp, lse, ent = (torch.empty(M, device=dev) for _ in range(3))
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    flops = 2.0 * M * V * d
    passes = [
        ("lmhead_fwd(logprob,lse)",
         lambda: vwc.lmhead_logprob_fwd(h, wt, tg, rows, w.tau, logprob=lp, lse=lse,
                                        workspace=ws, stream=stream), flops),
        ("lmhead_fwd(logprob,lse,entropy)",
         lambda: vwc.lmhead_logprob_fwd(h, wt, tg, rows, w.tau, logprob=lp, lse=lse,
                                        entropy=ent, workspace=ws, stream=stream), flops),
    ]
    samples, wall = time_passes(passes, args.steps, args.warmup, stream)
    stats = [ms_stats(smp) for smp in samples]
    ms = [st["ms"] for st in stats]
    per_pass = [{"pass": n, **st, "tflops": f / (st["ms"] * 1e-3) / 1e12,
                 "frac": f / (st["ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
                for (n, _, f), st in zip(passes, stats)]
    # Context: the unfused route materialises bf16 logits [M, V] with hipBLASLt.
    hc = h[rows.long()].contiguous()
    logits = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
    ws2 = torch.empty(max(vwc.workspace_bytes(M, V, logits.dtype), 1), dtype=torch.uint8,
                      device=dev)
    unf = [("gather+torch_bf16_gemm", lambda: torch.matmul(h[rows.long()], wt.T, out=logits), flops),
           ("fwd_over_logits", lambda: vwc.selected_logprob_fwd(logits, tg[rows.long()], w.tau,
                                                                logprob=lp, lse=lse, workspace=ws2,
                                                                stream=stream), 0)]
    usmp, _ = time_passes(unf, max(3, args.steps // 4), 1, stream)
    ums = [ms_stats(smp)["ms"] for smp in usmp]
    del logits, hc, ws2
    # The box's practical bf16 rate: hipBLASLt on a large square product (the
    # MFMA peak assumes a clock that dense MFMA work does not hold).
    sq = 16384
    a_sq = torch.randn((sq, sq), device=dev).to(torch.bfloat16)
    b_sq = torch.randn((sq, sq), device=dev).to(torch.bfloat16)
    c_sq = torch.empty((sq, sq), dtype=torch.bfloat16, device=dev)
    ssmp, _ = time_passes([("square", lambda: torch.matmul(a_sq, b_sq, out=c_sq), 0)],
                          max(3, args.steps // 4), 1, stream)
    sq_ms = ms_stats(ssmp[0])["ms"]
    del a_sq, b_sq, c_sq
    out = {
        "metric": f"kept rows/s of the fused LM head ({w.name})",
        "value": M / (ms[0] * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms[0], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {"workload": w.name, "hidden_rows": w.n_rows, "kept_rows": M, "vocab": V,
                   "hidden": d, "temperature": w.tau},
        "passes": per_pass,
        "roofline": {"bound": "mfma", "kernel": "lmhead_fwd_kernel",
                     "achieved": flops / (ms[0] * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops / (ms[0] * 1e-3) / 1e12 /
                     MFMA_BF16_PEAK_TFLOPS,
                     "traffic": recorded_traffic(["lmhead_fwd_kernel<false, false>"], w.name,
                                                 "vwc_lmhead.hip"),
                     "avg_launch_ms": ms[0],
                     "flops_alg_per_launch": flops,
                     "note": "launch = row gather + MFMA kernel + segment merge (HIP events)"},
        "unfused_context": {"gemm_ms": ums[0], "gemm_tflops": flops / (ums[0] * 1e-3) / 1e12,
                            "fwd_over_logits_ms": ums[1], "total_ms": ums[0] + ums[1],
                            "logits_bytes": M * V * 2},
        "square_gemm_context": {"shape": [sq, sq, sq], "ms": sq_ms,
                                "tflops": 2.0 * sq ** 3 / (sq_ms * 1e-3) / 1e12,
                                "lmhead_over_square": (flops / (ms[0] * 1e-3)) /
                                                      (2.0 * sq ** 3 / (sq_ms * 1e-3))},
    }
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = lmhead_cpu_baseline(w, h_h, wt_h, tg_h, rows_h, args.cpu_seconds)
        cpu["gpu_over_oracle"] = out["value"] / cpu["value"]
        out["cpu_baseline"] = cpu
    import hashlib
    out["inputs_sha256"] = {"hidden": hashlib.sha256(h_h.tobytes()).hexdigest(),
                            "weight": hashlib.sha256(wt_h.tobytes()).hexdigest(),
                            "targets": hashlib.sha256(tg_h.tobytes()).hexdigest(),
                            "row_idx": hashlib.sha256(rows_h.tobytes()).hexdigest()}
    return out


def lmhead_order(args, w):
    """One LM-head call per letter of args.lmhead_order (E: logprob, lse and entropy;
    L: logprob and lse), each synchronized, on the workload's inputs; for counter
    runs that attribute per-launch figures to an instance and a position."""
    import numpy as np
    import torch

    import vocab_wide_cross_amd as vwc
    import workloads as W

    dev = torch.device("cuda:0")
    wt_h = W.lmhead_weight(w)
    h_h = W.lmhead_hidden(w, weight=wt_h)
    wt = torch.from_numpy(wt_h.view(np.int16)).to(dev).view(torch.bfloat16)
    h = torch.from_numpy(h_h.view(np.int16)).to(dev).view(torch.bfloat16)
    tg = torch.from_numpy(W.targets(w)).to(dev)
    rows = torch.from_numpy(W.row_index(w)).to(dev)
    M = rows.numel()
    ws = torch.empty(vwc.lmhead_workspace_bytes(M, w.vocab, w.hidden), dtype=torch.uint8,
                     device=dev)
    lp, lse, ent = (torch.empty(M, device=dev) for _ in range(3))
    for k, e in enumerate(args.lmhead_order):
        if e not in "EL":
            raise SystemExit(f"--lmhead-order takes E and L, not {e!r}")
        vwc.lmhead_logprob_fwd(h, wt, tg, rows, w.tau, logprob=lp, lse=lse,
                               entropy=ent if e == "E" else None, workspace=ws)
        torch.cuda.synchronize()
    print(json.dumps({"lmhead_order": args.lmhead_order, "workload": w.name}))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU per process; --gpus must be 1",
                          "n_gpus": args.gpus}))
        print("bench.py: only --gpus 1 is supported (the measured path is one GPU's share)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import vocab_wide_cross_amd as vwc
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.get(args.workload)
    if w.hidden > 0:
        if args.lmhead_order:
            lmhead_order(args, w)
            return
        print(json.dumps(bench_lmhead(args, w)))
        return
    esize = 2 if w.dtype == "bf16" else 4
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    if args.copy_calibration:
        n = w.n_rows * w.vocab * esize
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return

    # Inputs, generated on the host in row blocks (in row order) and left
    # resident in HBM; SHA-256 of each buffer's bytes as uploaded.
    import hashlib

    t0 = time.time()
    x = torch.empty((w.n_rows, w.vocab), dtype=dt, device=dev)
    x_hash = hashlib.sha256()

    def sink(r0, blk):
        x_hash.update(np.ascontiguousarray(blk).data)
        src = torch.from_numpy(blk.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" \
            else torch.from_numpy(blk)
        x[r0:r0 + blk.shape[0]].copy_(src.to(dev))

    W.fill_logits(w, sink, block_rows=512)
    t_host = W.targets(w)
    g_host = W.grad_out(w)
    inputs_sha256 = {"logits": x_hash.hexdigest(),
                     "targets": hashlib.sha256(t_host.tobytes()).hexdigest(),
                     "grad_out": hashlib.sha256(g_host.tobytes()).hexdigest()}
    if w.mask != "none":
        inputs_sha256["loss_mask"] = hashlib.sha256(W.loss_mask(w).tobytes()).hexdigest()
    if w.name != DEFAULT_WORKLOAD:
        torch.cuda.synchronize()
        print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
        out = bench_other(args, w, x)
        out["inputs_sha256"] = inputs_sha256
        print(json.dumps(out))
        return
    targets = torch.from_numpy(t_host).to(dev)
    grad_out = torch.from_numpy(g_host).to(dev)
    live = int((g_host != 0).sum())
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    want_ent = args.entropy_in_step
    lp = torch.empty(w.n_rows, dtype=torch.float32, device=dev)
    lse = torch.empty_like(lp)
    ent_buf = torch.empty_like(lp)
    ent = ent_buf if want_ent else None
    grad = torch.empty((w.n_rows, w.vocab), dtype=dt, device=dev)
    ws_bytes = vwc.workspace_bytes(w.n_rows, w.vocab, dt)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        vwc.selected_logprob_fwd(x, targets, w.tau, logprob=lp, lse=lse, entropy=ent,
                                 workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        vwc.selected_logprob_bwd(x, targets, lse, grad_out, w.tau, grad_logits=grad,
                                 stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    fwd_st = ms_stats([e[0].elapsed_time(e[1]) for e in events])
    bwd_st = ms_stats([e[1].elapsed_time(e[2]) for e in events])
    fwd_avg = fwd_st["ms"]
    bwd_avg = bwd_st["ms"]
    ms_per_step = wall * 1e3 / args.steps
    fwd_b, bwd_b = alg_bytes(w.n_rows, w.vocab, esize, esize, live, want_ent)
    fwd_e_b, _ = alg_bytes(w.n_rows, w.vocab, esize, esize, live, True)

    # The forward with the entropy output as well, timed on its own.
    ent_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                  for _ in range(args.steps)]
    for k in range(args.steps):
        ent_events[k][0].record(stream)
        vwc.selected_logprob_fwd(x, targets, w.tau, logprob=lp, lse=lse, entropy=ent_buf,
                                 workspace=ws, stream=stream)
        ent_events[k][1].record(stream)
    torch.cuda.synchronize()
    fwd_e_st = ms_stats([e[0].elapsed_time(e[1]) for e in ent_events])
    fwd_e_avg = fwd_e_st["ms"]

    def gbs(b, ms):
        return b / (ms * 1e-3) / 1e9

    # The same step as one call (vwc_selected_logprob_fwd_bwd): the loss weight
    # is known up front here, so each row is read once and kept on chip between
    # the reduction and the gradient.  Timed on its own; not the step above.
    fused_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                for _ in range(args.steps)]
    for _ in range(args.warmup):
        vwc.selected_logprob_fwd_bwd(x, targets, grad_out, w.tau, logprob=lp, lse=lse,
                                     grad_logits=grad, workspace=ws, stream=stream)
    for k in range(args.steps):
        fused_ev[k][0].record(stream)
        vwc.selected_logprob_fwd_bwd(x, targets, grad_out, w.tau, logprob=lp, lse=lse,
                                     grad_logits=grad, workspace=ws, stream=stream)
        fused_ev[k][1].record(stream)
    torch.cuda.synchronize()
    fused_st = ms_stats([e[0].elapsed_time(e[1]) for e in fused_ev])
    # one read of the logits, grad_out and targets; logprob, lse and the gradient written
    fused_b = w.n_rows * (w.vocab * esize + 8) + w.n_rows * (8 + w.vocab * esize)

    # With the entropy term as well (d(g logprob + h H)/dx): the fused backward after
    # the forward with the entropy, and the same as one call
    # (vwc_logprob_entropy_fwd_bwd).  h ~ U(-1, 1) with 20 % zeros.
    hgen = torch.Generator(device=dev).manual_seed(8)
    h_out = torch.rand(w.n_rows, device=dev, generator=hgen) * 2 - 1
    h_out[torch.rand(w.n_rows, device=dev, generator=hgen) < 0.2] = 0

    def time_calls(fn):
        for _ in range(args.warmup):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for k in range(args.steps):
            ev[k][0].record(stream)
            fn()
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        return ms_stats([e[0].elapsed_time(e[1]) for e in ev])

    ent_bwd_st = time_calls(lambda: vwc.logprob_entropy_bwd(
        x, targets, lse, ent_buf, grad_out, h_out, w.tau, grad_logits=grad, stream=stream))
    ent_one_st = time_calls(lambda: vwc.logprob_entropy_fwd_bwd(
        x, targets, grad_out, h_out, w.tau, logprob=lp, lse=lse, entropy=ent_buf,
        grad_logits=grad, workspace=ws, stream=stream))
    live_e = int(((grad_out != 0) | (h_out != 0)).sum().item())
    # every row reads g and h and writes its gradient; live rows also read the logits,
    # the target, lse and the entropy
    ent_bwd_b = w.n_rows * (8 + w.vocab * esize) + live_e * (w.vocab * esize + 12)
    # one read of the logits, targets, g and h; logprob, lse, entropy and the gradient written
    ent_one_b = w.n_rows * (w.vocab * esize + 12) + w.n_rows * (12 + w.vocab * esize)

    # Dominant kernel: the launch with the longest average duration.  The
    # backward is one kernel; the forward is the segment kernel plus a small
    # merge kernel (its events bracket both).
    if bwd_avg >= fwd_avg:
        dom = ("bwd_segment_kernel", bwd_b, bwd_avg, ["bwd_segment_kernel<0, 0, true, false, false>"])
    else:
        dom = ("fwd_segment_kernel+combine_kernel", fwd_b, fwd_avg,
               ["fwd_segment_kernel<0, true, false, false>", "combine_kernel"])
    traffic = recorded_traffic(dom[3]) if w.name == "spiked_bf16_8192x248320" else None

    result = {
        "metric": "tokens/s + achieved HBM GB/s (fwd, fwd+bwd) at N=8192 V=248320 bf16",
        "value": w.n_rows / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {"workload": w.name, "rows": w.n_rows, "vocab": w.vocab,
                   "temperature": w.tau, "live_grad_rows": live,
                   "step": "fwd(logprob,lse" + (",entropy" if want_ent else "") +
                           ") + bwd(" + w.dtype + " grad)"},
        "fwd": {**fwd_st, "tokens_per_s": w.n_rows / (fwd_avg * 1e-3),
                "gbs_alg": gbs(fwd_b, fwd_avg), "frac": gbs(fwd_b, fwd_avg) / HBM_PEAK_GBS,
                "bytes_alg": fwd_b},
        "fwd_entropy": {**fwd_e_st, "tokens_per_s": w.n_rows / (fwd_e_avg * 1e-3),
                        "gbs_alg": gbs(fwd_e_b, fwd_e_avg),
                        "frac": gbs(fwd_e_b, fwd_e_avg) / HBM_PEAK_GBS, "bytes_alg": fwd_e_b},
        "bwd": {**bwd_st, "tokens_per_s": w.n_rows / (bwd_avg * 1e-3),
                "gbs_alg": gbs(bwd_b, bwd_avg), "frac": gbs(bwd_b, bwd_avg) / HBM_PEAK_GBS,
                "bytes_alg": bwd_b},
        "fwd_bwd": {"ms": fwd_avg + bwd_avg,
                    "tokens_per_s": w.n_rows / ((fwd_avg + bwd_avg) * 1e-3),
                    "gbs_alg": gbs(fwd_b + bwd_b, fwd_avg + bwd_avg),
                    "frac": gbs(fwd_b + bwd_b, fwd_avg + bwd_avg) / HBM_PEAK_GBS},
        "fused_fwd_bwd": {**fused_st, "tokens_per_s": w.n_rows / (fused_st["ms"] * 1e-3),
                          "gbs_alg": gbs(fused_b, fused_st["ms"]),
                          "frac": gbs(fused_b, fused_st["ms"]) / HBM_PEAK_GBS,
                          "bytes_alg": fused_b,
                          "note": "one call, loss weight known before the forward"},
        "entropy_grad": {
            "live_rows": live_e,
            "bwd": {**ent_bwd_st, "gbs_alg": gbs(ent_bwd_b, ent_bwd_st["ms"]),
                    "frac": gbs(ent_bwd_b, ent_bwd_st["ms"]) / HBM_PEAK_GBS,
                    "bytes_alg": ent_bwd_b},
            "fwd_bwd": {"ms": fwd_e_avg + ent_bwd_st["ms"],
                        "tokens_per_s": w.n_rows / ((fwd_e_avg + ent_bwd_st["ms"]) * 1e-3)},
            "one_call": {**ent_one_st, "tokens_per_s": w.n_rows / (ent_one_st["ms"] * 1e-3),
                         "gbs_alg": gbs(ent_one_b, ent_one_st["ms"]),
                         "frac": gbs(ent_one_b, ent_one_st["ms"]) / HBM_PEAK_GBS,
                         "bytes_alg": ent_one_b},
            "note": "loss g logprob + h entropy, h ~ U(-1,1) with 20% zeros: forward with the "
                    "entropy then the fused backward, against the same as one call"},
        "roofline": {"bound": "hbm", "kernel": dom[0],
                     "achieved": gbs(dom[1], dom[2]), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs(dom[1], dom[2]) / HBM_PEAK_GBS, "traffic": traffic,
                     "avg_launch_ms": dom[2], "bytes_alg_per_launch": dom[1]},
    }
    result["inputs_sha256"] = inputs_sha256
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_seconds)
        # GPU step throughput over the oracle's, both in rows/s of the same work
        # (forward + gradient of each row).
        cpu["gpu_over_oracle"] = result["value"] / cpu["value"]
        result["cpu_baseline"] = cpu
    print(json.dumps(result))


if __name__ == "__main__":
    main()
