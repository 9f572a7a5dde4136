"""Host logic of bench.py: timing statistics, algorithmic bytes, the code digest
that gates recorded HBM traffic, the single-GPU guard and the CPU-baseline leg."""
import json
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_ms_stats():
    assert bench.ms_stats([3.0, 1.0, 2.0]) == {"ms": 2.0, "ms_median": 2.0, "ms_min": 1.0}
    st = bench.ms_stats([4.0, 1.0, 2.0, 3.0])
    assert st == {"ms": 2.5, "ms_median": 2.5, "ms_min": 1.0}


def test_alg_bytes_of_the_default_step():
    w = W.get(bench.DEFAULT_WORKLOAD)
    live = 5757
    fwd, bwd = bench.alg_bytes(w.n_rows, w.vocab, 2, 2, live, entropy=False)
    # logits + target id + (logprob, lse) per row
    assert fwd == 8192 * (248320 * 2 + 4 + 8)
    # every row: grad_out in, a bf16 gradient row out; live rows also read the
    # logits, the target and lse
    assert bwd == 8192 * (4 + 248320 * 2) + live * (248320 * 2 + 8)
    fwd_e, _ = bench.alg_bytes(w.n_rows, w.vocab, 2, 2, live, entropy=True)
    assert fwd_e == fwd + 8192 * 4


def test_code_digest_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("/* header */ int f(int x)   { return x + 1; }")
    c.write_text("int f(int x) { return x + 2; }")
    assert bench.code_digest(str(a)) == bench.code_digest(str(b))
    assert bench.code_digest(str(a)) != bench.code_digest(str(c))


def test_recorded_traffic_is_gated_by_the_code_digest():
    path = os.path.join(ROOT, "profiles", f"traffic_{bench.DEFAULT_WORKLOAD}.json")
    rec = json.load(open(path))
    key = "bwd_segment_kernel<0, 0, true, false, false>"
    got = bench.recorded_traffic([key])
    if rec["kernel_code_digest"] == bench.traffic_digest("vwc_kernels.hip"):
        assert got == rec["per_launch_bytes"][key]["total"]
    else:
        assert got is None
    assert bench.recorded_traffic(["no_such_kernel"]) is None
    # the digest of another kernel's sources never matches
    assert bench.recorded_traffic([key], source="vwc_lmhead.hip") is None


def test_traffic_digest_covers_launch_geometry(tmp_path):
    """A change to any file that sets a kernel's code or launch shape (segment
    sizes, block sizes, the host's segment choice) changes the digest."""
    for src in ("vwc_kernels.hip", "vwc_lmhead.hip"):
        assert {"vwc_internal.h", "vwc_lane.h", "vwc_api.cpp"} <= set(bench.TRAFFIC_SOURCES[src])
    files = []
    for k in range(3):
        f = tmp_path / f"f{k}.h"
        f.write_text(f"constexpr int a{k} = {k};")
        files.append(str(f))
    d0 = bench.code_digest(files)
    (tmp_path / "f2.h").write_text("constexpr int a2 = 7;")
    assert bench.code_digest(files) != d0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout and "--gpus 1" in r.stderr


def test_cpu_baseline_reports_all_threads_and_one():
    w = W.get("tiny_fp32_64x2048")
    out = bench.cpu_baseline(w, 0.3)
    assert out["kind"] == "oracle" and out["unit"] == "tokens/s"
    assert out["cores"] >= 1 and out["value"] > 0 and out["value_1core"] > 0
    assert "1 thread" in out["sample_1core"]
    import oracle
    assert oracle.num_threads() == out["cores"]  # the thread count is restored


def test_fit_line_recovers_a_line():
    xs = [512, 1024, 1536, 2001]
    slope, icpt = bench.fit_line(xs, [0.008 + 4.35e-5 * x for x in xs])
    assert abs(slope - 4.35e-5) < 1e-12 and abs(icpt - 0.008) < 1e-9
    # noise-free points off the line pull it by the least-squares amount
    slope, icpt = bench.fit_line([0, 1, 2], [0.0, 1.0, 0.0])
    assert slope == 0.0 and abs(icpt - 1.0 / 3.0) < 1e-15
