"""The oracle pins must catch plausible mistakes.  Each case plants one mistake in a
private copy of oracle.c (on the CPU only), builds it, and runs the pin suite
against it in a subprocess: the suite must fail."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, mutated text, pin tests to run)
MUTATIONS = [
    ("entropy sign", "H -= p_times(p, z - LSE);", "H += p_times(p, z - LSE);", "entropy"),
    ("tau dropped on the target", "double zt = logit_at(logits, dtype, ld, r, targets[r]) / tau;",
     "double zt = logit_at(logits, dtype, ld, r, targets[r]);", "logprob or temperature"),
    ("max dropped from LSE", "double LSE = M + log(S);\n            if (lse) lse[i] = LSE;",
     "double LSE = log(S);\n            if (lse) lse[i] = LSE;", "logprob"),
    ("gradient sign", "gi[j] = g * (onehot - p) / tau;", "gi[j] = g * (p - onehot) / tau;",
     "grad"),
    ("gradient without tau", "gi[j] = g * (onehot - p) / tau;", "gi[j] = g * (onehot - p);",
     "grad"),
    ("combine drops the shift term", "W += f * (pw[q * m + i] + d * ps[q * m + i]);",
     "W += f * pw[q * m + i];", "vocab_chunks or split4"),
    # (a transposed read of only the maxima would be harmless: the merge is exact for
    # any reference point, so the planted mistake transposes the sums)
    ("combine reads partial sums transposed", "S += ps[q * m + i] * f;",
     "S += ps[i * k + q] * f;", "vocab_chunks or split4"),
    ("bf16 decode off by one bit", "uint32_t w = ((uint32_t)bits) << 16;",
     "uint32_t w = ((uint32_t)bits) << 15;", "sampled_rows"),
    ("target read by output index", "double zt = logit_at(logits, dtype, ld, r, targets[r]) / tau;",
     "double zt = logit_at(logits, dtype, ld, r, targets[i]) / tau;", "compact or chunks or errors"),
    ("entropy gradient sign of H",
     "gi[j] = (g * (onehot - p) - h * p_times(p, z - LSE + H)) / tau;",
     "gi[j] = (g * (onehot - p) - h * p_times(p, z - LSE - H)) / tau;", "entropy_grad"),
    # 0 log 0 = 0 for -inf logits (masked vocabulary entries)
    ("zero-probability term kept as 0 * inf", "return p == 0.0 ? 0.0 : p * a;", "return p * a;",
     "minus_inf"),
    ("exp of -inf minus -inf", "return z == -INFINITY ? 0.0 : exp(z - M);",
     "return exp(z - M);", "minus_inf"),
    ("combine keeps an empty slice", "if (ps[q * m + i] == 0.0) continue;", "/* kept */",
     "minus_inf"),
    ("tail mass from the student", "double pt = P < 1.0 ? 1.0 - P : 0.0;",
     "double pt = Q < 1.0 ? 1.0 - Q : 0.0;", "topk"),
    ("truncated clamp dropped", "if (L < 0.0) L = 0.0; /* clamp_min(0) of the truncated objective */",
     "/* no clamp */", "topk"),
    ("bf16 rounding ties away", "double r = rint(v / q) * q;", "double r = round(v / q) * q;",
     "bf16"),
    # (a slice that also claimed the first column past its end would read that same
    # logit, which the merge's max leaves unchanged, so the case drops the first one)
    ("slice misses its first column", "if (t >= v_start && t < v_start + v_local)",
     "if (t > v_start && t < v_start + v_local)", "vocab_chunks or split4 or slice"),
    ("slice target read at the global column",
     "pt[i] = logit_at(logits_slice, dtype, ld, r, t - v_start) / tau;",
     "pt[i] = logit_at(logits_slice, dtype, ld, r, t) / tau;", "vocab_chunks or split4 or slice"),
    ("combine takes the last slice's target", "if (pt && pt[q * m + i] > T) T = pt[q * m + i];",
     "if (pt) T = pt[q * m + i];", "vocab_chunks or split4 or slice"),
    ("KL gradient without tau", "gi[j] = g * d / tau;", "gi[j] = g * d;", "topk"),
    ("KL d log q sign", "double dlogq = (idx[n] == j ? 1.0 : 0.0) - qj;",
     "double dlogq = qj - (idx[n] == j ? 1.0 : 0.0);", "topk"),
    ("KL tail term sign", "d += dl_dlogqt * (-(qj * in_t - qj * Q) / (1.0 - Q));",
     "d += dl_dlogqt * ((qj * in_t - qj * Q) / (1.0 - Q));", "topk"),
    ("KL tail guard inverted", "if (mode == 1 && 1.0 - Q >= tail_eps)",
     "if (mode == 1 && 1.0 - Q < tail_eps)", "topk"),
    ("KL clamped row keeps its gradient",
     "int row_dead = (mode == 0 && Lraw < 0.0) || g == 0.0;", "int row_dead = g == 0.0;", "topk"),
    ("LM head reads the weight transposed",
     "double p = decode_bf16(h[k]) * decode_bf16(w[k]);",
     "double p = decode_bf16(h[k]) * decode_bf16(weight[k * ldw + j]);", "lmhead"),
    ("LM head hidden row by output index", "const uint16_t *h = hidden + row_of(rows, i) * ldh;",
     "const uint16_t *h = hidden + i * ldh;", "lmhead"),
    ("LM head drops the last hidden column", "for (int64_t k = 0; k < d; ++k) {",
     "for (int64_t k = 0; k + 1 < d; ++k) {", "lmhead"),
    ("LM head target of the output index",
     "sub_targets[i] = targets ? targets[sub_rows[i]] : 0;",
     "sub_targets[i] = targets ? targets[c0 + i] : 0;", "lmhead"),
]


@pytest.mark.parametrize("name,orig,mut,select", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, orig, mut, select):
    src = open(SRC).read()
    assert src.count(orig) >= 1, f"mutation anchor for '{name}' not found in oracle.c"
    bad = src.replace(orig, mut, 1)
    csrc = tmp_path / "oracle.c"
    csrc.write_text(bad)
    (tmp_path / "oracle.h").write_text(open(os.path.join(ROOT, "oracle", "oracle.h")).read())
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(lib), str(csrc), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", select],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, (f"the pins did not catch '{name}' (exit {r.returncode}):\n"
                               f"{r.stdout[-2000:]}")


# The blocked LM-head oracle (numpy): each case plants one mistake in a copy of the
# module, which a subprocess installs in place of oracle.lmhead_blocked before it
# runs the blocked oracle's pins.
BLOCKED_SRC = os.path.join(ROOT, "oracle", "lmhead_blocked.py")
BLOCKED_MUTATIONS = [
    ("tau dropped", "z = (h @ w.T) / tau", "z = (h @ w.T)"),
    ("tau taken as a double", "tau = float(np.float32(tau))", "tau = float(tau)"),
    ("weight rows reversed", "z = (h @ w.T) / tau", "z = (h @ w[::-1].T) / tau"),
    ("max dropped from lse", "lse = zmax[:, 0] + np.log(s)", "lse = np.log(s)"),
    ("entropy sign", 'out["entropy"][sel] = lse - (e * z).sum(axis=1) / s',
     'out["entropy"][sel] = (e * z).sum(axis=1) / s - lse'),
    ("targets by output index", "t = np.asarray(targets, np.int64)[rows]",
     "t = np.asarray(targets, np.int64)[: rows.size]"),
    ("bf16 decode off by one bit", "(b.astype(np.uint32) << 16)", "(b.astype(np.uint32) << 15)"),
    ("last hidden column dropped", "w = _decode_bf16(weight[:, :d])",
     "d = d - 1\n    w = _decode_bf16(weight[:, :d])"),
    ("error scale without absolute values", "a = np.abs(h) @ wabs.T", "a = h @ wabs.T"),
]

_RUN_BLOCKED_PINS = r"""
import importlib.util, os, sys
sys.path.insert(0, os.environ["VWC_ROOT"])
import oracle
spec = importlib.util.spec_from_file_location("oracle.lmhead_blocked", os.environ["MUT_SRC"])
mod = importlib.util.module_from_spec(spec)
spec.loader.exec_module(mod)
sys.modules["oracle.lmhead_blocked"] = mod
oracle.lmhead_blocked = mod
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider",
                      os.path.join(os.environ["VWC_ROOT"], "tests", "test_oracle_pins.py"),
                      "-k", "blocked"]))
"""


@pytest.mark.parametrize("name,orig,mut", BLOCKED_MUTATIONS, ids=[m[0] for m in BLOCKED_MUTATIONS])
def test_blocked_lmhead_pins_catch_planted_mistake(tmp_path, name, orig, mut):
    src = open(BLOCKED_SRC).read()
    assert src.count(orig) >= 1, f"mutation anchor for '{name}' not found in lmhead_blocked.py"
    path = tmp_path / "lmhead_blocked.py"
    path.write_text(src.replace(orig, mut, 1))
    env = dict(os.environ, VWC_ROOT=ROOT, MUT_SRC=str(path))
    r = subprocess.run([sys.executable, "-c", _RUN_BLOCKED_PINS], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, (f"the pins did not catch '{name}' (exit {r.returncode}):\n"
                               f"{r.stdout[-2000:]}")


def test_blocked_lmhead_pins_pass_unmutated(tmp_path):
    """The same harness on the module as it stands passes (so the cases above fail
    for their mistake, not for the harness)."""
    path = tmp_path / "lmhead_blocked.py"
    path.write_text(open(BLOCKED_SRC).read())
    env = dict(os.environ, VWC_ROOT=ROOT, MUT_SRC=str(path))
    r = subprocess.run([sys.executable, "-c", _RUN_BLOCKED_PINS], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
