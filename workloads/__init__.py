"""Seeded synthetic inputs for selected-token log-probability workloads.

This module is the only code that the HIP path's tests/benchmark and the CPU
oracle share.  It draws inputs and holds none of the method's arithmetic: no
softmax, no log-sum-exp, no gradient.

Every random quantity comes from its own counter-based stream,
``numpy.random.Philox`` keyed by (seed, stream name, row), so any row of any
workload can be regenerated on its own, bit for bit, without drawing the rows
before it.  That is what lets a test regenerate a handful of sampled rows of a
multi-gigabyte input for the oracle.

Workload shapes follow the pages' own workloads:
  * V = 248320 is the Qwen3.5 vocabulary named in "[megatron] feat: add
    memory-efficient chunked top-k KL computation" (section "Test") and in the
    slime issue on full-vocab fp32 logits (section "Bug Description");
  * V = 151936 stands for the "vocab=150k" of the torchforge parallel-logprob PR
    (section "Memory savings");
  * 62080 columns per slice is the TP=4 V_local of the verl PR (section "Peak
    memory");
  * packed sequences where only response spans carry loss follow the slime
    issue ("Steps to Reproduce");
  * the tiny [64, 2048] case follows the verl PR's small test (V=2048, odd
    chunk sizes);
  * the LM-head workloads project bf16 hidden states of size d = 2560 (the pages
    name 4B-class Qwen models but not their hidden size; 2560 is that size) onto
    the 248320-entry vocabulary, keeping the loss-mask rows of packed sequences
    before the projection, as the slime issue's maintainer comment proposes.
"""
from __future__ import annotations

import dataclasses
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Callable

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "scaled", "logits_rows", "targets", "loss_mask",
           "grad_out", "row_index", "fill_logits", "bf16_bits_to_float32", "float32_to_bf16_bits",
           "lmhead_weight", "lmhead_weight_rows", "lmhead_hidden", "lmhead_hidden_rows"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "bf16" or "fp32"
    n_rows: int
    vocab: int
    sigma: float          # standard deviation of the Gaussian logits
    seed: int
    tau: float = 1.0
    spike_row_prob: float = 0.0    # rows that get +spike_value at one uniform column
    spike_value: float = 0.0
    extreme_prob: float = 0.0      # entries replaced by +-extreme_value (fair sign)
    extreme_value: float = 0.0
    mask: str = "none"             # "none" | "bernoulli" | "packed"
    mask_prob: float = 0.0
    n_seqs: int = 0                # packed: sequences of n_rows / n_seqs tokens
    response_len: int = 0          # packed: one contiguous response span per sequence
    grad: str = "uniform"          # grad_out ~ U(-1, 1)
    grad_zero_prob: float = 0.0    # rows whose grad_out is set to 0
    n_slices: int = 1              # vocabulary slices for the split-V path
    topk: int = 0                  # teacher top-k payload size (distillation workloads)
    topk_boost: float = 0.0        # student logits at the teacher's columns get + U(0, boost)
    hidden: int = 0                # LM-head workloads: hidden size d (> 0); sigma is then the
                                   # standard deviation of the logits hidden . weight_j
    align_prob: float = 0.0        # LM head: rows whose hidden state leans toward the target's
    align_lo: float = 0.0          # weight row, raising the target logit by U(align_lo,
    align_hi: float = 0.0          # align_hi) on average
    lattice: bool = False          # LM head: hidden entries on multiples of 1/8 in [-4, 4],
                                   # weight entries on multiples of 1/64, so every partial
                                   # sum of a logit (|x| < 2^15, multiples of 2^-9) is exact
                                   # in fp32 whatever the summation order

    @property
    def esize(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def np_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32


WORKLOADS = {
    # fp32 [64, 2048] ~ N(0,1): forward logprob + entropy + fp32 backward.
    "tiny_fp32_64x2048": Workload(
        "tiny_fp32_64x2048", "fp32", 64, 2048, 1.0, seed=0),
    # bf16 [4096, 151936] ~ N(0, 3^2), Bernoulli(0.5) loss mask, compacted rows.
    "masked_bf16_4096x151936": Workload(
        "masked_bf16_4096x151936", "bf16", 4096, 151936, 3.0, seed=1,
        mask="bernoulli", mask_prob=0.5),
    # bf16 [8192, 248320] ~ N(0, 3^2) with a +8 spike in 10% of rows; 30% of
    # rows carry zero grad_out.
    "spiked_bf16_8192x248320": Workload(
        "spiked_bf16_8192x248320", "bf16", 8192, 248320, 3.0, seed=2,
        spike_row_prob=0.1, spike_value=8.0, grad_zero_prob=0.3),
    # bf16 [32768, 248320] ~ N(0, 2^2): 8 packed sequences of 4096 tokens, one
    # contiguous 1024-token response span each (25% of tokens).
    "packed_bf16_32768x248320": Workload(
        "packed_bf16_32768x248320", "bf16", 32768, 248320, 2.0, seed=3,
        mask="packed", n_seqs=8, response_len=1024),
    # fp32 [16384, 248320] ~ N(0, 4^2) with 1% of entries at +-1e4, tau=0.7,
    # vocabulary in 4 slices of 62080.
    "extreme_fp32_16384x248320": Workload(
        "extreme_fp32_16384x248320", "fp32", 16384, 248320, 4.0, seed=4, tau=0.7,
        extreme_prob=0.01, extreme_value=1.0e4, n_slices=4),
    # Top-k distillation (verl PR, "Test": b=2, s=96, V=2048, K=32): fp32 student
    # logits ~ N(0,1) boosted at the teacher's 32 columns.
    "distill_fp32_192x2048_k32": Workload(
        "distill_fp32_192x2048_k32", "fp32", 192, 2048, 1.0, seed=5, topk=32, topk_boost=4.0),
    # The page's Qwen3.5-4B distillation dimensions: V=248320, K=128, N=4096 tokens.
    "distill_bf16_4096x248320_k128": Workload(
        "distill_bf16_4096x248320_k128", "bf16", 4096, 248320, 2.0, seed=6, topk=128,
        topk_boost=6.0),
    # Fused LM head, small: bf16 hidden [300, 320] and weight [2000, 320] (ragged in
    # every tile dimension), logits ~ N(0, 2^2), half of the rows confident.
    "lmhead_bf16_300x2000_d320": Workload(
        "lmhead_bf16_300x2000_d320", "bf16", 300, 2000, 2.0, seed=7, hidden=320,
        align_prob=0.5, align_lo=2.0, align_hi=10.0),
    # Fused LM head at the pages' vocabulary: 4 packed sequences of 4096 tokens with a
    # 2048-token response span each (8192 loss rows of 16384), d = 2560.
    "lmhead_bf16_16384x248320_d2560": Workload(
        "lmhead_bf16_16384x248320_d2560", "bf16", 16384, 248320, 2.0, seed=8, hidden=2560,
        mask="packed", n_seqs=4, response_len=2048, align_prob=0.5, align_lo=4.0,
        align_hi=16.0),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(name: str, n_rows: int, vocab: int, **overrides) -> Workload:
    """Same distributions as a named workload at another shape (parity sizes)."""
    w = WORKLOADS[name]
    kw = dict(n_rows=n_rows, vocab=vocab, name=f"{w.name}@{n_rows}x{vocab}")
    if w.mask == "packed" and "response_len" not in overrides:
        kw["response_len"] = max(1, (n_rows // max(w.n_seqs, 1)) // 4)
    kw.update(overrides)
    return dataclasses.replace(w, **kw)


# --------------------------------------------------------------------------- streams

def _stream_key(seed: int, stream: str) -> int:
    h = hashlib.sha256(f"{seed}:{stream}".encode()).digest()
    return int.from_bytes(h[:8], "little")


def _gen(w: Workload, stream: str, index: int = 0) -> np.random.Generator:
    key = np.array([_stream_key(w.seed, stream), index], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def float32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); NaN stays NaN. Input quantization."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    b = ((u + r) >> 16).astype(np.uint16)
    if nan.any():
        b[nan] = 0x7FC0
    return b


def bf16_bits_to_float32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def topk_payload_rows(w: Workload, rows):
    """Teacher top-k payload of rows `rows`: (int32 [n, K] distinct columns,
    float32 [n, K] teacher log-probabilities, descending).  Teacher
    probabilities are exponential weights scaled to a per-row mass P ~ U(0.5, 0.98)."""
    rows = np.atleast_1d(np.asarray(rows, dtype=np.int64))
    K = w.topk
    idx = np.empty((rows.size, K), np.int32)
    tlp = np.empty((rows.size, K), np.float32)
    for i, r in enumerate(rows):
        g = _gen(w, "topk", int(r))
        idx[i] = g.choice(w.vocab, size=K, replace=False).astype(np.int32)
        mass = g.uniform(0.5, 0.98)
        e = np.sort(g.exponential(size=K))[::-1]
        tlp[i] = np.log(mass * e / e.sum()).astype(np.float32)
    return idx, tlp


def topk_payload(w: Workload):
    return topk_payload_rows(w, np.arange(w.n_rows))


def _row_values(w: Workload, r: int) -> np.ndarray:
    """float32 values of row r before storage rounding."""
    x = _gen(w, "logits", r).standard_normal(w.vocab, dtype=np.float32)
    x *= np.float32(w.sigma)
    if w.topk > 0:
        idx, _ = topk_payload_rows(w, [r])
        boost = _gen(w, "boost", r).uniform(0.0, w.topk_boost, size=w.topk).astype(np.float32)
        x[idx[0]] += boost
    if w.spike_row_prob > 0.0:
        g = _gen(w, "spike", r)
        has = g.random() < w.spike_row_prob
        col = int(g.integers(0, w.vocab))
        if has:
            x[col] += np.float32(w.spike_value)
    if w.extreme_prob > 0.0:
        g = _gen(w, "extreme", r)
        hit = g.random(w.vocab) < w.extreme_prob
        sign = g.random(w.vocab) < 0.5
        x[hit & sign] = np.float32(w.extreme_value)
        x[hit & ~sign] = np.float32(-w.extreme_value)
    return x


def logits_rows(w: Workload, rows, ld: int | None = None) -> np.ndarray:
    """Rows `rows` of the workload's logits: uint16 bf16 bits or float32, [len(rows), ld]."""
    rows = np.atleast_1d(np.asarray(rows, dtype=np.int64))
    ld = w.vocab if ld is None else ld
    out = np.zeros((rows.shape[0], ld), dtype=w.np_dtype)
    for i, r in enumerate(rows):
        if not 0 <= r < w.n_rows:
            raise IndexError(f"row {r} outside [0, {w.n_rows})")
        x = _row_values(w, int(r))
        out[i, : w.vocab] = float32_to_bf16_bits(x) if w.dtype == "bf16" else x
    return out


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def fill_logits(w: Workload, sink: Callable[[int, np.ndarray], None], block_rows: int = 256,
                threads: int | None = None, ld: int | None = None) -> None:
    """Generate all rows in blocks; sink(row0, block) is called in row order."""
    threads = threads or default_threads()
    starts = list(range(0, w.n_rows, block_rows))

    def make(r0):
        return logits_rows(w, np.arange(r0, min(r0 + block_rows, w.n_rows)), ld=ld)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        # Keep at most 2 * threads blocks in flight so host memory stays bounded.
        pending = {}
        nxt = 0
        for i, r0 in enumerate(starts):
            while nxt < len(starts) and nxt < i + 2 * threads:
                pending[nxt] = ex.submit(make, starts[nxt])
                nxt += 1
            sink(r0, pending.pop(i).result())


def all_logits(w: Workload, ld: int | None = None) -> np.ndarray:
    """Whole logits array on the host (small workloads only)."""
    ld = w.vocab if ld is None else ld
    out = np.empty((w.n_rows, ld), dtype=w.np_dtype)

    def sink(r0, blk):
        out[r0: r0 + blk.shape[0]] = blk

    fill_logits(w, sink, block_rows=64)
    return out


def targets(w: Workload) -> np.ndarray:
    """int32[n_rows], i.i.d. uniform over [0, vocab)."""
    return _gen(w, "targets").integers(0, w.vocab, size=w.n_rows, dtype=np.int64).astype(np.int32)


def loss_mask(w: Workload) -> np.ndarray:
    """uint8[n_rows] loss mask (all ones when the workload has none)."""
    if w.mask == "none":
        return np.ones(w.n_rows, np.uint8)
    if w.mask == "bernoulli":
        return (_gen(w, "mask").random(w.n_rows) < w.mask_prob).astype(np.uint8)
    if w.mask == "packed":
        seq = w.n_rows // w.n_seqs
        if w.response_len > seq:
            raise ValueError("response span longer than its sequence")
        m = np.zeros(w.n_rows, np.uint8)
        g = _gen(w, "spans")
        # Each packed sequence holds a prompt/tool prefix, one contiguous response
        # span at a seeded offset, and possibly a suffix.
        for s in range(w.n_seqs):
            off = int(g.integers(0, seq - w.response_len + 1))
            m[s * seq + off: s * seq + off + w.response_len] = 1
        return m
    raise ValueError(w.mask)


def row_index(w: Workload) -> np.ndarray:
    """Ascending int32 row ids where the loss mask is set."""
    return np.flatnonzero(loss_mask(w)).astype(np.int32)


# --------------------------------------------------------------------------- LM head

def _weight_sigma(w: Workload) -> float:
    return w.sigma / float(np.sqrt(w.hidden))


_WEIGHT_BLOCK = 256


def _weight_block_values(w: Workload, b: int) -> np.ndarray:
    """float32 weight rows [b * 256, min((b + 1) * 256, vocab)) before storage rounding;
    one counter-based stream per block of 256 vocabulary rows."""
    j0 = b * _WEIGHT_BLOCK
    n = min(_WEIGHT_BLOCK, w.vocab - j0)
    x = _gen(w, "weight", b).standard_normal((n, w.hidden), dtype=np.float32)
    x *= np.float32(_weight_sigma(w))
    if w.lattice:
        x = np.clip(np.round(x * 64.0), -127.0, 127.0).astype(np.float32) / np.float32(64.0)
    return x


def lmhead_weight_rows(w: Workload, rows, ld: int | None = None) -> np.ndarray:
    """bf16 bits [len(rows), ld] of the output-layer weight (one row per vocabulary
    entry), entries N(0, (sigma / sqrt(d))^2) so that a N(0, 1) hidden state gives
    logits of standard deviation sigma."""
    rows = np.atleast_1d(np.asarray(rows, dtype=np.int64))
    ld = w.hidden if ld is None else ld
    if rows.size and (rows.min() < 0 or rows.max() >= w.vocab):
        raise IndexError(f"weight rows outside [0, {w.vocab})")
    out = np.zeros((rows.shape[0], ld), np.uint16)
    for b in np.unique(rows // _WEIGHT_BLOCK):
        sel = np.flatnonzero(rows // _WEIGHT_BLOCK == b)
        blk = float32_to_bf16_bits(_weight_block_values(w, int(b)))
        out[sel, : w.hidden] = blk[rows[sel] - b * _WEIGHT_BLOCK]
    return out


def lmhead_weight(w: Workload, ld: int | None = None, threads: int | None = None) -> np.ndarray:
    """The whole weight [vocab, ld] as bf16 bits (blocks generated in parallel)."""
    ld = w.hidden if ld is None else ld
    out = np.zeros((w.vocab, ld), np.uint16)

    def make(b):
        j0 = b * _WEIGHT_BLOCK
        out[j0: j0 + _WEIGHT_BLOCK, : w.hidden] = float32_to_bf16_bits(_weight_block_values(w, b))

    nblk = (w.vocab + _WEIGHT_BLOCK - 1) // _WEIGHT_BLOCK
    with ThreadPoolExecutor(max_workers=threads or default_threads()) as ex:
        list(ex.map(make, range(nblk)))
    return out


def lmhead_hidden_rows(w: Workload, rows, ld: int | None = None,
                       weight: np.ndarray | None = None) -> np.ndarray:
    """bf16 bits [len(rows), ld] of the final hidden states.  Each row is N(0, 1); on a
    Bernoulli(align_prob) subset a multiple of the target's weight row is added,
    alpha * W_t / (sigma_w^2 d) with alpha ~ U(align_lo, align_hi), which raises the
    target logit by about alpha.  `weight` (the bf16 weight, if already generated)
    saves regenerating the target rows."""
    rows = np.atleast_1d(np.asarray(rows, dtype=np.int64))
    ld = w.hidden if ld is None else ld
    tg = targets(w)
    out = np.zeros((rows.shape[0], ld), np.uint16)
    sw2d = np.float32(_weight_sigma(w) ** 2 * w.hidden)
    for i, r in enumerate(rows):
        if not 0 <= r < w.n_rows:
            raise IndexError(f"row {r} outside [0, {w.n_rows})")
        x = _gen(w, "hidden", int(r)).standard_normal(w.hidden, dtype=np.float32)
        if w.align_prob > 0.0:
            g = _gen(w, "align", int(r))
            if g.random() < w.align_prob:
                alpha = np.float32(g.uniform(w.align_lo, w.align_hi))
                wrow = (weight[tg[r], : w.hidden] if weight is not None
                        else lmhead_weight_rows(w, [tg[r]])[0])
                x += alpha * bf16_bits_to_float32(wrow) / sw2d
        if w.lattice:
            x = np.clip(np.round(x * 8.0), -32.0, 32.0).astype(np.float32) / np.float32(8.0)
        out[i, : w.hidden] = float32_to_bf16_bits(x)
    return out


def lmhead_hidden(w: Workload, ld: int | None = None, threads: int | None = None,
                  weight: np.ndarray | None = None) -> np.ndarray:
    """All hidden rows [n_rows, ld] as bf16 bits."""
    ld = w.hidden if ld is None else ld
    out = np.empty((w.n_rows, ld), np.uint16)
    starts = list(range(0, w.n_rows, 256))

    def make(r0):
        out[r0: r0 + 256] = lmhead_hidden_rows(w, np.arange(r0, min(r0 + 256, w.n_rows)), ld,
                                               weight=weight)

    with ThreadPoolExecutor(max_workers=threads or default_threads()) as ex:
        list(ex.map(make, starts))
    return out


def grad_out(w: Workload) -> np.ndarray:
    """float32[n_rows] incoming gradient of each row's logprob, U(-1, 1); zero on a
    Bernoulli(grad_zero_prob) subset of rows."""
    g = _gen(w, "grad").uniform(-1.0, 1.0, size=w.n_rows).astype(np.float32)
    if w.grad_zero_prob > 0.0:
        z = _gen(w, "grad_zero").random(w.n_rows) < w.grad_zero_prob
        g[z] = 0.0
    return g
