"""The seeded input generator: the full-size GPU tests regenerate sampled rows
for the oracle, so any row, block split or thread count must give the same bytes."""
import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("name", ["spiked_bf16_8192x248320", "extreme_fp32_16384x248320",
                                  "distill_bf16_4096x248320_k128", "tiny_fp32_64x2048"])
def test_rows_regenerate_bit_for_bit(name):
    w = W.scaled(name, 40, 3001)
    full = W.all_logits(w)
    assert np.array_equal(full, W.all_logits(w))  # same call, same bytes
    rows = np.array([39, 0, 17, 17, 5])
    assert np.array_equal(W.logits_rows(w, rows), full[rows])
    # block size and thread count change nothing
    for block, threads in ((1, 1), (7, 3), (64, 8)):
        got = np.empty_like(full)

        def sink(r0, blk):
            got[r0:r0 + blk.shape[0]] = blk

        W.fill_logits(w, sink, block_rows=block, threads=threads)
        assert np.array_equal(got, full)
    # a padded row stride keeps the values in the leading columns
    padded = W.logits_rows(w, rows, ld=3008)
    assert padded.shape == (5, 3008) and np.array_equal(padded[:, :3001], full[rows])


def test_row_values_do_not_depend_on_the_row_count():
    """Row r of a scaled workload equals row r of the same workload with more rows
    (every stream is keyed by (seed, stream, row))."""
    a = W.all_logits(W.scaled("spiked_bf16_8192x248320", 16, 2048))
    b = W.all_logits(W.scaled("spiked_bf16_8192x248320", 48, 2048))
    assert np.array_equal(a, b[:16])


def test_side_inputs_are_seeded():
    w = W.get("masked_bf16_4096x151936")
    assert np.array_equal(W.targets(w), W.targets(w))
    assert np.array_equal(W.loss_mask(w), W.loss_mask(w))
    assert np.array_equal(W.grad_out(w), W.grad_out(w))
    assert W.row_index(w).size == int(W.loss_mask(w).sum())
    p = W.get("packed_bf16_32768x248320")
    m = W.loss_mask(p)
    assert int(m.sum()) == 8 * 1024
    # one contiguous response span per 4096-token sequence
    for s in range(8):
        seg = m[s * 4096:(s + 1) * 4096]
        on = np.flatnonzero(seg)
        assert on.size == 1024 and on[-1] - on[0] == 1023


def test_lmhead_rows_regenerate():
    w = W.scaled("lmhead_bf16_300x2000_d320", 300, 2000)
    wt = W.lmhead_weight(w)
    rows = np.array([1999, 0, 255, 256, 1024])
    assert np.array_equal(W.lmhead_weight_rows(w, rows), wt[rows])
    assert np.array_equal(W.lmhead_weight(w, threads=1), wt)
    h = W.lmhead_hidden(w, weight=wt)
    hr = np.array([299, 3, 150])
    assert np.array_equal(W.lmhead_hidden_rows(w, hr, weight=wt), h[hr])
    assert np.array_equal(W.lmhead_hidden(w), h)  # without the weight handed in


def test_topk_payload_rows_are_distinct_and_seeded():
    w = W.get("distill_fp32_192x2048_k32")
    idx, tlp = W.topk_payload(w)
    i2, t2 = W.topk_payload_rows(w, [5, 100])
    assert np.array_equal(i2, idx[[5, 100]]) and np.array_equal(t2, tlp[[5, 100]])
    for r in range(w.n_rows):
        assert np.unique(idx[r]).size == w.topk
    P = np.exp(tlp.astype(np.float64)).sum(1)
    assert (P > 0.5 - 1e-5).all() and (P < 0.98 + 1e-5).all()
