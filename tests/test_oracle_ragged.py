"""Pins of the oracle's ragged causal prefill scores (Modular page
"sparse_index_fp8_sm100", module description: causal masking and the -inf
tail fill over a batch of sequences), against what the reading fixes:

* the visible part of every row equals the pinned dense scorer run on that
  sequence's own query rows and key slice (so the row, key-slice and column
  indexing are checked by an independent call);
* the mask: a sequence's first query sees k_len - q_len + 1 keys, each next
  query one more, the last sees all k_len; counts clamp to [0, width];
  everything past the count is -inf; columns >= width are not written;
* a query chunk longer than its context leaves its first rows empty."""

import numpy as np

import oracle
import workloads


def _batch(seed, q_lens, k_lens, H, width_pad=0, gap=5):
    rng = np.random.default_rng(seed)
    S = len(q_lens)
    q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    k_start = np.zeros(S, np.int32)
    off = 3
    for s in range(S):
        k_start[s] = off
        off += k_lens[s] + gap
    T, N = int(q_start[-1]), off
    p = workloads.prefill_inputs("ragged-pin", seed, max(T, 1), H, N)
    width = max(k_lens) + width_pad
    del rng
    return p, q_start, k_start, np.asarray(k_lens, np.int32), width


def test_visible_part_equals_dense_scores_per_sequence():
    q_lens, k_lens = [5, 1, 0, 9, 3], [40, 1, 7, 9, 70]
    p, qs_, ks_, kl, width = _batch(1, q_lens, k_lens, 3, width_pad=4)
    got, row_len = oracle.score_prefill_ragged(p.q, p.q_scale, p.k, p.k_scale, qs_, ks_, kl, width,
                                               ld=width + 2)
    for s in range(len(q_lens)):
        rows = slice(qs_[s], qs_[s + 1])
        dense = oracle.score_prefill(p.q[rows], p.q_scale[rows], p.k[ks_[s]:ks_[s] + kl[s]],
                                     p.k_scale[ks_[s]:ks_[s] + kl[s]])
        for i in range(q_lens[s]):
            t = qs_[s] + i
            c = row_len[t]
            assert np.array_equal(got[t, :c], dense[i, :c])
            assert np.all(np.isneginf(got[t, c:width]))
            assert np.all(np.isnan(got[t, width:]))         # past width: untouched


def test_mask_counts():
    q_lens, k_lens = [4, 6, 2], [10, 6, 300]
    p, qs_, ks_, kl, width = _batch(2, q_lens, k_lens, 1)
    _, row_len = oracle.score_prefill_ragged(p.q, p.q_scale, p.k, p.k_scale, qs_, ks_, kl, width)
    assert list(row_len[0:4]) == [7, 8, 9, 10]                # first sees k_len - q_len + 1
    assert list(row_len[4:10]) == [1, 2, 3, 4, 5, 6]          # q_len == k_len: lower triangle
    assert list(row_len[10:12]) == [299, 300]


def test_counts_clamp_to_width_and_zero():
    assert oracle.causal_count(3, 10, 2, 8) == 8              # width below the context
    assert oracle.causal_count(5, 2, 0, 100) == 0             # chunk longer than the context
    assert oracle.causal_count(5, 2, 3, 100) == 1
    assert oracle.causal_count(5, 2, 4, 100) == 2              # the last query sees all k_len
    assert oracle.causal_count(1, 0, 0, 100) == 0
    q_lens, k_lens = [6], [3]
    p, qs_, ks_, kl, width = _batch(3, q_lens, k_lens, 2, width_pad=2)
    got, row_len = oracle.score_prefill_ragged(p.q, p.q_scale, p.k, p.k_scale, qs_, ks_, kl, width)
    assert list(row_len) == [0, 0, 0, 1, 2, 3]
    assert np.all(np.isneginf(got[:3]))
