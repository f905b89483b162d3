"""The threaded oracle driver (tests/oracle_pool.py) gives the same bits as
the oracle's own serial calls: it only splits the work into independent
pieces."""

import numpy as np

import oracle
import oracle_pool
import workloads


def test_pooled_decode_equals_serial():
    d = workloads.decode_inputs("pool", 21, [3000, 129, 700, 0, 2500], qlen=5, width=20,
                                pad_reqs=1)
    base = np.full((d.q.shape[0], 32, d.width), np.float32(-3.5), np.float32)
    want, _ = oracle.score_decode(d.kv_cache, d.block_table, d.seq_lens, d.q, d.q_scale,
                                  d.num_reqs, d.qlen, d.width, scores=base[:d.num_reqs].copy())
    got, stored = oracle_pool.score_decode(d, base=base)
    assert np.array_equal(got[:d.num_reqs].view(np.int32), want.view(np.int32))
    assert np.array_equal(got[d.num_reqs:].view(np.int32), base[d.num_reqs:].view(np.int32))
    assert np.array_equal(stored[:d.num_reqs], want != np.float32(-3.5))
    assert not stored[d.num_reqs:].any()


def test_pooled_prefill_rows_equal_serial():
    p = workloads.prefill_inputs("pool", 22, 9, 3, 70)
    rows = [8, 0, 4, 5, 1]
    want = oracle.score_prefill_rows(p.q, p.q_scale, p.k, p.k_scale, rows)
    got = oracle_pool.score_prefill_rows(p.q, p.q_scale, p.k, p.k_scale, rows)
    assert np.array_equal(got.view(np.int32), want.view(np.int32))


def test_pooled_topk_equals_serial():
    t = workloads.injected_rows(23, 37, 300)
    ap = np.arange(37, dtype=np.int32) - 3
    want = oracle.topk16(t.scores, t.valid, t.force_begin, t.force_end, ap)
    got = oracle_pool.topk16(t.scores, t.valid, t.force_begin, t.force_end, ap, rows_per_task=5)
    assert np.array_equal(got, want)
