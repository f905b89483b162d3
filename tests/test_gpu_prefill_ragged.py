"""GPU parity of indexer_score_prefill_ragged against the oracle (Modular page
"sparse_index_fp8_sm100", module description: a ragged batch, causal
masking, the -inf tail fill): visible scores within
|gpu - oracle| <= 1e-6 + 1e-5 |oracle|, every masked column exactly -inf,
row_len exact, nothing written at or past the width, and the top-16 of each
row (valid_len = row_len) equal to the oracle's selection over the GPU's own
scores."""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import workloads
from gpu_util import CANARY_F32, CANARY_I32, announce, assert_scores_close, dev, host

pytestmark = pytest.mark.gpu


def ragged_batch(seed, q_lens, k_lens, H, gap=5):
    q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    k_start = np.zeros(len(k_lens), np.int32)
    off = 3
    for s, kl in enumerate(k_lens):
        k_start[s] = off
        off += kl + gap
    T = int(q_start[-1])
    p = workloads.prefill_inputs("ragged", seed, T, H, off)
    return p, q_start, k_start, np.asarray(k_lens, np.int32)


def run(p, q_start, k_start, k_len, width, ld, max_q=None):
    import page_scoring_top_amd as ps
    T = p.q.shape[0]
    scores = torch.full((T, ld), float(CANARY_F32), dtype=torch.float32, device="cuda")
    row_len = torch.full((T,), int(CANARY_I32), dtype=torch.int32, device="cuda")
    max_q = int(np.diff(q_start).max()) if max_q is None else max_q
    ps.indexer_score_prefill_ragged(dev(p.q), dev(p.q_scale), dev(p.k), dev(p.k_scale),
                                    dev(q_start), dev(k_start), dev(k_len), max_q, width, scores,
                                    row_len)
    ids = torch.full((T, 16), int(CANARY_I32), dtype=torch.int32, device="cuda")
    ps.topk16_select(scores, width, ids, valid_len=row_len)
    return host(scores), host(row_len), host(ids)


CASES = [
    # (q_lens, k_lens): single tokens, a chunk equal to its context (lower
    # triangle), long contexts split over key groups, an empty sequence, a
    # chunk longer than its context, ragged token groups.
    ([1, 37, 130, 5, 0, 64, 150, 10], [1, 1000, 130, 3000, 200, 64, 2000, 3]),
    ([129], [129]),
    ([3, 2], [5000, 7]),
    # query groups that see no key (40 queries over 5 keys; a sequence with no
    # keys), a single query, and sequences of many chunks, split over the
    # shares of several work-groups of the balanced schedule (57 chunks in
    # all, fewer than the work-groups, so most shares are one chunk or none)
    ([40, 24, 8, 1, 17], [5, 1500, 0, 129, 700]),
]


@pytest.mark.parametrize("H", [4, 20, 64])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_ragged_batch(H, case):
    q_lens, k_lens = CASES[case]
    p, q_start, k_start, k_len = ragged_batch(31 * case + H, q_lens, k_lens, H)
    width = max(k_lens) + 2
    announce(f"ragged prefill H={H} q_lens={q_lens} k_lens={k_lens}")
    got, row_len, ids = run(p, q_start, k_start, k_len, width, width + 3)
    want, want_len = oracle.score_prefill_ragged(p.q, p.q_scale, p.k, p.k_scale, q_start, k_start,
                                                 k_len, width)
    assert np.array_equal(row_len, want_len), "row_len differs"
    assert_scores_close(got[:, :width], want, f"H={H} case {case}")
    assert (got[:, width:].view(np.int32) == CANARY_F32.view(np.int32)).all(), "write past width"
    want_ids = oracle.topk16(got[:, :width], valid_len=want_len)
    assert np.array_equal(ids, want_ids), "top-16 differs"


@pytest.mark.parametrize("H", [4, 20])
def test_width_below_context(H):
    """Rows are cut at the width: counts clamp to it and nothing is written
    past it (four heads: the packed grid; 20: the balanced schedule, whose
    costs clamp to the width too)."""
    p, q_start, k_start, k_len = ragged_batch(7, [40, 8], [900, 50], H)
    width = 300
    announce(f"ragged prefill width below context H={H}")
    got, row_len, _ = run(p, q_start, k_start, k_len, width, width + 1)
    want, want_len = oracle.score_prefill_ragged(p.q, p.q_scale, p.k, p.k_scale, q_start, k_start,
                                                 k_len, width)
    assert np.array_equal(row_len, want_len)
    assert_scores_close(got[:, :width], want, "width below context")
    assert (got[:, width:].view(np.int32) == CANARY_F32.view(np.int32)).all()


@pytest.mark.timeout(600)
def test_big_batch_rows_of_every_wave():
    """Four sequences of 512 queries with 4,096 .. 16,384-token contexts and
    64 heads (2,048 rows x 16,384 columns, the benchmark's launch
    configuration): 33 full rows of every sequence -- one per two work-groups
    of eight queries, the wave position cycling through all eight, and the
    last query -- against the oracle; the -inf fill of all 2,048 rows."""
    d = workloads.ragged_prefill()
    announce("ragged prefill 4 x 512 x 64 heads, contexts 4096..16384")
    got, row_len, _ = run(d.p, d.q_start, d.k_start, d.k_len, d.width, d.width)
    pieces = []
    for s in range(len(d.k_len)):
        q_len = int(d.q_start[s + 1] - d.q_start[s])
        for i in [16 * k + (k % 8) for k in range(32)] + [q_len - 1]:
            pieces.append((s, int(d.q_start[s]) + i, oracle.causal_count(q_len, int(d.k_len[s]), i,
                                                                         d.width)))
    for s in range(len(d.k_len)):
        q_len = int(d.q_start[s + 1] - d.q_start[s])
        for i in range(q_len):
            t = int(d.q_start[s]) + i
            c = oracle.causal_count(q_len, int(d.k_len[s]), i, d.width)
            assert row_len[t] == c, f"row_len of row {t}"
            assert np.all(np.isneginf(got[t, c:])), f"-inf fill of row {t}"

    def one(piece):
        s, t, c = piece
        k0 = int(d.k_start[s])
        return oracle.score_prefill_rows(d.p.q, d.p.q_scale, d.p.k[k0:k0 + c],
                                         d.p.k_scale[k0:k0 + c], [t])[0]

    for (s, t, c), want in zip(pieces, oracle_pool.map_pieces(one, pieces, "ragged rows")):
        assert_scores_close(got[t, :c], want, f"row {t}")


def test_most_sequences_in_one_call():
    """65,535 sequences, the most one call takes (one grid slice each): most
    have no query, 1 in 128 has two queries over a short context."""
    S = 65535
    q_lens = np.where(np.arange(S) % 128 == 3, 2, 0)
    k_lens = np.where(np.arange(S) % 128 == 3, 40, 3)
    p, q_start, k_start, k_len = ragged_batch(52, list(q_lens), list(k_lens), 4, gap=0)
    width = 42
    announce("ragged prefill 65,535 sequences")
    got, row_len, ids = run(p, q_start, k_start, k_len, width, width)
    want, want_len = oracle.score_prefill_ragged(p.q, p.q_scale, p.k, p.k_scale, q_start, k_start,
                                                 k_len, width)
    assert np.array_equal(row_len, want_len)
    assert_scores_close(got, want, "65,535 sequences")
    assert np.array_equal(ids, oracle.topk16(got, valid_len=want_len))


@pytest.mark.parametrize("H", [20, 33, 64])
def test_most_sequences_of_the_balanced_schedule(H):
    """256 sequences, the most the balanced schedule takes (every lane costs
    four of them): empty sequences, query groups past their few keys
    (zero-chunk groups owned by whichever share holds them), one-chunk and
    several-chunk groups, so that shares start and end inside sequences,
    at group ends and on empty groups.  The oracle scores each sequence on
    its own (the pieces run on host threads)."""
    rng = np.random.default_rng(256 + H)
    S = 256
    q_lens = rng.integers(0, 21, S)
    q_lens[rng.integers(0, S, 40)] = 0
    k_lens = rng.integers(0, 300, S)
    k_lens[::17] = rng.integers(0, 6, len(k_lens[::17]))
    p, q_start, k_start, k_len = ragged_batch(77 + H, list(q_lens), list(k_lens), H, gap=1)
    width = 310
    announce(f"ragged prefill 256 sequences H={H}")
    got, row_len, ids = run(p, q_start, k_start, k_len, width, width + 2)

    def one(s):
        a0, a1, k0, kl = int(q_start[s]), int(q_start[s + 1]), int(k_start[s]), int(k_len[s])
        return oracle.score_prefill_ragged(p.q[a0:a1], p.q_scale[a0:a1], p.k[k0:k0 + kl],
                                           p.k_scale[k0:k0 + kl], np.array([0, a1 - a0], np.int32),
                                           np.zeros(1, np.int32), np.array([kl], np.int32), width)

    parts = oracle_pool.map_pieces(one, range(S), "ragged sequences")
    want = np.concatenate([w for w, _ in parts])
    want_len = np.concatenate([n for _, n in parts])
    assert np.array_equal(row_len, want_len), "row_len differs"
    assert_scores_close(got[:, :width], want, f"256 sequences H={H}")
    assert (got[:, width:].view(np.int32) == CANARY_F32.view(np.int32)).all(), "write past width"
    assert np.array_equal(ids, oracle.topk16(got[:, :width], valid_len=want_len)), "top-16 differs"
