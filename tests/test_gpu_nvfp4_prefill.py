"""GPU parity of the NVFP4 prefill chain (Q8KV8 prefill indexer, vLLM API page
``gather_nvfp4_index_k``, module description): each request's NVFP4 index-K
pages are gathered into contiguous E4M3 keys by nvfp4_index_k_dequant, its
queries are scored against the first ``context`` keys by
indexer_score_prefill with every key scale 1 (the pages carry no global
scale), and topk16_select picks the 16 best keys of every query row.

Each stage is checked against the oracle on the same inputs: the gathered
bytes exactly, the scores against the oracle's scores of the oracle's
gathered keys, and the top-16 exactly against the oracle's selection over the
GPU's own score rows.

Score tolerance.  Block scales span the whole positive E4M3 range, so keys
reach 448 and a token's dot products can cancel to a result far below their
terms; an f32 accumulation is then off by a few units in the last place of
the terms, not of the result.  This path therefore does not meet the plain
bound |gpu - oracle| <= 1e-6 + 1e-5 |oracle| on every score.  Every score
must meet |gpu - oracle| <= 1e-6 + 1e-5 max(|oracle|, M), M = k_scale *
sum_h q_scale * sum_d |q k| (the size of the summed terms); the scores
outside the plain bound are counted, printed, and may be at most 0.1%."""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import workloads
from gpu_util import (ATOL, CANARY_F32, CANARY_I32, RTOL, announce, assert_scores_close, dev, host,
                      prefill_term_magnitude)

pytestmark = pytest.mark.gpu


def gather_gpu(d: workloads.Nvfp4PrefillInputs, extra_pages: int = 1):
    import page_scoring_top_amd as ps
    total = d.total_pages
    out = torch.full((total + extra_pages, 128, 128), 0xA5, dtype=torch.uint8, device="cuda")
    ps.nvfp4_index_k_dequant(dev(d.kv_cache), dev(d.block_table), dev(d.num_pages),
                             dev(d.page_offsets), d.block_table.shape[1], out)
    return out


def gather_oracle(d: workloads.Nvfp4PrefillInputs, extra_pages: int = 1):
    out = np.full((d.total_pages + extra_pages, 128, 128), 0xA5, dtype=np.uint8)
    return oracle.gather(d.kv_cache, d.block_table, d.num_pages, d.page_offsets,
                         d.block_table.shape[1], out)


def request_keys(keys, d, b):
    """Keys [context[b], 128] of request b inside the gathered pages."""
    off = int(d.page_offsets[b])
    return keys[off:off + int(d.num_pages[b])].reshape(-1, 128)[:int(d.context[b])]


def check_scores(got, want, magnitude, what):
    """Every score within the term bound; returns (outside the plain bound,
    compared), which is printed and may be at most 0.1%."""
    assert_scores_close(got, want, what, magnitude=magnitude)
    fin = np.isfinite(want)
    plain = np.abs(got[fin].astype(np.float64) - want[fin]) <= ATOL + RTOL * np.abs(want[fin])
    n_out, n = int((~plain).sum()), int(fin.sum())
    print(f"[nvfp4-prefill] {what}: {n_out} of {n} scores outside the plain bound", flush=True)
    assert n_out <= 1e-3 * n, f"{what}: {n_out} scores need the term bound"
    return n_out, n


def run_chain(d: workloads.Nvfp4PrefillInputs, keys_gpu):
    """Per request: scores [tokens, context + 2] (two canary columns) and
    top-16 ids, on the GPU."""
    import page_scoring_top_amd as ps
    res = []
    t0 = 0
    for b in range(len(d.tokens)):
        T, N = int(d.tokens[b]), int(d.context[b])
        q = dev(d.q[t0:t0 + T])
        qs = dev(d.q_scale[t0:t0 + T])
        k = request_keys(keys_gpu, d, b)
        ones = torch.ones(N, dtype=torch.float32, device="cuda")
        scores = torch.full((T, N + 2), float(CANARY_F32), dtype=torch.float32, device="cuda")
        ps.indexer_score_prefill(q, qs, k, ones, scores)
        ids = torch.full((T, 16), int(CANARY_I32), dtype=torch.int32, device="cuda")
        ps.topk16_select(scores, N, ids)
        res.append((scores, ids))
        t0 += T
    return res


@pytest.mark.parametrize("tokens,contexts,heads", [
    ([37, 100, 1], [1000, 3000, 129], 4),   # ragged token groups and key tails
    ([64], [128], 4),                       # whole tiles only
    ([20, 9], [300, 17], 1),
    ([11], [700], 3),
    ([5], [260], 8),                        # more heads than one packed tile holds
])
def test_chain_small(tokens, contexts, heads):
    d = workloads.nvfp4_prefill_inputs("nvfp4-prefill-small", 100 + sum(contexts) + heads,
                                       tokens, contexts, heads)
    announce(f"nvfp4 prefill chain tokens={tokens} contexts={contexts} heads={heads}")
    keys_gpu = gather_gpu(d)
    keys_ora = gather_oracle(d)
    assert np.array_equal(host(keys_gpu), keys_ora), "gathered E4M3 keys differ"
    t0 = 0
    for b, (scores, ids) in enumerate(run_chain(d, keys_gpu)):
        T, N = int(d.tokens[b]), int(d.context[b])
        got = host(scores)
        ones = np.ones(N, dtype=np.float32)
        k_ora = request_keys(keys_ora, d, b)
        want = oracle.score_prefill(d.q[t0:t0 + T], d.q_scale[t0:t0 + T], k_ora, ones)
        mag = prefill_term_magnitude(d.q[t0:t0 + T], d.q_scale[t0:t0 + T], k_ora, ones)
        check_scores(got[:, :N], want, mag, f"request {b}")
        assert (got[:, N:].view(np.int32) == CANARY_F32.view(np.int32)).all(), "store past context"
        assert np.array_equal(host(ids), oracle.topk16(got[:, :N])), f"request {b}: top-16 differ"
        t0 += T


@pytest.mark.timeout(600)
def test_chain_long_context_rows_of_every_wave():
    """A 2,048-token chunk with 4 heads against a 65,536-token context (512
    pages), in the benchmark's launch configuration (16 tokens per wave,
    eight waves per work-group, 16 token groups): every gathered byte; two
    full score rows from every (token group, wave), their positions in the
    wave cycling through all 16; and the top-16 of all 2,048 rows against
    the oracle's selection over the GPU's own scores."""
    d = workloads.nvfp4_prefill()
    announce("nvfp4 prefill 2048 x 4 heads x 65536 keys")
    keys_gpu = gather_gpu(d, extra_pages=0)
    keys_ora = gather_oracle(d, extra_pages=0)
    assert np.array_equal(host(keys_gpu), keys_ora), "gathered E4M3 keys differ"
    (scores, ids), = run_chain(d, keys_gpu)
    N = int(d.context[0])
    got_all = host(scores)
    assert (got_all[:, N:].view(np.int32) == CANARY_F32.view(np.int32)).all()
    rows = sorted({128 * g + 16 * w + (8 * g + w + 8 * r) % 16
                   for g in range(16) for w in range(8) for r in range(2)})
    assert len(rows) == 256
    got = got_all[rows]
    k_ora = request_keys(keys_ora, d, 0)
    ones = np.ones(N, dtype=np.float32)
    want = oracle_pool.score_prefill_rows(d.q, d.q_scale, k_ora, ones, rows)
    mag = prefill_term_magnitude(d.q[rows], d.q_scale[rows], k_ora, ones)
    check_scores(got[:, :N], want, mag, "long-context prefill")
    assert np.array_equal(host(ids), oracle_pool.topk16(got_all[:, :N])), "top-16 differ"


def test_chain_ragged_causal_batch():
    """The whole batch in one causal launch: the gathered pages of all
    requests are one key buffer (request b's keys start at page_offsets[b] x
    128), each request's queries are the last tokens of its context, and each
    row keeps the 16 best of its visible keys."""
    import page_scoring_top_amd as ps
    d = workloads.nvfp4_prefill_inputs("nvfp4-prefill-ragged", 77, [37, 100, 1, 64],
                                       [1000, 3000, 129, 64])
    announce("nvfp4 prefill chain, ragged causal batch")
    keys_gpu = gather_gpu(d, extra_pages=0)
    keys_ora = gather_oracle(d, extra_pages=0)
    assert np.array_equal(host(keys_gpu), keys_ora), "gathered E4M3 keys differ"
    T = int(d.tokens.sum())
    q_start = np.concatenate([[0], np.cumsum(d.tokens)]).astype(np.int32)
    k_start = (d.page_offsets * 128).astype(np.int32)
    N = d.total_pages * 128
    width = int(d.context.max()) + 3
    ones = np.ones(N, dtype=np.float32)
    scores = torch.full((T, width + 2), float(CANARY_F32), dtype=torch.float32, device="cuda")
    row_len = torch.empty(T, dtype=torch.int32, device="cuda")
    ps.indexer_score_prefill_ragged(dev(d.q), dev(d.q_scale), keys_gpu.view(-1, 128), dev(ones),
                                    dev(q_start), dev(k_start), dev(d.context),
                                    int(d.tokens.max()), width, scores, row_len)
    ids = torch.full((T, 16), int(CANARY_I32), dtype=torch.int32, device="cuda")
    ps.topk16_select(scores, width, ids, valid_len=row_len)
    got, got_len, got_ids = host(scores), host(row_len), host(ids)
    want, want_len = oracle.score_prefill_ragged(d.q, d.q_scale, keys_ora.reshape(-1, 128), ones,
                                                 q_start, k_start, d.context, width)
    assert np.array_equal(got_len, want_len), "row lengths differ"
    assert np.array_equal(np.isneginf(got[:, :width]), np.isneginf(want)), "causal mask differs"
    assert (got[:, width:].view(np.int32) == CANARY_F32.view(np.int32)).all(), "write past width"
    for s in range(len(d.tokens)):
        rows = slice(q_start[s], q_start[s + 1])
        kl = int(d.context[s])
        k_ora = keys_ora.reshape(-1, 128)[k_start[s]:k_start[s] + kl]
        mag = prefill_term_magnitude(d.q[rows], d.q_scale[rows], k_ora, ones[:kl])
        g, w = got[rows, :kl], want[rows, :kl]
        vis = ~np.isneginf(w)
        check_scores(g[vis], w[vis], mag[vis], f"request {s}")
    assert np.array_equal(got_ids, oracle.topk16(got[:, :width], valid_len=want_len))
