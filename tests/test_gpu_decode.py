"""GPU parity of indexer_score_decode against the oracle.

Every stored score within |gpu - oracle| <= 1e-6 + 1e-5 |oracle| (NaN meets
NaN), own pages exact, and every entry the call must not write (columns at
or past a row's own page, rows without a query, padding requests, pages
whose id is out of range) bit-unchanged.  The large configurations are
compared in full too: the oracle runs on host threads (tests/oracle_pool.py).
"""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import workloads
from gpu_util import CANARY_F32, CANARY_I32, announce, assert_scores_close, dev, host

pytestmark = pytest.mark.gpu


def run_decode(d: workloads.DecodeInputs, repeat: int = 1):
    import page_scoring_top_amd as ps
    Rt = d.q.shape[0]
    scores = torch.full((Rt, 32, d.width), float(CANARY_F32), dtype=torch.float32, device="cuda")
    own = torch.full((Rt, 32), int(CANARY_I32), dtype=torch.int32, device="cuda")
    kv, bt, sl, q, qs = dev(d.kv_cache), dev(d.block_table), dev(d.seq_lens), dev(d.q), dev(d.q_scale)
    outs = []
    for _ in range(repeat):
        ps.indexer_score_decode(kv, bt, sl, q, qs, d.qlen, d.width, scores, own, num_reqs=d.num_reqs)
        outs.append(host(scores).copy())
    return outs if repeat > 1 else outs[0], host(own)


def expected_own(d):
    R = d.num_reqs
    own = np.full((d.q.shape[0], 32), CANARY_I32, np.int32)
    for b in range(R):
        for row in range(32):
            own[b, row] = oracle.decode_own(int(d.seq_lens[b]), d.qlen, row // 4)
    return own


def written_mask(d, own):
    """Entries the call must write: j < min(own, pages scored, width)."""
    Rt = d.q.shape[0]
    m = np.zeros((Rt, 32, d.width), bool)
    cols = np.arange(d.width)
    for b in range(d.num_reqs):
        npg = min(oracle.decode_pages(int(d.seq_lens[b])), d.width)
        for row in range(32):
            m[b, row] = cols < min(max(own[b, row], 0), npg)
    return m


def check_full(d, got_scores, got_own, pooled=False):
    """Every entry of the score buffer: stored ones against the oracle, the
    rest bit-unchanged.  ``pooled`` runs the oracle on host threads."""
    want_own = expected_own(d)
    assert np.array_equal(got_own, want_own), "row_own differs"
    base = np.full(got_scores.shape, CANARY_F32, np.float32)
    if pooled:
        want, stored = oracle_pool.score_decode(d, base=base)
    else:
        want = base
        want[:d.num_reqs], _ = oracle.score_decode(d.kv_cache, d.block_table, d.seq_lens, d.q,
                                                   d.q_scale, d.num_reqs, d.qlen, d.width,
                                                   scores=want[:d.num_reqs].copy())
        stored = None
    m = written_mask(d, want_own)
    if stored is not None:
        assert np.array_equal(stored, m), "the oracle's stored region differs from the geometry"
    assert np.array_equal(got_scores[~m].view(np.int32), want[~m].view(np.int32)), \
        "an entry outside the stored region was written"
    assert_scores_close(got_scores[m], want[m], d.name)
    return int(m.sum())


def test_tiny_config_full():
    d = workloads.tiny_decode()
    announce("decode tiny (1 req, qlen 1, 64 pages)")
    s, own = run_decode(d)
    check_full(d, s, own)
    assert (own[0, :28] == -1).all() and (own[0, 28:] == 63).all()


@pytest.mark.parametrize("qlen", [1, 2, 3, 5, 7, 8])
def test_geometry_edges_full(qlen):
    """Contexts around page boundaries, shorter than qlen, empty, and longer than
    the width (pages past the width are never scored)."""
    seqs = [0, 1, 3, 127, 128, 129, 255, 256, 257, 1000, 2300]
    d = workloads.decode_inputs(f"edges-q{qlen}", 100 + qlen, seqs, qlen=qlen, width=11,
                                pad_reqs=2)
    announce(f"decode geometry edges qlen={qlen}")
    s, own = run_decode(d)
    check_full(d, s, own)


def test_special_values_full():
    """Every scale byte (negative, zero, subnormal, NaN), NaN query bytes, zero
    q_scale: NaN must propagate to the whole page or row, signs must flip."""
    d = workloads.decode_inputs("special", 7, [1500, 1200, 900], qlen=8, width=12,
                                scale_low=0, scale_high=255)
    d.q[0, 3, 1, 17] = 0x7F          # NaN query byte: row 13 of request 0 is NaN everywhere
    d.q[1, 6, 2, 100] = 0xFF
    d.q_scale[2, 5, 0] = 0.0
    d.q_scale[2, 4, 3] = np.nan
    announce("decode special values")
    s, own = run_decode(d)
    check_full(d, s, own)
    assert np.isnan(s[0, 13, :own[0, 13]]).all()


def test_all_nan_free_scales_with_negatives():
    """Scales drawn from all finite bytes of both signs (no NaN)."""
    d = workloads.decode_inputs("signed", 8, [2000, 700], qlen=4, width=16, scale_low=0,
                                scale_high=255)
    nanb = (d.kv_cache[:, 8192:] & 0x7F) == 0x7F
    d.kv_cache[:, 8192:][nanb] = 0xC0
    announce("decode signed scales")
    s, own = run_decode(d)
    check_full(d, s, own)


def test_mtp_config_full():
    """16 requests x 8 slots at 30,000 tokens: all 512 rows x 234 pages."""
    d = workloads.mtp_decode()
    announce("decode mtp (16 req x 8 slots, 30,000 tokens), every score")
    s, own = run_decode(d)
    assert check_full(d, s, own, pooled=True) == 16 * 32 * 234


def test_ragged_config_full_with_padding_requests():
    """64 requests with contexts of 1,000..172,032 tokens and 8 padding
    requests, width 1,344: every stored score of the 2,048 real rows."""
    d = workloads.ragged_decode()
    announce("decode ragged (64 req + 8 padding, width 1344), every score")
    s, own = run_decode(d)
    n = check_full(d, s, own, pooled=True)
    assert n > 0
    assert (s[64:].view(np.int32) == CANARY_F32.view(np.int32)).all()
    assert (own[64:] == CANARY_I32).all()


def test_long_config_full_and_deterministic():
    """The 500,000-token configuration in the launch configuration the
    benchmark times: all 128 rows x 3,906 pages against the oracle, and two
    runs bit-identical."""
    d = workloads.long_decode()
    announce("decode long (4 req x 8 slots, 500,000 tokens), every score")
    (s1, s2), own = run_decode(d, repeat=2)
    assert np.array_equal(s1.view(np.int32), s2.view(np.int32)), "not deterministic"
    assert check_full(d, s1, own, pooled=True) == 4 * 32 * 3906


def test_out_of_range_page_ids_are_skipped():
    """Block-table ids below 0 or at and past num_blocks: such a page is not
    read and its column keeps its canaries in every row; every other column
    matches the oracle (which is given a valid id in their place)."""
    d = workloads.decode_inputs("bad-ids", 11, [3000, 2500, 1800], qlen=8, width=24)
    nb = d.num_blocks
    bad = {(0, 0): -1, (0, 5): nb, (0, 22): -2147483648, (1, 3): nb + 1000,
           (1, 18): 2147483647, (2, 7): -7, (2, 13): nb}
    bt_gpu = d.block_table.copy()
    for (b, j), v in bad.items():
        bt_gpu[b, j] = v
    announce("decode out-of-range page ids")
    import page_scoring_top_amd as ps
    scores = torch.full((3, 32, d.width), float(CANARY_F32), dtype=torch.float32, device="cuda")
    own = torch.full((3, 32), int(CANARY_I32), dtype=torch.int32, device="cuda")
    ps.indexer_score_decode(dev(d.kv_cache), dev(bt_gpu), dev(d.seq_lens), dev(d.q),
                            dev(d.q_scale), d.qlen, d.width, scores, own, num_reqs=3)
    got, got_own = host(scores), host(own)
    want_own = expected_own(d)
    assert np.array_equal(got_own, want_own)
    want, _ = oracle.score_decode(d.kv_cache, d.block_table, d.seq_lens, d.q, d.q_scale, 3,
                                  d.qlen, d.width,
                                  scores=np.full(got.shape, CANARY_F32, np.float32))
    m = written_mask(d, want_own)
    for (b, j) in bad:
        assert m[b, :, j].any(), "the test must put a bad id in a scored column"
        m[b, :, j] = False
    assert np.array_equal(got[~m].view(np.int32),
                          np.full(got.shape, CANARY_F32, np.float32)[~m].view(np.int32)), \
        "a column with an out-of-range id, or outside the stored region, was written"
    assert_scores_close(got[m], want[m], "bad ids")


def test_most_requests_in_one_call():
    """65,535 requests, the most one call takes (one grid row each): every
    request writes its own pages, 1 in 64 has two scored pages and the rest
    none; the pages are drawn from a shared pool of 64."""
    R, W = 65535, 2
    rng = np.random.default_rng(41)
    seq = np.where(np.arange(R) % 64 == 5, 300, 100).astype(np.int32)
    base = workloads.decode_inputs("max-reqs-pool", 41, [300], qlen=8, width=W, pool_pages=64)
    kv = base.kv_cache
    bt = rng.integers(0, kv.shape[0], size=(R, W), dtype=np.int32)
    q = workloads.e4m3_bytes_from_normal(rng, (R, 8, 4, 128))
    qs = rng.uniform(0.5, 2.0, size=(R, 8, 4)).astype(np.float32)
    d = workloads.DecodeInputs("max-reqs", kv, bt, seq, q, qs, 8, W, R)
    announce("decode 65,535 requests")
    s, own = run_decode(d)
    n = check_full(d, s, own, pooled=True)
    assert n == (R // 64 + (1 if R % 64 > 5 else 0)) * 32 * 2


@pytest.mark.timeout(900)
def test_flat_schedule_with_shares_over_64_pages():
    """A batch over one round of 8 pages per wave takes the flat schedule;
    here 38 requests of 3,492 scored pages each (132,696 pages, more than 64
    per wave on 2,048 waves), so each wave scores runs of 64 pages and some
    shares cross a request boundary.  Pages come from a shared pool of 4,096
    (ids repeat); every stored score is compared."""
    R, seq_len = 38, 447_000
    W = (seq_len + 127) // 128
    rng = np.random.default_rng(43)
    base = workloads.decode_inputs("flat-pool", 43, [300], qlen=8, width=4, pool_pages=4096)
    kv = base.kv_cache
    bt = rng.integers(0, kv.shape[0], size=(R, W), dtype=np.int32)
    q = workloads.e4m3_bytes_from_normal(rng, (R, 8, 4, 128))
    qs = rng.uniform(0.5, 2.0, size=(R, 8, 4)).astype(np.float32)
    seq = np.full(R, seq_len, np.int32)
    d = workloads.DecodeInputs("flat-long-runs", kv, bt, seq, q, qs, 8, W, R)
    announce("decode flat schedule, 38 x 3,492 pages")
    s, own = run_decode(d)
    n = check_full(d, s, own, pooled=True)
    assert n == R * 32 * (W - 1)
