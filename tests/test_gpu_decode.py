"""GPU parity of indexer_score_decode against the oracle.

Scores within |gpu - oracle| <= 1e-6 + 1e-5 |oracle| (NaN meets NaN), own
pages exact, and every entry the call must not write (columns at or past a
row's own page, rows without a query, padding requests) bit-unchanged.
"""

import numpy as np
import pytest
import torch

import oracle
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


def check_full(d, got_scores, got_own):
    want_own = expected_own(d)
    assert np.array_equal(got_own, want_own), "row_own differs"
    want = np.full(got_scores.shape, CANARY_F32, np.float32)
    want[:d.num_reqs], _ = oracle.score_decode(d.kv_cache, d.block_table, d.seq_lens, d.q,
                                               d.q_scale, d.num_reqs, d.qlen, d.width,
                                               scores=want[:d.num_reqs].copy())
    m = written_mask(d, want_own)
    assert np.array_equal(got_scores[~m].view(np.int32), want[~m].view(np.int32)), \
        "an entry outside the stored region was written"
    assert_scores_close(got_scores[m], want[m], d.name)


def check_sampled(d, got_scores, got_own, columns):
    want_own = expected_own(d)
    assert np.array_equal(got_own, want_own), "row_own differs"
    m = written_mask(d, want_own)
    assert (got_scores[~m].view(np.int32) == CANARY_F32.view(np.int32)).all(), \
        "an entry outside the stored region was written"
    assert not (got_scores[m].view(np.int32) == CANARY_F32.view(np.int32)).any(), \
        "an entry of the stored region was not written"
    for b, j in columns:
        col, stored = oracle.score_decode_column(d.kv_cache, d.block_table, d.seq_lens, d.q,
                                                 d.q_scale, d.qlen, d.width, b, j)
        assert np.array_equal(stored, m[b, :, j])
        assert_scores_close(got_scores[b, stored, j], col[stored], f"{d.name} b={b} j={j}")


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


def test_mtp_config():
    d = workloads.mtp_decode()
    announce("decode mtp (16 req x 8 slots, 30,000 tokens)")
    s, own = run_decode(d)
    rng = np.random.default_rng(0)
    cols = [(0, j) for j in range(0, 234, 9)] + \
           [(int(rng.integers(0, 16)), int(rng.integers(0, 234))) for _ in range(24)] + \
           [(15, 233), (7, 0)]
    check_sampled(d, s, own, cols)


def test_ragged_config_with_padding_requests():
    d = workloads.ragged_decode()
    announce("decode ragged (64 req + 8 padding, width 1344)")
    s, own = run_decode(d)
    rng = np.random.default_rng(1)
    cols = []
    for b in rng.choice(64, size=12, replace=False):
        npg = min(oracle.decode_pages(int(d.seq_lens[b])), d.width)
        cols += [(int(b), 0), (int(b), npg - 1), (int(b), int(rng.integers(0, npg)))]
    check_sampled(d, s, own, cols)
    assert (s[64:].view(np.int32) == CANARY_F32.view(np.int32)).all()
    assert (own[64:] == CANARY_I32).all()


def test_long_config_sampled_and_deterministic():
    """The 500,000-token configuration in the launch configuration the benchmark
    times; sampled columns against the oracle, every write region checked, and
    two runs bit-identical."""
    d = workloads.long_decode()
    announce("decode long (4 req x 8 slots, 500,000 tokens)")
    (s1, s2), own = run_decode(d, repeat=2)
    assert np.array_equal(s1.view(np.int32), s2.view(np.int32)), "not deterministic"
    rng = np.random.default_rng(2)
    cols = [(b, j) for b in range(4) for j in (0, 1, 1234, 3905)] + \
           [(int(rng.integers(0, 4)), int(rng.integers(0, 3906))) for _ in range(12)]
    check_sampled(d, s1, own, cols)
