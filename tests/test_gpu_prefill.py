"""GPU parity of indexer_score_prefill against the oracle
(|gpu - oracle| <= 1e-6 + 1e-5 |oracle|, NaN meets NaN)."""

import numpy as np
import pytest
import torch

import oracle
import oracle_pool
import workloads
from gpu_util import CANARY_F32, announce, assert_scores_close, dev, host

pytestmark = pytest.mark.gpu


def gpu_prefill(p: workloads.PrefillInputs, ld=None):
    import page_scoring_top_amd as ps
    T, N = p.q.shape[0], p.k.shape[0]
    ld = N if ld is None else ld
    out = torch.full((T, ld), float(CANARY_F32), dtype=torch.float32, device="cuda")
    ps.indexer_score_prefill(dev(p.q), dev(p.q_scale), dev(p.k), dev(p.k_scale), out)
    return host(out)


@pytest.mark.parametrize("T,H,N", [(1, 1, 1), (3, 1, 33), (5, 3, 64), (7, 32, 100), (9, 33, 31),
                                   (17, 64, 257), (4, 65, 130),
                                   # many 128-key chunks, a ragged last chunk and token
                                   # group, key ranges split over several work-groups
                                   (13, 48, 1000), (2, 64, 5000), (8, 64, 128), (9, 1, 129),
                                   # up to four heads, eight tokens per wave: ragged last
                                   # wave and work-group, several token groups
                                   (67, 4, 1000), (130, 2, 300), (513, 4, 2000), (64, 4, 128)])
def test_small_shapes_full(T, H, N):
    p = workloads.prefill_inputs("small", T * 1000 + H * 10 + N, T, H, N)
    announce(f"prefill T={T} H={H} N={N}")
    got = gpu_prefill(p, ld=N + 3)
    want = oracle.score_prefill(p.q, p.q_scale, p.k, p.k_scale)
    assert_scores_close(got[:, :N], want, f"T={T} H={H} N={N}")
    assert (got[:, N:].view(np.int32) == CANARY_F32.view(np.int32)).all()


def test_scale_edges():
    p = workloads.prefill_inputs("edges", 5, 6, 8, 40)
    p.q_scale[1, :] = 0.0
    p.q_scale[2, 3] = -1.5            # negative scales are just multipliers here
    p.k_scale[7] = 0.0
    p.k_scale[8] = -2.0
    announce("prefill scale edges")
    got = gpu_prefill(p)
    want = oracle.score_prefill(p.q, p.q_scale, p.k, p.k_scale)
    assert_scores_close(got, want, "scale edges")


def test_nan_inputs_propagate():
    p = workloads.prefill_inputs("nan", 6, 4, 4, 64)
    p.q[1, 2, 5] = 0x7F               # token 1: NaN through head 2
    p.k[9, 100] = 0xFF                # key 9: NaN for every token
    announce("prefill NaN inputs")
    got = gpu_prefill(p)
    want = oracle.score_prefill(p.q, p.q_scale, p.k, p.k_scale)
    assert np.isnan(want[1]).all() and np.isnan(want[:, 9]).all()
    assert_scores_close(got, want, "nan inputs")


@pytest.mark.timeout(600)
def test_big_config_rows_of_every_group():
    """2,048 tokens x 64 heads x 16,384 keys in the benchmark's launch
    configuration (one token per wave, eight waves per work-group, 256
    work-groups over all keys): one full row from every work-group, the
    wave position cycling through all eight, against the oracle."""
    p = workloads.big_prefill()
    announce("prefill 2048 x 64 x 16384")
    got = gpu_prefill(p)
    assert np.isfinite(got).all()
    rows = [8 * g + (g % 8) for g in range(256)]
    want = oracle_pool.score_prefill_rows(p.q, p.q_scale, p.k, p.k_scale, rows)
    assert_scores_close(got[rows], want, "big prefill")


def test_most_heads():
    """224 heads, the most one call takes (a work-group holds one token's
    query rows as f16 in its LDS)."""
    p = workloads.prefill_inputs("max-heads", 224, 5, 224, 300)
    announce("prefill T=5 H=224 N=300")
    got = gpu_prefill(p, ld=301)
    want = oracle.score_prefill(p.q, p.q_scale, p.k, p.k_scale)
    assert_scores_close(got[:, :300], want, "H=224")
    assert (got[:, 300:].view(np.int32) == CANARY_F32.view(np.int32)).all()
