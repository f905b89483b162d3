"""indexer_prefill_topk16, the top-16 of every prefill score row without the
score matrix, against the two-call chain it replaces: for every query row it
must return exactly what topk16_select returns on the scores
indexer_score_prefill writes from the same inputs (its rescoring repeats the
score kernel's arithmetic bit for bit, and its selection is exact), and on
sampled rows exactly what the oracle's top-16 of those scores is.  Shapes
cover both score-kernel layouts (up to four heads packed into the MFMA rows,
one token per wave above), ragged token and key counts, and the inputs that
make many blocks tie (equal scores, zeros, NaN, infinities, signed scales)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu


def _chain(q, qs, k, ks):
    import page_scoring_top_amd as ps
    T, N = q.shape[0], k.shape[0]
    scores = torch.empty((T, N), dtype=torch.float32, device="cuda")
    ps.indexer_score_prefill(q, qs, k, ks, scores)
    out = torch.empty((T, 16), dtype=torch.int32, device="cuda")
    ps.topk16_select(scores, N, out)
    return scores, out


def _fused(q, qs, k, ks, out_cols=16):
    import page_scoring_top_amd as ps
    T, N = q.shape[0], k.shape[0]
    out = torch.full((T, out_cols), -7, dtype=torch.int32, device="cuda")
    ws = ps.prefill_topk16_workspace(T, N, "cuda")
    ws.fill_(0xA5)                          # stale contents must not matter
    ps.indexer_prefill_topk16(q, qs, k, ks, out, ws)
    return out


def _check(name, q, qs, k, ks, oracle_rows=6):
    """Fused == chain on every row; == oracle top-16 of the chain's scores on
    `oracle_rows` rows spread over the batch."""
    T = q.shape[0]
    announce(f"prefill top-16 {name}: T={T} H={q.shape[1]} N={k.shape[0]}")
    scores, want = _chain(q, qs, k, ks)
    got = _fused(q, qs, k, ks)
    g, w = host(got), host(want)
    bad = np.nonzero((g != w).any(axis=1))[0]
    assert bad.size == 0, f"{name}: {bad.size} rows differ, first {bad[:5]}: {g[bad[0]]} vs {w[bad[0]]}"
    rows = np.unique(np.linspace(0, T - 1, min(oracle_rows, T)).astype(np.int64))
    ora = oracle.topk16(host(scores[torch.from_numpy(rows).cuda()]))
    assert np.array_equal(g[rows], ora), f"{name}: differs from the oracle's top-16 of the scores"


def _inputs(name, seed, T, H, N):
    p = workloads.prefill_inputs(name, seed, T, H, N)
    return p.q, p.q_scale, p.k, p.k_scale


SHAPES = [
    # (T, H, N): packed layout (H <= 4) with one or two 8-token tiles per wave,
    # then the one-token layout with one or two 32-head tiles; key counts
    # below one block group, at and past group boundaries, below 16.
    (1, 1, 1), (3, 4, 15), (5, 4, 16), (17, 4, 1000), (70, 4, 1025), (130, 3, 5000),
    (9, 5, 3000), (8, 32, 2100), (11, 33, 4097), (6, 64, 2048), (200, 2, 9000),
]


@pytest.mark.parametrize("T,H,N", SHAPES)
def test_random_inputs(T, H, N):
    q, qs, k, ks = _inputs(f"ptk-{T}-{H}-{N}", 40 + T + H, T, H, N)
    _check(f"random {T}x{H}x{N}", dev(q), dev(qs), dev(k), dev(ks))


@pytest.mark.parametrize("H", [4, 64])
def test_every_score_equal(H):
    """One key repeated: every row's scores tie, so every block qualifies and
    all 5,000 keys survive the filter (the compaction path); the answer is
    columns 0..15."""
    T, N = 12, 5000
    q, qs, k, ks = _inputs(f"ptk-eq-{H}", 61, T, H, N)
    k = np.repeat(k[:1], N, axis=0)
    ks = np.full(N, 1.25, np.float32)
    got = _fused(dev(q), dev(qs), dev(k), dev(ks))
    assert np.array_equal(host(got), np.tile(np.arange(16, dtype=np.int32), (T, 1)))
    _check(f"all equal H={H}", dev(q), dev(qs), dev(k), dev(ks))


@pytest.mark.parametrize("H", [4, 40])
def test_special_values(H):
    """NaN key scales and a NaN row (NaN ranks lowest), a zero query (every
    score 0, ties), infinite key scales, negative query scales (negative
    scores) and negative key scales (-0 against +0)."""
    T, N = 20, 3100
    q, qs, k, ks = _inputs(f"ptk-sp-{H}", 62, T, H, N)
    ks = ks.copy()
    qs = qs.copy()
    q = q.copy()
    ks[::7] = np.nan
    ks[5:40:9] = np.inf
    ks[1000:1100] = -ks[1000:1100]
    qs[1, :] = np.nan            # row 1: every score NaN -> columns 0..15
    q[2] = 0                     # row 2: every score 0 (or NaN where k_scale is) -> ties
    qs[3, ::2] = -qs[3, ::2]     # row 3: signed head weights
    qs[4, :] = -1.0              # row 4: every score <= 0
    _check(f"special H={H}", dev(q), dev(qs), dev(k), dev(ks), oracle_rows=T)


def test_wide_out_stride_and_short_rows():
    """out rows wider than 16 keep their other entries; N < 16 pads with -1."""
    import page_scoring_top_amd as ps
    T, H, N = 7, 4, 9
    q, qs, k, ks = _inputs("ptk-short", 63, T, H, N)
    announce("prefill top-16 short rows, out stride 24")
    out = torch.full((T, 24), -7, dtype=torch.int32, device="cuda")
    ps.indexer_prefill_topk16(dev(q), dev(qs), dev(k), dev(ks), out,
                              ps.prefill_topk16_workspace(T, N, "cuda"))
    o = host(out)
    assert (o[:, 16:] == -7).all()
    assert (o[:, N:16] == -1).all()
    s, want = _chain(dev(q), dev(qs), dev(k), dev(ks))
    assert np.array_equal(o[:, :16], host(want))


def test_lightning_indexer_config():
    """2,048 tokens x 64 heads against 16,384 keys (the prefill configuration)."""
    p = workloads.big_prefill()
    _check("2048x64x16384", dev(p.q), dev(p.q_scale), dev(p.k), dev(p.k_scale), oracle_rows=8)


def test_nvfp4_prefill_chain():
    """The NVFP4 prefill: 512 pages gathered to E4M3 keys (65,536), 2,048
    tokens x 4 heads, unit key scales."""
    import page_scoring_top_amd as ps
    d = workloads.nvfp4_prefill()
    N = int(d.context[0])
    keys = torch.empty((d.total_pages, 128, 128), dtype=torch.uint8, device="cuda")
    ps.nvfp4_index_k_dequant(dev(d.kv_cache), dev(d.block_table), dev(d.num_pages),
                             dev(d.page_offsets), d.block_table.shape[1], keys)
    ones = torch.ones(N, dtype=torch.float32, device="cuda")
    _check("nvfp4 2048x4x65536", dev(d.q), dev(d.q_scale), keys.view(-1, 128)[:N].contiguous(), ones,
           oracle_rows=8)


@pytest.mark.parametrize("H", [1, 4, 64])
def test_two_best_keys_in_one_block_with_nan_between(H):
    """A block (the keys 5 + 32 i of the first 1,024) holding the row's two
    best keys, at i = 3 and i = 20, with NaN scores at i = 0 and i = 10 of
    the same block: the block's second largest score must survive the NaNs,
    or the second best key would be missed.  Every other key scores the
    same (ties to the lowest columns)."""
    T, N = 3, 2048
    one = 0x38                                     # E4M3 1.0: every dot is 128
    q = np.full((T, H, 128), one, np.uint8)
    k = np.full((N, 128), one, np.uint8)
    qs = np.ones((T, H), np.float32)
    ks = np.ones(N, np.float32)
    ks[5 + 32 * 3] = 100.0
    ks[5 + 32 * 20] = 90.0
    ks[5 + 32 * 0] = np.nan
    ks[5 + 32 * 10] = np.nan
    got = host(_fused(dev(q), dev(qs), dev(k), dev(ks)))
    rest = [c for c in range(N) if c not in (5, 5 + 320, 101, 645)][:14]
    assert (got == np.array([101, 645] + rest, np.int32)).all(), got[0]
    _check(f"two best in one block H={H}", dev(q), dev(qs), dev(k), dev(ks), oracle_rows=T)
