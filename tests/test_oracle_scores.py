"""Pins of the oracle's decode and prefill scores.

Checks against things other than the oracle itself:
  * exact rational dot products (fractions) -- the double-precision dot is
    exact because every partial sum needs at most 43 significant bits;
  * the relu identity and its special cases;
  * closed forms: one-hot queries read a single dequantized element, all-ones
    queries and keys give 128 * q_scale, mixed-sign heads drop out of the
    prefill head sum, per-row scales land on their own rows;
  * torch CPU matmul (a library routine) for H = 1 with unit scales;
  * the decode/prefill consistency stated on the gather page (both modes rank
    pages from identical keys): a decode page score is the maximum over the
    page's tokens of the one-head prefill score on the dequantized page;
  * the decode geometry fixture (tests/golden/decode_geometry.txt).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e4m3_frac(b):
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    mag = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if s else mag


def _finite_e4m3_bytes(rng, n):
    b = rng.integers(0, 256, size=n).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x7E
    return b


def test_dot_is_exact():
    rng = np.random.default_rng(0)
    for trial in range(200):
        a = _finite_e4m3_bytes(rng, 128)
        b = _finite_e4m3_bytes(rng, 128)
        if trial % 4 == 0:   # wide dynamic range: large and tiny magnitudes together
            a[:64] = 0x7E
            b[:64] = rng.choice([0x7E, 0xFE], size=64)
        exact = sum(_e4m3_frac(int(x)) * _e4m3_frac(int(y)) for x, y in zip(a, b))
        assert Fraction(oracle.dot_e4m3(a, b)) == exact


def test_relu_identity():
    rng = np.random.default_rng(1)
    for x in list(rng.standard_normal(1000) * 1e3) + [0.0, -0.0, 1e300, -1e300, 5e-324, -5e-324]:
        r = oracle.relu(x)
        assert r == max(x, 0.0)
        assert math.copysign(1, r) == 1.0  # -0 and negatives become +0
    assert math.isnan(oracle.relu(float("nan")))
    assert oracle.relu(float("inf")) == float("inf")


def _one_page_inputs(page, q_bytes, q_scale, seq_len=129, qlen=8, width=8):
    """One request whose every logical page is `page` (physical page 0)."""
    kv = page.reshape(1, 9216)
    bt = np.zeros((1, width), dtype=np.int32)
    return kv, bt, np.array([seq_len], dtype=np.int32), q_bytes, q_scale


def test_decode_one_hot_query_reads_dequantized_elements():
    rng = np.random.default_rng(2)
    page = workloads.random_pages(rng, rng, 1)[0]
    page[8192:] = rng.integers(0, 256, size=1024)  # every scale byte, NaN and negatives too
    k = oracle.dequant_page(page)
    kval = torch.from_numpy(k.copy()).view(torch.float8_e4m3fn).double().numpy()
    for d in (0, 1, 15, 16, 77, 126, 127):
        q = np.zeros((1, 8, 4, 128), dtype=np.uint8)
        q[0, 7, :, d] = 0x38  # 1.0 in slot 7, every head
        qs = np.linspace(0.5, 2.0, 32, dtype=np.float32).reshape(1, 8, 4)
        kv, bt, sl, q, qs = _one_page_inputs(page, q, qs, seq_len=129, qlen=1, width=2)
        col, stored = oracle.score_decode_column(kv, bt, sl, q, qs, 1, 2, 0, 0)
        assert stored.tolist() == [False] * 28 + [True] * 4
        colk = kval[:, d]
        for h in range(4):
            if np.isnan(colk).any():
                assert math.isnan(col[28 + h])
            else:
                want = np.float32(max(0.0, colk.max()) * np.float64(qs[0, 7, h]))
                assert col[28 + h] == want


def test_decode_all_ones_and_row_scales():
    page = np.zeros(9216, dtype=np.uint8)
    page[:8192] = 0x22           # both nibbles: code 2 = 1.0
    page[8192:] = 0x38           # scale 1.0
    q = np.full((1, 8, 4, 128), 0x38, dtype=np.uint8)
    q[0, 3, 2, :] = 0xB8         # slot 3, head 2: all -1 -> every dot is -128 -> relu 0
    qs = (np.arange(32, dtype=np.float32) / 8 + 0.25).reshape(1, 8, 4)
    kv, bt, sl, q, qs = _one_page_inputs(page, q, qs, seq_len=1000, qlen=8)
    scores, own = oracle.score_decode(kv, bt, sl, q, qs, 1, 8, 8)
    # seq_len 1000: pos 992..999 -> own page 7 for every slot; 7 pages scored
    assert (own == 7).all()
    for row in range(32):
        want = 0.0 if row == 3 * 4 + 2 else np.float32(128.0 * float(qs.reshape(32)[row]))
        assert (scores[0, row, :7] == want).all(), row
        assert np.isnan(scores[0, row, 7])   # the own page is not stored


def test_prefill_closed_forms():
    rng = np.random.default_rng(4)
    T, H, N = 3, 5, 7
    q = np.full((T, H, 128), 0x38, dtype=np.uint8)
    sign = rng.integers(0, 2, size=(T, H))
    q[sign == 1] = 0xB8                              # heads with q = -1 contribute 0
    k = np.full((N, 128), 0x38, dtype=np.uint8)
    qs = rng.uniform(0.5, 2.0, size=(T, H)).astype(np.float32)
    ks = rng.uniform(0.5, 2.0, size=(N,)).astype(np.float32)
    s = oracle.score_prefill(q, qs, k, ks)
    for t in range(T):
        hs = sum(128.0 * float(qs[t, h]) for h in range(H) if sign[t, h] == 0)
        for n in range(N):
            assert s[t, n] == np.float32(float(ks[n]) * hs)


def test_prefill_one_head_matches_torch_matmul():
    rng = np.random.default_rng(5)
    T, N = 9, 33
    q = workloads.e4m3_bytes_from_normal(rng, (T, 1, 128))
    k = workloads.e4m3_bytes_from_normal(rng, (N, 128))
    s = oracle.score_prefill(q, np.ones((T, 1), np.float32), k, np.ones(N, np.float32))
    qf = torch.from_numpy(q.reshape(T, 128)).view(torch.float8_e4m3fn).double()
    kf = torch.from_numpy(k).view(torch.float8_e4m3fn).double()
    want = torch.relu(qf @ kf.T).float().numpy()
    assert np.array_equal(s, want)


def test_decode_equals_max_of_one_head_prefill():
    d = workloads.tiny_decode(seed=7)
    b, slot, qlen = 0, 7, 1
    for j in (0, 17, 62):
        col, stored = oracle.score_decode_column(d.kv_cache, d.block_table, d.seq_lens, d.q,
                                                 d.q_scale, qlen, d.width, b, j)
        kpage = oracle.dequant_page(d.kv_cache[d.block_table[b, j]])
        for h in range(4):
            qv = d.q[b, slot, h].reshape(1, 1, 128)
            qsv = d.q_scale[b, slot, h].reshape(1, 1)
            pre = oracle.score_prefill(qv, qsv, kpage, np.ones(128, np.float32))
            assert stored[slot * 4 + h]
            assert col[slot * 4 + h] == pre.max()


def test_decode_geometry_fixture():
    n = 0
    with open(os.path.join(GOLDEN, "decode_geometry.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(x) for x in line.split()]
            seq, qlen, pages, own = v[0], v[1], v[2], v[3:]
            assert oracle.decode_pages(seq) == pages, line
            assert [oracle.decode_own(seq, qlen, s) for s in range(8)] == own, line
            n += 1
    assert n >= 8


def test_decode_writes_only_below_own_page():
    """Columns at or past a row's own page, rows without a query and columns
    past the width keep their previous contents."""
    d = workloads.decode_inputs("geom", 9, [129, 3, 600, 0], qlen=8, width=4)
    canary = np.float32(-12345.0)
    scores = np.full((4, 32, 4), canary, dtype=np.float32)
    scores, own = oracle.score_decode(d.kv_cache, d.block_table, d.seq_lens, d.q, d.q_scale,
                                      4, 8, 4, scores=scores)
    for b in range(4):
        for row in range(32):
            o = own[b, row]
            seq = int(d.seq_lens[b])
            assert o == oracle.decode_own(seq, 8, row // 4)
            limit = min(max(o, 0), 4, oracle.decode_pages(seq))
            assert (scores[b, row, :limit] != canary).all()
            assert (scores[b, row, limit:] == canary).all()


def test_prefill_rows_equal_the_full_prefill():
    """score_prefill_rows, the checker of sampled rows, is the full score
    restricted to the rows asked for: same bits, in the order asked
    (repeated and unsorted rows included)."""
    p = workloads.prefill_inputs("rows", 12, 11, 6, 45)
    full = oracle.score_prefill(p.q, p.q_scale, p.k, p.k_scale)
    rows = [10, 0, 3, 3, 7, 1, 10]
    got = oracle.score_prefill_rows(p.q, p.q_scale, p.k, p.k_scale, rows)
    assert np.array_equal(got.view(np.int32), full[rows].view(np.int32))


def test_prefill_rows_exact_rational():
    """score_prefill_rows against an exact rational evaluation of
    k_scale * sum_h relu(q_h . k) * q_scale_h on wide-range E4M3 inputs with
    signed scales; the oracle rounds its double head sum once to float, so
    it must be the float nearest to the exact value or a neighbour of it
    (the double sum may sit on the other side of a float midpoint)."""
    rng = np.random.default_rng(13)
    T, H, N = 4, 3, 9
    q = _finite_e4m3_bytes(rng, T * H * 128).reshape(T, H, 128)
    k = _finite_e4m3_bytes(rng, N * 128).reshape(N, 128)
    qs = rng.uniform(-2.0, 2.0, size=(T, H)).astype(np.float32)
    ks = rng.uniform(-2.0, 2.0, size=(N,)).astype(np.float32)
    rows = [2, 0, 3]
    got = oracle.score_prefill_rows(q, qs, k, ks, rows)
    for i, t in enumerate(rows):
        for n in range(N):
            acc = Fraction(0)
            for h in range(H):
                dot = sum(_e4m3_frac(int(a)) * _e4m3_frac(int(b)) for a, b in zip(q[t, h], k[n]))
                acc += max(dot, Fraction(0)) * Fraction(float(qs[t, h]))
            exact = Fraction(float(ks[n])) * acc
            g = np.float32(got[i, n])
            lo, hi = np.nextafter(g, np.float32(-np.inf)), np.nextafter(g, np.float32(np.inf))
            assert Fraction(float(lo)) <= exact <= Fraction(float(hi)), (t, n)
            # and it is within half a float ulp plus the double rounding
            assert abs(Fraction(float(g)) - exact) <= (Fraction(float(hi)) - Fraction(float(g))) \
                * Fraction(1, 2) * (1 + Fraction(1, 2 ** 20)) + abs(exact) * Fraction(1, 2 ** 50)
