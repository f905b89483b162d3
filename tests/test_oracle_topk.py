"""Pins of the oracle's exact top-16.

  * hand-built rows whose expected output follows from the ordering rules the
    MSA pull request states (tests/golden/key_order.json);
  * a brute-force pure-Python ranking (every candidate's rank is the number of
    candidates that beat it) on tiny random rows with special values;
  * the exact-merge property stated on the decode-CP page: the top 16 of a row
    lies in the union of the top 16s of any partition of its columns, so
    merging per-partition results gives the global result.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FLT_MAX = float(np.finfo(np.float32).max)
_SPECIAL = {"nan": float("nan"), "inf": float("inf"), "-inf": float("-inf"),
            "FLT_MAX": FLT_MAX, "-FLT_MAX": -FLT_MAX, "-0.0": -0.0}


def _val(s):
    return _SPECIAL[s] if s in _SPECIAL else float(s)


def test_golden_key_order():
    with open(os.path.join(GOLDEN, "key_order.json")) as f:
        cases = json.load(f)
    assert len(cases) >= 12
    for c in cases:
        s = np.array([[_val(x) for x in c["scores"]]], dtype=np.float32)
        kw = {}
        if "valid" in c:
            kw["valid_len"] = np.array([c["valid"]], np.int32)
        if "force" in c:
            kw["force_begin"] = np.array([c["force"][0]], np.int32)
            kw["force_end"] = np.array([c["force"][1]], np.int32)
        if "append" in c:
            kw["append_page"] = np.array([c["append"]], np.int32)
        got = oracle.topk16(s, **kw)[0].tolist()
        assert got == c["expected"], c["why"]


def _beats(a, b):
    """True when candidate a = (value, col, forced) ranks above b."""
    def v(x):
        s, _, forced = x
        if forced:
            return math.inf
        if math.isnan(s):
            return -math.inf
        return 0.0 if s == 0 else s
    va, vb = v(a), v(b)
    return va > vb or (va == vb and a[1] < b[1])


def _brute(row, valid, fb, fe, append):
    width = len(row)
    n = min(max(valid, 0), width)
    cands = [(float(row[c]), c, fb <= c < fe) for c in range(n)]
    rank = {c[1]: sum(_beats(o, c) for o in cands) for c in cands}
    k = 15 if append is not None else 16
    picked = sorted((r, col) for col, r in rank.items() if r < k)
    out = [col for _, col in picked]
    if append is not None and append >= 0:
        out.append(append)
    return out + [-1] * (16 - len(out))


def test_brute_force_tiny_rows():
    rng = np.random.default_rng(0)
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.5, np.inf, -np.inf, np.nan, FLT_MAX, -FLT_MAX],
                    dtype=np.float32)
    for width in list(range(1, 40)) + [63, 64, 65, 100, 127, 128, 129, 200]:
        for trial in range(4):
            rows = 8
            s = rng.standard_normal((rows, width)).astype(np.float32)
            mask = rng.random((rows, width)) < 0.3
            s[mask] = rng.choice(pool, size=mask.sum())
            if trial == 3:
                with np.errstate(over="ignore"):
                    s = np.round(s * 2) / 2      # many exact ties
            valid = rng.integers(-2, width + 5, size=rows).astype(np.int32)
            fb = rng.integers(0, width + 1, size=rows).astype(np.int32)
            fe = (fb + rng.integers(0, 5, size=rows)).astype(np.int32)
            ap = rng.integers(-1, 5000, size=rows).astype(np.int32)
            use_ap = trial % 2 == 1
            got = oracle.topk16(s, valid, fb, fe, ap if use_ap else None)
            for r in range(rows):
                want = _brute(s[r], int(valid[r]), int(fb[r]), int(fe[r]),
                              int(ap[r]) if use_ap else None)
                assert got[r].tolist() == want, (width, trial, r)


@pytest.mark.parametrize("parts", [2, 3, 4, 7, 16])
def test_exact_merge_invariant(parts):
    """Per-partition top-16s merged with the same order give the global top-16."""
    ti = workloads.injected_rows(seed=parts, rows=24, width=700)
    rng = np.random.default_rng(parts)
    for r in range(ti.scores.shape[0]):
        row = ti.scores[r]
        fb, fe = int(ti.force_begin[r]), int(ti.force_end[r])
        glob = oracle.topk16(row[None], None, np.array([fb], np.int32),
                             np.array([fe], np.int32))[0]
        owner = rng.integers(0, parts, size=row.size)
        cands = []
        for p in range(parts):
            cols = np.nonzero(owner == p)[0]
            if cols.size == 0:
                continue
            sub = row[cols][None]
            forced = ((cols >= fb) & (cols < fe)).astype(np.int32)
            # Forced columns become +inf in the sub-row; lower original column keeps its
            # place because partition columns stay in ascending order.
            sub = np.where(forced[None] == 1, np.float32(np.inf), sub)
            top = oracle.topk16(sub)[0]
            cands.extend(int(cols[i]) for i in top if i >= 0)
        cands = sorted(set(cands))
        merged_row = row[cands][None]
        forced = np.array([fb <= c < fe for c in cands])
        merged_row = np.where(forced[None], np.float32(np.inf), merged_row)
        mtop = oracle.topk16(merged_row)[0]
        merged = [cands[i] if i >= 0 else -1 for i in mtop]
        assert merged == glob.tolist(), r


def test_rank_value_rules():
    assert oracle.rank_value(float("nan")) == -math.inf
    assert math.copysign(1, oracle.rank_value(-0.0)) == 1.0
    assert oracle.rank_value(-3.0, forced=True) == math.inf
    assert oracle.rank_value(float("nan"), forced=True) == math.inf
    assert oracle.rank_value(FLT_MAX) == FLT_MAX < oracle.rank_value(0.0, forced=True)
