"""The oracle over a whole workload, spread over host threads.

The oracle is single-threaded C; each call below scores an independent
piece (one decode column, a few prefill rows, a few top-16 rows) and the
pieces run on a thread pool.  ctypes releases the interpreter lock for the
duration of a foreign call, so the pieces run in parallel inside this one
process: nothing is forked or exec'ed, which matters because the GPU tests
call this after the process has initialised the GPU.  The oracle itself is
unchanged; only the order in which its pieces are computed differs, and
each piece is a deterministic function of its inputs.
"""

from __future__ import annotations

import concurrent.futures
import os
import sys
import time

import numpy as np

import oracle


def threads() -> int:
    """Host threads for the oracle: the process's CPU share, at most 16."""
    n = 0
    try:
        n = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        n = 0
    if n <= 0:
        n = len(os.sched_getaffinity(0))
    return max(1, min(16, n))


def map_pieces(fn, items, what: str = "oracle"):
    """fn over items on the pool, results in order; a progress line on
    stderr about every 20 s, so a long run is visibly alive."""
    items = list(items)
    out = [None] * len(items)
    t0 = last = time.monotonic()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads()) as ex:
        futs = {ex.submit(fn, it): i for i, it in enumerate(items)}
        for done, f in enumerate(concurrent.futures.as_completed(futs), 1):
            out[futs[f]] = f.result()
            now = time.monotonic()
            if now - last > 20.0:
                last = now
                print(f"[oracle-pool] {what}: {done}/{len(items)} pieces, {now - t0:.0f} s",
                      file=sys.stderr, flush=True)
    return out


def score_decode(d, base=None):
    """Every decode score of ``d`` (a workloads.DecodeInputs): returns
    ``(scores [R_total, 32, width], stored [R_total, 32, width] bool)``.
    Entries that are not stored keep ``base`` (NaN when it is None)."""
    Rt = d.q.shape[0]
    scores = np.full((Rt, 32, d.width), np.nan, np.float32) if base is None else base.copy()
    stored = np.zeros((Rt, 32, d.width), bool)
    kv = np.ascontiguousarray(d.kv_cache)
    cols = []
    for b in range(d.num_reqs):
        npg = min(oracle.decode_pages(int(d.seq_lens[b])), d.width)
        cols += [(b, j) for j in range(npg)]

    def one(bj):
        b, j = bj
        return oracle.score_decode_column(kv, d.block_table, d.seq_lens, d.q, d.q_scale, d.qlen,
                                          d.width, b, j)

    for (b, j), (col, st) in zip(cols, map_pieces(one, cols, "decode columns")):
        scores[b, st, j] = col[st]
        stored[b, :, j] = st
    return scores, stored


def score_prefill_rows(q, q_scale, k, k_scale, rows, rows_per_task: int = 2):
    """Full oracle rows ``[len(rows), N]`` of the prefill score."""
    rows = [int(r) for r in rows]
    chunks = [rows[i:i + rows_per_task] for i in range(0, len(rows), rows_per_task)]
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    parts = map_pieces(lambda c: oracle.score_prefill_rows(q, q_scale, k, k_scale, c), chunks,
                 "prefill rows")
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, k.shape[0]), np.float32)


def topk16(scores, valid_len=None, force_begin=None, force_end=None, append_page=None,
           rows_per_task: int = 16):
    """The oracle's top-16 of every row of ``scores [rows, width]``."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    n = scores.shape[0]
    starts = list(range(0, n, rows_per_task))

    def cut(a, s):
        return None if a is None else np.asarray(a)[s:s + rows_per_task]

    parts = map_pieces(lambda s: oracle.topk16(scores[s:s + rows_per_task], cut(valid_len, s),
                                         cut(force_begin, s), cut(force_end, s),
                                         cut(append_page, s)), starts, "top-16 rows")
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, 16), np.int32)
