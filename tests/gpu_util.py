"""Helpers shared by the GPU parity tests."""

import sys

import numpy as np
import torch

# Scores: |gpu - oracle| <= ATOL + RTOL * |oracle|; NaN must meet NaN and +-inf must match.
RTOL = 1e-5
ATOL = 1e-6


def announce(msg: str) -> None:
    """Name the case before a GPU step, so a crash still tells which one ran."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_scores_close(got: np.ndarray, want: np.ndarray, what: str = "") -> None:
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, (got.shape, want.shape)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ ({np.argwhere(gn != wn)[:5]})"
    gi, wi = np.isinf(got), np.isinf(want)
    assert np.array_equal(gi, wi) and np.array_equal(got[gi], want[wi]), f"{what}: inf differ"
    fin = ~(wn | wi)
    err = np.abs(got[fin].astype(np.float64) - want[fin].astype(np.float64))
    lim = ATOL + RTOL * np.abs(want[fin].astype(np.float64))
    bad = err > lim
    if bad.any():
        idx = np.argwhere(fin)[np.argmax(err / lim)]
        raise AssertionError(f"{what}: {bad.sum()} of {fin.sum()} scores out of tolerance; worst at "
                             f"{tuple(idx)}: gpu {got[tuple(idx)]!r} oracle {want[tuple(idx)]!r}")


CANARY_F32 = np.float32(-7.25e31)
CANARY_I32 = np.int32(-123456789)
