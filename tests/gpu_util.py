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


def prefill_term_magnitude(q, q_scale, k, k_scale) -> np.ndarray:
    """k_scale[n] * sum_h |q_scale[t,h]| * sum_d |q[t,h,d] k[n,d]| in float64:
    the size of the terms a prefill score is summed from.  An f32 sum of
    them carries an error of a few units in the last place of this size, not
    of the result, so a score whose dot products cancel is compared against
    it.  (E4M3 bytes are read through torch's float8_e4m3fn, exactly.)"""
    def val(b):
        return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).double().abs()
    qa = val(q)                                   # [T, H, 128]
    ka = val(k)                                   # [N, 128]
    qs = torch.from_numpy(np.asarray(q_scale, dtype=np.float64)).abs()
    ks = torch.from_numpy(np.asarray(k_scale, dtype=np.float64)).abs()
    dots = torch.matmul(qa, ka.T.contiguous())    # [T, H, N]
    return ((dots * qs[:, :, None]).sum(dim=1) * ks[None, :]).numpy()


def assert_scores_close(got: np.ndarray, want: np.ndarray, what: str = "",
                        magnitude: np.ndarray | None = None) -> None:
    """|got - want| <= ATOL + RTOL * |want|; with ``magnitude`` (the size of
    the summed terms, for sums that cancel) RTOL scales max(|want|, magnitude)."""
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, (got.shape, want.shape)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ ({np.argwhere(gn != wn)[:5]})"
    gi, wi = np.isinf(got), np.isinf(want)
    assert np.array_equal(gi, wi) and np.array_equal(got[gi], want[wi]), f"{what}: inf differ"
    fin = ~(wn | wi)
    err = np.abs(got[fin].astype(np.float64) - want[fin].astype(np.float64))
    scale = np.abs(want[fin].astype(np.float64))
    if magnitude is not None:
        scale = np.maximum(scale, np.asarray(magnitude, dtype=np.float64)[fin])
    lim = ATOL + RTOL * scale
    bad = err > lim
    if bad.any():
        idx = np.argwhere(fin)[np.argmax(err / lim)]
        raise AssertionError(f"{what}: {bad.sum()} of {fin.sum()} scores out of tolerance; worst at "
                             f"{tuple(idx)}: gpu {got[tuple(idx)]!r} oracle {want[tuple(idx)]!r}")


CANARY_F32 = np.float32(-7.25e31)
CANARY_I32 = np.int32(-123456789)
