"""Shared by the matrix-instruction accuracy test (GPU) and the check of its
committed record (CPU): the exact dot products of the probe's tiles and the
error figures of a method's outputs against them.

The probe (tests/probe/mfma_accuracy.hip) computes a[t, i] . b[t, j] for 16 x
16 pairs of depth-128 E4M3 vectors per tile with three gfx950 instructions.
E4M3 values are integers in units of 2^-9 below 2^18 (read through torch's
float8_e4m3fn, exactly), so the exact dot product is an integer in units of
2^-18 and int64 holds it."""

import numpy as np
import torch

METHODS = ("f16 MFMA 16x16x32 (x4)", "fp8 MFMA 16x16x32 (x4)", "f8f6f4 MFMA 16x16x128 (unit scales)")


def units(e4m3_bytes) -> np.ndarray:
    v = torch.from_numpy(np.ascontiguousarray(e4m3_bytes)).view(torch.float8_e4m3fn).double()
    return (v * 512).round().to(torch.int64).numpy()


def exact(a, b):
    """(dots, max |product|) per tile, [tiles, 16, 16], in units of 2^-18."""
    ia, ib = units(a), units(b)
    dots = np.einsum("tik,tjk->tij", ia, ib)
    maxp = np.abs(ia[:, :, None, :] * ib[:, None, :, :]).max(axis=3)
    return dots, maxp


def worst_log2(got, dots, maxp) -> float:
    """max over outputs of log2(|got - exact| / max |product|), or -inf."""
    err = np.abs(np.asarray(got, np.float64) * 2.0 ** 18 - dots.astype(np.float64))
    rel = err / np.maximum(maxp.astype(np.float64), 1.0)
    m = rel.max()
    return float(np.log2(m)) if m > 0 else float("-inf")


def worst_rel_to_result(got, dots) -> float:
    """max over outputs with a nonzero exact dot of |got - exact| / |exact|."""
    d = dots.astype(np.float64)
    nz = d != 0
    return float((np.abs(np.asarray(got, np.float64) * 2.0 ** 18 - d)[nz] / np.abs(d[nz])).max())
