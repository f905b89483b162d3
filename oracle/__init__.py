"""CPU oracle of the page-scoring indexer path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product library
(``page_scoring_top_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain, scalar, single-threaded C in
double precision); this module builds it with gcc and exposes numpy-level
wrappers with the same argument meaning as the product's C-ABI, on host
arrays.  Citations of the source pages are in ``oracle.c``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so.  No fast-math, no FMA contraction:
    every operation rounds as written in C."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        sig = {
            "ora_e2m1_value": (D, [ctypes.c_int]),
            "ora_e4m3_value": (D, [ctypes.c_int]),
            "ora_e4m3_rn_satfinite": (ctypes.c_int, [D]),
            "ora_page_element": (ctypes.c_int, [P, ctypes.c_int, ctypes.c_int]),
            "ora_dequant_page": (None, [P, P]),
            "ora_gather": (None, [P, I64, P, I64, P, P, I32, I32, P]),
            "ora_relu": (D, [D]),
            "ora_dot_e4m3": (D, [P, P]),
            "ora_decode_own": (ctypes.c_int, [I32, I32, ctypes.c_int]),
            "ora_decode_pages": (ctypes.c_int, [I32]),
            "ora_score_decode_column": (None, [P, I64, P, I64, P, P, P, I32, I32,
                                               ctypes.c_int, ctypes.c_int, P, P]),
            "ora_score_decode": (None, [P, I64, P, I64, P, P, P, I32, I32, I32, P, P]),
            "ora_score_prefill_one": (ctypes.c_float, [P, P, P, P, I32, I64, I64]),
            "ora_score_prefill": (None, [P, P, P, P, I32, I32, I32, P, I64]),
            "ora_score_prefill_rows": (None, [P, P, P, P, I32, I32, P, I32, P]),
            "ora_rank_value": (D, [ctypes.c_float, ctypes.c_int]),
            "ora_topk16": (None, [P, I64, I32, I32, P, P, P, P, P, I64]),
            "ora_causal_count": (I32, [I32, I32, I32, I32]),
            "ora_score_prefill_ragged": (None, [P, P, P, P, I32, I32, P, P, P, I32, P, I64, P]),
            "ora_bf16_value": (D, [ctypes.c_int]),
            "ora_mx_block_scale": (ctypes.c_int, [P]),
            "ora_mxfp8_quantize": (None, [P, I64, I32, I32, P, I64, P, I64]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
# Element level
# ---------------------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().ora_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return lib().ora_e4m3_value(int(byte))


def e4m3_rn_satfinite(x: float) -> int:
    return lib().ora_e4m3_rn_satfinite(float(x))


def relu(x: float) -> float:
    return lib().ora_relu(float(x))


def dot_e4m3(a: np.ndarray, b: np.ndarray) -> float:
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    assert a.size == 128 and b.size == 128
    return lib().ora_dot_e4m3(_p(a), _p(b))


# ---------------------------------------------------------------------------
# Pages
# ---------------------------------------------------------------------------

def dequant_page(page: np.ndarray) -> np.ndarray:
    """``[9216]`` uint8 packed page -> ``[128, 128]`` uint8 E4M3 bytes."""
    page = _c(page, np.uint8).reshape(-1)
    assert page.size == 9216
    out = np.empty((128, 128), dtype=np.uint8)
    lib().ora_dequant_page(_p(page), _p(out))
    return out


def gather(kv_cache, block_table, num_pages, page_offsets, max_num_pages, out):
    """Dequantizing gather into ``out`` ``[>= sum pages, 128, 128]`` uint8
    (modified in place, so canaries outside the written pages survive)."""
    kv = _c(kv_cache, np.uint8)
    bt = _c(block_table, np.int32)
    assert out.flags.c_contiguous and out.dtype == np.uint8
    lib().ora_gather(_p(kv), kv.shape[1] if kv.ndim == 2 else 9216, _p(bt), bt.shape[1],
                     _p(_c(num_pages, np.int32)), _p(_c(page_offsets, np.int32)),
                     bt.shape[0], int(max_num_pages), _p(out))
    return out


# ---------------------------------------------------------------------------
# Scores
# ---------------------------------------------------------------------------

def score_decode(kv_cache, block_table, seq_lens, q, q_scale, num_reqs, qlen, width,
                 scores=None, row_own=None):
    """Decode scores ``[num_reqs, 32, width]`` float32 and ``row_own``
    ``[num_reqs, 32]``.  Unstored entries keep the contents of ``scores``
    (NaN-filled when it is not given)."""
    kv = _c(kv_cache, np.uint8)
    bt = _c(block_table, np.int32)
    if scores is None:
        scores = np.full((num_reqs, 32, width), np.nan, dtype=np.float32)
    if row_own is None:
        row_own = np.full((num_reqs, 32), -7, dtype=np.int32)
    assert scores.flags.c_contiguous and scores.dtype == np.float32
    lib().ora_score_decode(_p(kv), kv.shape[1], _p(bt), bt.shape[1],
                           _p(_c(seq_lens, np.int32)), _p(_c(q, np.uint8)),
                           _p(_c(q_scale, np.float32)), int(num_reqs), int(qlen), int(width),
                           _p(scores), _p(row_own))
    return scores, row_own


def score_decode_column(kv_cache, block_table, seq_lens, q, q_scale, qlen, width, b, j):
    """One (request b, page j) column: ``(values[32], stored[32])``."""
    kv = _c(kv_cache, np.uint8)
    bt = _c(block_table, np.int32)
    col = np.empty(32, dtype=np.float32)
    st = np.empty(32, dtype=np.int32)
    lib().ora_score_decode_column(_p(kv), kv.shape[1], _p(bt), bt.shape[1],
                                  _p(_c(seq_lens, np.int32)), _p(_c(q, np.uint8)),
                                  _p(_c(q_scale, np.float32)), int(qlen), int(width),
                                  int(b), int(j), _p(col), _p(st))
    return col, st.astype(bool)


def decode_own(seq_len: int, qlen: int, slot: int) -> int:
    return lib().ora_decode_own(int(seq_len), int(qlen), int(slot))


def decode_pages(seq_len: int) -> int:
    return lib().ora_decode_pages(int(seq_len))


def score_prefill(q, q_scale, k, k_scale, scores=None, ld=None):
    q = _c(q, np.uint8)
    T, H = q.shape[0], q.shape[1]
    k = _c(k, np.uint8)
    N = k.shape[0]
    ld = N if ld is None else ld
    if scores is None:
        scores = np.full((T, ld), np.nan, dtype=np.float32)
    lib().ora_score_prefill(_p(q), _p(_c(q_scale, np.float32)), _p(k),
                            _p(_c(k_scale, np.float32)), T, H, N, _p(scores), int(ld))
    return scores


def score_prefill_rows(q, q_scale, k, k_scale, rows):
    q = _c(q, np.uint8)
    H = q.shape[1]
    k = _c(k, np.uint8)
    N = k.shape[0]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((len(rows), N), dtype=np.float32)
    lib().ora_score_prefill_rows(_p(q), _p(_c(q_scale, np.float32)), _p(k),
                                 _p(_c(k_scale, np.float32)), H, N, _p(rows), len(rows),
                                 _p(out))
    return out


def causal_count(q_len: int, k_len: int, i: int, width: int) -> int:
    return lib().ora_causal_count(int(q_len), int(k_len), int(i), int(width))


def score_prefill_ragged(q, q_scale, k, k_scale, q_start, k_start, k_len, width, scores=None,
                         ld=None):
    """Causal scores of a ragged batch: ``scores [T, ld >= width]`` float32
    (columns >= width untouched; a new array is NaN there) and ``row_len [T]``."""
    q = _c(q, np.uint8)
    T, H = q.shape[0], q.shape[1]
    k = _c(k, np.uint8)
    q_start = _c(q_start, np.int32)
    S = len(q_start) - 1
    ld = width if ld is None else ld
    if scores is None:
        scores = np.full((T, ld), np.nan, dtype=np.float32)
    row_len = np.full(T, -1, dtype=np.int32)
    lib().ora_score_prefill_ragged(_p(q), _p(_c(q_scale, np.float32)), _p(k),
                                   _p(_c(k_scale, np.float32)), H, S, _p(q_start),
                                   _p(_c(k_start, np.int32)), _p(_c(k_len, np.int32)), int(width),
                                   _p(scores), int(ld), _p(row_len))
    return scores, row_len


# ---------------------------------------------------------------------------
# Top-16
# ---------------------------------------------------------------------------

def rank_value(s: float, forced: bool = False) -> float:
    return lib().ora_rank_value(float(s), int(bool(forced)))


def topk16(scores, valid_len=None, force_begin=None, force_end=None, append_page=None):
    """Exact top-16 rows ``[rows, 16]`` int32 of ``scores [rows, width]``."""
    s = _c(scores, np.float32)
    rows, width = s.shape
    out = np.empty((rows, 16), dtype=np.int32)
    vl, fb, fe, ap = (_c(a, np.int32) for a in (valid_len, force_begin, force_end, append_page))
    lib().ora_topk16(_p(s), width, rows, width, _p(vl), _p(fb), _p(fe), _p(ap), _p(out), 16)
    return out


# ---------------------------------------------------------------------------
# MXFP8 quantization
# ---------------------------------------------------------------------------

def bf16_value(bits: int) -> float:
    return lib().ora_bf16_value(int(bits))


def mx_block_scale(block) -> int:
    """E8M0 byte of one block of 32 bf16 bit patterns."""
    b = _c(block, np.uint16).reshape(-1)
    assert b.size == 32
    return lib().ora_mx_block_scale(_p(b))


def mxfp8_quantize(x):
    """``x [rows, cols]`` bf16 bit patterns (uint16, cols a multiple of 32) ->
    (E4M3 bytes ``[rows, cols]``, E8M0 bytes ``[rows, cols / 32]``)."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    assert cols % 32 == 0
    q = np.empty((rows, cols), dtype=np.uint8)
    s = np.empty((rows, cols // 32), dtype=np.uint8)
    lib().ora_mxfp8_quantize(_p(x), cols, rows, cols, _p(q), cols, _p(s), cols // 32)
    return q, s
