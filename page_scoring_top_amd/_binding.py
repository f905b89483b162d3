"""ctypes binding of libpagescore.so (C ABI: include/pagescore.h).

Argument marshalling only: each function checks the tensors' dtype, device and
layout, turns them into raw device pointers and strides, passes torch's
current HIP stream, and raises on a non-zero status.  Every step of the path
runs in the library's kernels.  If the library has not been built the import
fails loudly; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagescore.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build it with `python page_scoring_top_amd/build.py` "
        "(or __graft_entry__.build()); the indexer path has no CPU fallback")

_lib = ctypes.CDLL(_LIB_PATH)

_P, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
_lib.nvfp4_index_k_dequant.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P, _I32, _I32, _P, _I64, _P]
_lib.indexer_score_decode.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P, _P, _I32, _I32, _I32,
                                      _P, _P, _P]
_lib.indexer_score_prefill.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _P, _I64, _P]
_lib.topk16_select.argtypes = [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _I64, _P]
_lib.mxfp8_e4m3_quantize.argtypes = [_P, _I64, _I32, _I32, _P, _I64, _P, _I64, _P]
_lib.indexer_score_prefill_ragged.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P,
                                              _I32, _I32, _P, _I64, _P, _P]
_lib.indexer_prefill_topk16.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _P, _I64, _P, _I64, _P]
_lib.indexer_prefill_topk16_workspace.argtypes = [_I32, _I32]
_lib.indexer_prefill_topk16_workspace.restype = ctypes.c_int64
for _f in (_lib.nvfp4_index_k_dequant, _lib.indexer_score_decode, _lib.indexer_score_prefill,
           _lib.topk16_select, _lib.mxfp8_e4m3_quantize, _lib.indexer_score_prefill_ragged,
           _lib.indexer_prefill_topk16):
    _f.restype = ctypes.c_int
_lib.pagescore_strerror.argtypes = [ctypes.c_int]
_lib.pagescore_strerror.restype = ctypes.c_char_p
_lib.pagescore_last_hip_error.argtypes = []
_lib.pagescore_last_hip_error.restype = ctypes.c_int

PAGE_BYTES = 9216
LIB_PATH = _LIB_PATH


class PageScoreError(RuntimeError):
    def __init__(self, fn: str, code: int):
        msg = _lib.pagescore_strerror(code).decode()
        if code == -5:
            msg += f" (hip error {_lib.pagescore_last_hip_error()})"
        super().__init__(f"{fn}: status {code}: {msg}")
        self.code = code


def _check(fn, code):
    if code != 0:
        raise PageScoreError(fn, code)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtypes, cuda=True):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if cuda and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


_U8 = (torch.uint8, torch.float8_e4m3fn)
_I32T = (torch.int32,)
_F32 = (torch.float32,)


def _page_stride(kv_cache: torch.Tensor) -> int:
    # A page is 9,216 bytes: [num_blocks, 9216] or [num_blocks, 128, 72], each page contiguous.
    if kv_cache.dim() == 3:
        if tuple(kv_cache.shape[1:]) != (128, 72) or kv_cache.stride(2) != 1 or kv_cache.stride(1) != 72:
            raise ValueError("kv_cache [num_blocks, 128, 72] must have contiguous pages")
    elif kv_cache.dim() == 2:
        if kv_cache.shape[1] != PAGE_BYTES or kv_cache.stride(1) != 1:
            raise ValueError("kv_cache [num_blocks, 9216] must have contiguous pages")
    else:
        raise ValueError("kv_cache must be [num_blocks, 9216] or [num_blocks, 128, 72]")
    return kv_cache.stride(0)


def nvfp4_index_k_dequant(kv_cache, block_table, num_pages, page_offsets, max_num_pages: int, out):
    """Dequantizing gather of NVFP4 index-K pages into ``out [>=pages, 128, 128]``."""
    _need(kv_cache, "kv_cache", _U8)
    _need(block_table, "block_table", _I32T)
    _need(num_pages, "num_pages", _I32T)
    _need(page_offsets, "page_offsets", _I32T)
    _need(out, "out", _U8)
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [num_reqs, max_blocks] with unit column stride")
    if block_table.shape[1] < max_num_pages:
        raise ValueError("block_table has fewer columns than max_num_pages")
    R = block_table.shape[0]
    if num_pages.numel() < R or page_offsets.numel() < R:
        raise ValueError("num_pages and page_offsets need one entry per block-table row")
    if not out.is_contiguous() or out.numel() % (128 * 128) != 0:
        raise ValueError("out must be contiguous [pages, 128, 128]")
    _check("nvfp4_index_k_dequant", _lib.nvfp4_index_k_dequant(
        _ptr(kv_cache), _page_stride(kv_cache), kv_cache.shape[0], _ptr(block_table),
        block_table.stride(0), _ptr(num_pages), _ptr(page_offsets), R,
        int(max_num_pages), _ptr(out), out.numel() // (128 * 128), _stream(kv_cache)))
    return out


def indexer_score_decode(kv_cache, block_table, seq_lens, q, q_scale, qlen: int, width: int,
                         scores, row_own=None, num_reqs: int | None = None):
    """Fused NVFP4 dequant + decode page scores into ``scores [R, 32, width]``."""
    _need(kv_cache, "kv_cache", _U8)
    _need(block_table, "block_table", _I32T)
    _need(seq_lens, "seq_lens", _I32T)
    _need(q, "q", _U8)
    _need(q_scale, "q_scale", _F32)
    _need(scores, "scores", _F32)
    _need(row_own, "row_own", _I32T)
    if num_reqs is None:
        num_reqs = seq_lens.shape[0]
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be [num_reqs, max_blocks] with unit column stride")
    if block_table.shape[1] < width:
        raise ValueError("block_table needs at least `width` columns")
    if not (q.is_contiguous() and q_scale.is_contiguous() and scores.is_contiguous()):
        raise ValueError("q, q_scale and scores must be contiguous")
    if q.numel() < num_reqs * 4096 or q_scale.numel() < num_reqs * 32 or \
            scores.numel() < num_reqs * 32 * width or block_table.shape[0] < num_reqs or \
            seq_lens.shape[0] < num_reqs or (row_own is not None and row_own.numel() < num_reqs * 32):
        raise ValueError("a buffer is smaller than num_reqs requires")
    _check("indexer_score_decode", _lib.indexer_score_decode(
        _ptr(kv_cache), _page_stride(kv_cache), kv_cache.shape[0], _ptr(block_table),
        block_table.stride(0), _ptr(seq_lens), _ptr(q), _ptr(q_scale), int(num_reqs), int(qlen),
        int(width), _ptr(scores), _ptr(row_own), _stream(kv_cache)))
    return scores


def indexer_score_prefill(q, q_scale, k, k_scale, scores):
    """Lightning-indexer scores ``scores [T, ld>=N]`` of ``q [T,H,128]`` vs ``k [N,128]``."""
    _need(q, "q", _U8)
    _need(q_scale, "q_scale", _F32)
    _need(k, "k", _U8)
    _need(k_scale, "k_scale", _F32)
    _need(scores, "scores", _F32)
    T, H = q.shape[0], q.shape[1]
    N = k.shape[0]
    if not (q.is_contiguous() and q_scale.is_contiguous() and k.is_contiguous() and k_scale.is_contiguous()):
        raise ValueError("q, q_scale, k and k_scale must be contiguous")
    if scores.dim() != 2 or scores.stride(1) != 1 or scores.shape[0] < T or scores.shape[1] < N:
        raise ValueError("scores must be [T, >=N] with unit column stride")
    if q.dim() != 3 or q.shape[2] != 128 or k.dim() != 2 or k.shape[1] != 128 or \
            q_scale.numel() < T * H or k_scale.numel() < N:
        raise ValueError("q [T,H,128], q_scale [T,H], k [N,128], k_scale [N] expected")
    _check("indexer_score_prefill", _lib.indexer_score_prefill(
        _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), T, H, N, _ptr(scores), scores.stride(0),
        _stream(q)))
    return scores


def indexer_score_prefill_ragged(q, q_scale, k, k_scale, q_start, k_start, k_len, max_q: int,
                                 width: int, scores, row_len=None):
    """Causal lightning-indexer scores of a ragged batch into ``scores [T, >=width]``
    (columns relative to each sequence's first key, -inf past a row's visible
    keys) and the visible counts into ``row_len [T]``."""
    _need(q, "q", _U8)
    _need(q_scale, "q_scale", _F32)
    _need(k, "k", _U8)
    _need(k_scale, "k_scale", _F32)
    for name, t in (("q_start", q_start), ("k_start", k_start), ("k_len", k_len),
                    ("row_len", row_len)):
        _need(t, name, _I32T)
    _need(scores, "scores", _F32)
    T, H = q.shape[0], q.shape[1]
    N = k.shape[0]
    S = q_start.numel() - 1
    if not all(t.is_contiguous() for t in (q, q_scale, k, k_scale, q_start, k_start, k_len)):
        raise ValueError("inputs must be contiguous")
    if scores.dim() != 2 or scores.stride(1) != 1 or scores.shape[0] < T or scores.shape[1] < width:
        raise ValueError("scores must be [T, >=width] with unit column stride")
    if S < 0 or k_start.numel() < S or k_len.numel() < S or (row_len is not None and
                                                             row_len.numel() < T):
        raise ValueError("q_start [S+1], k_start [S], k_len [S], row_len [T] expected")
    _check("indexer_score_prefill_ragged", _lib.indexer_score_prefill_ragged(
        _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), T, H, N, S, _ptr(q_start), _ptr(k_start),
        _ptr(k_len), int(max_q), int(width), _ptr(scores), scores.stride(0), _ptr(row_len),
        _stream(q)))
    return scores


def topk16_select(scores, width: int, out, valid_len=None, force_begin=None, force_end=None,
                  append_page=None, num_rows: int | None = None):
    """Exact top-16 column ids of each row of ``scores [rows, >=width]`` into ``out [rows, >=16]``."""
    _need(scores, "scores", _F32)
    _need(out, "out", _I32T)
    for name, t in (("valid_len", valid_len), ("force_begin", force_begin),
                    ("force_end", force_end), ("append_page", append_page)):
        _need(t, name, _I32T)
    if scores.dim() != 2 or scores.stride(1) != 1 or out.dim() != 2 or out.stride(1) != 1:
        raise ValueError("scores and out must be 2-D with unit column stride")
    if num_rows is None:
        num_rows = scores.shape[0]
    if out.shape[0] < num_rows or out.shape[1] < 16 or scores.shape[0] < num_rows or \
            scores.shape[1] < width:
        raise ValueError("buffers smaller than num_rows x width requires")
    for name, t in (("valid_len", valid_len), ("force_begin", force_begin),
                    ("force_end", force_end), ("append_page", append_page)):
        if t is not None and t.numel() < num_rows:
            raise ValueError(f"{name} needs one entry per row")
    _check("topk16_select", _lib.topk16_select(
        _ptr(scores), scores.stride(0), int(num_rows), int(width), _ptr(valid_len),
        _ptr(force_begin), _ptr(force_end), _ptr(append_page), _ptr(out), out.stride(0),
        _stream(scores)))
    return out


def prefill_topk16_workspace_bytes(T: int, N: int) -> int:
    """Bytes of workspace indexer_prefill_topk16 needs for T query rows and N keys."""
    n = int(_lib.indexer_prefill_topk16_workspace(int(T), int(N)))
    if n < 0:
        raise ValueError("T >= 0 and N >= 1 expected")
    return n


def prefill_topk16_workspace(T: int, N: int, device):
    """A uint8 device tensor big enough to serve as that workspace."""
    return torch.empty(prefill_topk16_workspace_bytes(T, N), dtype=torch.uint8, device=device)


def indexer_prefill_topk16(q, q_scale, k, k_scale, out, workspace):
    """Top-16 key ids of every row of the lightning-indexer scores of ``q [T,H,128]``
    against ``k [N,128]`` into ``out [T, >=16]``, without the score matrix
    (``workspace``: a uint8 device tensor from ``prefill_topk16_workspace``)."""
    _need(q, "q", _U8)
    _need(q_scale, "q_scale", _F32)
    _need(k, "k", _U8)
    _need(k_scale, "k_scale", _F32)
    _need(out, "out", _I32T)
    _need(workspace, "workspace", (torch.uint8,))
    T, H = q.shape[0], q.shape[1]
    N = k.shape[0]
    if not all(t.is_contiguous() for t in (q, q_scale, k, k_scale, workspace)):
        raise ValueError("q, q_scale, k, k_scale and workspace must be contiguous")
    if q.dim() != 3 or q.shape[2] != 128 or k.dim() != 2 or k.shape[1] != 128 or \
            q_scale.numel() < T * H or k_scale.numel() < N:
        raise ValueError("q [T,H,128], q_scale [T,H], k [N,128], k_scale [N] expected")
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] < T or out.shape[1] < 16:
        raise ValueError("out must be [T, >=16] with unit column stride")
    _check("indexer_prefill_topk16", _lib.indexer_prefill_topk16(
        _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), T, H, N, _ptr(out), out.stride(0),
        _ptr(workspace), workspace.numel(), _stream(q)))
    return out


def mxfp8_e4m3_quantize(x, q, scales):
    """MXFP8 quantization of ``x [rows, cols]`` bf16 into ``q [rows, >=cols]``
    E4M3 bytes and ``scales [rows, >=cols/32]`` E8M0 bytes."""
    _need(x, "x", (torch.bfloat16, torch.int16, torch.uint16))
    _need(q, "q", _U8)
    _need(scales, "scales", (torch.uint8,))
    for name, t in (("x", x), ("q", q), ("scales", scales)):
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be 2-D with unit column stride")
    rows, cols = x.shape
    if q.shape[0] < rows or q.shape[1] < cols or scales.shape[0] < rows or \
            scales.shape[1] < cols // 32:
        raise ValueError("q [rows, >=cols] and scales [rows, >=cols/32] expected")
    _check("mxfp8_e4m3_quantize", _lib.mxfp8_e4m3_quantize(
        _ptr(x), x.stride(0), int(rows), int(cols), _ptr(q), q.stride(0), _ptr(scales),
        scales.stride(0), _stream(x)))
    return q, scales


def raw_library():
    """The loaded ctypes library (for tests of the C ABI itself)."""
    return _lib


class PreparedCall:
    """A C-ABI call whose arguments were checked and marshalled once.

    Calling it re-issues the same launch on the same stream with no Python-side
    work beyond the ctypes call; the tensors it was prepared with are kept
    alive and must not be reallocated.  Useful in serving or timing loops."""

    def __init__(self, name, fn, args, keep):
        self._name, self._fn, self._args, self._keep = name, fn, tuple(args), keep

    def __call__(self):
        code = self._fn(*self._args)
        if code != 0:
            raise PageScoreError(self._name, code)

    def again(self) -> "PreparedCall":
        """The same call prepared afresh on the stream that is current now
        (to capture it into a graph on another stream)."""
        args, kwargs = self._keep
        return prepare(globals()[self._name], *args, **kwargs)


def _capture_args(fn, *a, **kw):
    """Run `fn` with the C function swapped for a recorder, returning its argument list."""
    rec = {}

    class _Rec:
        def __init__(self, real):
            self.real = real

        def __call__(self, *args):
            rec["args"] = args
            return 0

    name = fn.__name__
    real = getattr(_lib, name)
    setattr(_lib, name, _Rec(real))
    try:
        fn(*a, **kw)
    finally:
        setattr(_lib, name, real)
    return name, real, rec["args"]


def prepare(fn, *args, **kwargs) -> PreparedCall:
    """Validate and marshal a call of one of the four entry points once.

    ``prepare(indexer_score_decode, kv, bt, ...)`` returns a PreparedCall that
    launches exactly what ``indexer_score_decode(kv, bt, ...)`` would."""
    name, real, cargs = _capture_args(fn, *args, **kwargs)
    return PreparedCall(name, real, cargs, (args, kwargs))
