"""The C ABI: libpagescore.so loads, exports every function include/pagescore.h
declares, and its host-side argument checks reject bad calls before anything
is enqueued (no GPU is touched on these paths, so they run on the CPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagescore.h")
LIB = os.path.join(ROOT, "page_scoring_top_amd", "libpagescore.so")

EINVAL = -22


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libpagescore.so is not built (python page_scoring_top_amd/build.py)")
    return ctypes.CDLL(LIB)


def test_header_declares_every_call():
    fns = declared_functions()
    for name in ("nvfp4_index_k_dequant", "indexer_score_decode", "indexer_score_prefill",
                 "indexer_score_prefill_ragged", "topk16_select", "mxfp8_e4m3_quantize",
                 "indexer_prefill_topk16", "indexer_prefill_topk16_workspace",
                 "indexer_prefill_topk16_noalloc"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    missing = [f for f in declared_functions() if not hasattr(lib, f)]
    assert not missing, missing


def test_binding_loads_the_in_tree_library():
    import page_scoring_top_amd as p
    assert os.path.samefile(p.LIB_PATH, LIB)


P = ctypes.c_void_p
FAKE = P(0x1000)          # 16-byte aligned, never dereferenced on these paths
ODD = P(0x1001)


def _dequant(lib, **kw):
    a = dict(kv=FAKE, stride=9216, nb=4, bt=FAKE, bts=8, num_pages=FAKE, offs=FAKE, R=2, maxp=8,
             out=FAKE, out_pages=16)
    a.update(kw)
    f = lib.nvfp4_index_k_dequant
    f.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, ctypes.c_int64, P, P, ctypes.c_int32,
                  ctypes.c_int32, P, ctypes.c_int64, P]
    return f(a["kv"], a["stride"], a["nb"], a["bt"], a["bts"], a["num_pages"], a["offs"], a["R"],
             a["maxp"], a["out"], a["out_pages"], None)


def test_dequant_host_checks(lib):
    assert _dequant(lib, R=0) == 0                       # nothing to do: no launch
    assert _dequant(lib, maxp=0) == 0
    assert _dequant(lib, R=-1) == EINVAL
    assert _dequant(lib, R=65536) == EINVAL              # beyond the per-call request limit
    assert _dequant(lib, kv=None) == EINVAL
    assert _dequant(lib, kv=ODD) == EINVAL               # misaligned
    assert _dequant(lib, stride=9215) == EINVAL
    assert _dequant(lib, stride=9224) == EINVAL          # not a multiple of 16
    assert _dequant(lib, nb=0) == EINVAL
    assert _dequant(lib, bts=7) == EINVAL                # narrower than max_num_pages
    assert _dequant(lib, out=None) == EINVAL
    assert _dequant(lib, out=ODD) == EINVAL
    assert _dequant(lib, out_pages=-1) == EINVAL
    assert _dequant(lib, num_pages=None) == EINVAL


def _decode(lib, **kw):
    a = dict(kv=FAKE, stride=9216, nb=4, bt=FAKE, bts=64, seq=FAKE, q=FAKE, qs=FAKE, R=1, qlen=1,
             W=64, scores=FAKE, own=None)
    a.update(kw)
    f = lib.indexer_score_decode
    f.argtypes = [P, ctypes.c_int64, ctypes.c_int64, P, ctypes.c_int64, P, P, P, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_int32, P, P, P]
    return f(a["kv"], a["stride"], a["nb"], a["bt"], a["bts"], a["seq"], a["q"], a["qs"], a["R"],
             a["qlen"], a["W"], a["scores"], a["own"], None)


def test_decode_host_checks(lib):
    assert _decode(lib, R=0) == 0
    assert _decode(lib, R=-3) == EINVAL
    assert _decode(lib, R=65536) == EINVAL               # beyond the per-call request limit
    assert _decode(lib, qlen=0) == EINVAL
    assert _decode(lib, qlen=9) == EINVAL
    assert _decode(lib, W=0) == EINVAL
    assert _decode(lib, bts=63) == EINVAL                # block table narrower than the width
    assert _decode(lib, q=ODD) == EINVAL
    assert _decode(lib, q=None) == EINVAL
    assert _decode(lib, qs=None) == EINVAL
    assert _decode(lib, scores=None) == EINVAL
    assert _decode(lib, seq=None) == EINVAL
    assert _decode(lib, kv=None) == EINVAL


def _prefill(lib, **kw):
    a = dict(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, T=4, H=2, N=8, scores=FAKE, ld=8)
    a.update(kw)
    f = lib.indexer_score_prefill
    f.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int64, P]
    return f(a["q"], a["qs"], a["k"], a["ks"], a["T"], a["H"], a["N"], a["scores"], a["ld"], None)


def test_prefill_host_checks(lib):
    assert _prefill(lib, T=0) == 0
    assert _prefill(lib, N=0) == 0
    assert _prefill(lib, H=0) == EINVAL
    assert _prefill(lib, H=225) == EINVAL               # beyond the LDS-resident head limit
    assert _prefill(lib, T=-1) == EINVAL
    assert _prefill(lib, ld=7) == EINVAL
    assert _prefill(lib, q=ODD) == EINVAL
    assert _prefill(lib, k=ODD) == EINVAL
    assert _prefill(lib, ks=None) == EINVAL


def _workspace(lib, T, N):
    f = lib.indexer_prefill_topk16_workspace
    f.argtypes = [ctypes.c_int32, ctypes.c_int32]
    f.restype = ctypes.c_int64
    return f(T, N)


def test_prefill_topk16_workspace_size(lib):
    # Block records: three planes [T, 32 ceil(N / 1024)] of 4 bytes each.
    assert _workspace(lib, 2048, 65536) == 2048 * 3 * 2048 * 4
    assert _workspace(lib, 5, 1) == 5 * 3 * 32 * 4
    assert _workspace(lib, 3, 1025) == 3 * 3 * 64 * 4
    assert _workspace(lib, 0, 7) == 0
    assert _workspace(lib, -1, 7) < 0
    assert _workspace(lib, 4, 0) < 0


WS = P(0x10000)           # 256-byte aligned, never dereferenced on these paths


def _prefill_topk(lib, **kw):
    a = dict(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, T=4, H=4, N=100, out=FAKE, os=16, ws=WS,
             wsb=1 << 20)
    a.update(kw)
    f = lib.indexer_prefill_topk16
    f.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int64, P,
                  ctypes.c_int64, P]
    return f(a["q"], a["qs"], a["k"], a["ks"], a["T"], a["H"], a["N"], a["out"], a["os"], a["ws"],
             a["wsb"], None)


def test_prefill_topk16_host_checks(lib):
    # Every call below fails one check (or has T == 0), so nothing is enqueued.
    assert _prefill_topk(lib, T=0) == 0
    assert _prefill_topk(lib, T=-1) == EINVAL
    assert _prefill_topk(lib, N=0) == EINVAL
    assert _prefill_topk(lib, H=0) == EINVAL
    assert _prefill_topk(lib, H=65) == EINVAL
    assert _prefill_topk(lib, os=15) == EINVAL
    assert _prefill_topk(lib, q=ODD) == EINVAL
    assert _prefill_topk(lib, k=ODD) == EINVAL
    assert _prefill_topk(lib, qs=None) == EINVAL
    assert _prefill_topk(lib, out=None) == EINVAL
    assert _prefill_topk(lib, ws=None) == EINVAL
    assert _prefill_topk(lib, ws=P(0x10010)) == EINVAL          # 16- but not 256-byte aligned
    assert _prefill_topk(lib, wsb=_workspace(lib, 4, 100) - 1) == EINVAL


def test_prefill_topk16_noalloc_host_checks(lib):
    # Refusals only: nothing here reaches the device.
    f = lib.indexer_prefill_topk16_noalloc
    f.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int64, P]
    f.restype = ctypes.c_int

    def call(T=4, H=4, N=100, q=FAKE, os=16):
        return f(q, FAKE, FAKE, FAKE, T, H, N, FAKE, os, None)
    assert call(T=0) == 0
    assert call(H=0) == EINVAL
    assert call(N=0) == EINVAL
    assert call(q=ODD) == EINVAL
    assert call(os=15) == EINVAL
    # 4,096 tokens x 2,048 blocks x 12 bytes = 96 MiB > the 64 MiB array.
    assert call(T=4096, N=65536) == -28


def _topk(lib, **kw):
    a = dict(s=FAKE, rs=100, rows=3, W=100, valid=None, fb=None, fe=None, ap=None, out=FAKE, os=16)
    a.update(kw)
    f = lib.topk16_select
    f.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, ctypes.c_int64, P]
    return f(a["s"], a["rs"], a["rows"], a["W"], a["valid"], a["fb"], a["fe"], a["ap"], a["out"],
             a["os"], None)


def test_topk_host_checks(lib):
    assert _topk(lib, rows=0) == 0
    assert _topk(lib, rows=-1) == EINVAL
    assert _topk(lib, W=0) == EINVAL
    assert _topk(lib, W=(1 << 28) + 1, rs=(1 << 28) + 1) == EINVAL   # width past the limit
    assert _topk(lib, rs=99) == EINVAL
    assert _topk(lib, os=15) == EINVAL
    assert _topk(lib, fb=FAKE) == EINVAL                 # begin without end
    assert _topk(lib, out=None) == EINVAL
    assert _topk(lib, s=None) == EINVAL


def _ragged(lib, **kw):
    a = dict(q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, T=8, H=4, N=100, S=2, q_start=FAKE, k_start=FAKE,
             k_len=FAKE, max_q=8, W=100, s=FAKE, ld=100, row_len=None)
    a.update(kw)
    f = lib.indexer_score_prefill_ragged
    I32 = ctypes.c_int32
    f.argtypes = [P, P, P, P, I32, I32, I32, I32, P, P, P, I32, I32, P, ctypes.c_int64, P, P]
    return f(a["q"], a["qs"], a["k"], a["ks"], a["T"], a["H"], a["N"], a["S"], a["q_start"],
             a["k_start"], a["k_len"], a["max_q"], a["W"], a["s"], a["ld"], a["row_len"], None)


def test_ragged_prefill_host_checks(lib):
    assert _ragged(lib, T=0) == 0
    assert _ragged(lib, S=0) == 0
    assert _ragged(lib, max_q=0) == 0
    assert _ragged(lib, H=65) == EINVAL                 # beyond the small-head kernel
    assert _ragged(lib, H=0) == EINVAL
    assert _ragged(lib, S=65536) == EINVAL
    assert _ragged(lib, W=0) == EINVAL
    assert _ragged(lib, ld=99) == EINVAL
    assert _ragged(lib, q=ODD) == EINVAL
    assert _ragged(lib, k_len=None) == EINVAL
    assert _ragged(lib, q_start=None) == EINVAL


def _mx(lib, **kw):
    a = dict(x=FAKE, xs=64, rows=4, cols=64, q=FAKE, qs=64, s=FAKE, ss=2)
    a.update(kw)
    f = lib.mxfp8_e4m3_quantize
    f.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int64, P,
                  ctypes.c_int64, P]
    return f(a["x"], a["xs"], a["rows"], a["cols"], a["q"], a["qs"], a["s"], a["ss"], None)


def test_mxfp8_host_checks(lib):
    assert _mx(lib, rows=0) == 0
    assert _mx(lib, cols=0) == 0
    assert _mx(lib, rows=-1) == EINVAL
    assert _mx(lib, cols=48) == EINVAL                   # not whole 32-element blocks
    assert _mx(lib, x=ODD) == EINVAL
    assert _mx(lib, xs=60) == EINVAL                     # stride below cols
    assert _mx(lib, xs=68) == EINVAL                     # rows not 16-byte aligned
    assert _mx(lib, q=ODD) == EINVAL
    assert _mx(lib, qs=72) == EINVAL                     # q rows not 16-byte aligned
    assert _mx(lib, ss=1) == EINVAL
    assert _mx(lib, s=None) == EINVAL


def test_strerror(lib):
    lib.pagescore_strerror.restype = ctypes.c_char_p
    assert lib.pagescore_strerror(0) == b"ok"
    assert b"invalid" in lib.pagescore_strerror(EINVAL)
