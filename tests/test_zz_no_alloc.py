"""indexer_prefill_topk16_noalloc, the allocation-free variant of the fused
prefill top-16 (its workspace is a static device array inside the library),
called through the C ABI: two calls in a row, the second on a smaller batch,
must each give exactly what indexer_prefill_topk16 gives with a workspace of
its own; a batch too large for the array is refused before anything runs."""

import ctypes
import os

import numpy as np
import pytest
import torch

import workloads
from gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "page_scoring_top_amd", "libpagescore.so")
ENOSPACE = -28
SCRATCH_BYTES = 64 << 20


def _noalloc():
    lib = ctypes.CDLL(LIB)
    f = lib.indexer_prefill_topk16_noalloc
    P = ctypes.c_void_p
    f.argtypes = [P, P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int64, P]
    f.restype = ctypes.c_int
    return f


def _call(f, q, qs, k, ks, out):
    P = ctypes.c_void_p
    stream = torch.cuda.current_stream().cuda_stream
    return f(P(q.data_ptr()), P(qs.data_ptr()), P(k.data_ptr()), P(ks.data_ptr()), q.shape[0], q.shape[1],
             k.shape[0], P(out.data_ptr()), out.stride(0), P(stream))


def test_noalloc_matches_the_workspace_call_twice():
    import page_scoring_top_amd as ps
    f = _noalloc()
    # The NVFP4-sized batch first (48 MiB of records), then a smaller one
    # with other heads and keys, so the second call reads over what the
    # first one left in the shared array.
    for name, (T, H, N) in (("first", (2048, 4, 65536)), ("second, smaller", (37, 33, 3000))):
        p = workloads.prefill_inputs(f"noalloc-{T}", 70 + T, T, H, N)
        q, qs, k, ks = dev(p.q), dev(p.q_scale), dev(p.k), dev(p.k_scale)
        announce(f"noalloc prefill top-16 {name}: T={T} H={H} N={N}")
        want = torch.empty((T, 16), dtype=torch.int32, device="cuda")
        ps.indexer_prefill_topk16(q, qs, k, ks, want, ps.prefill_topk16_workspace(T, N, "cuda"))
        got = torch.full((T, 16), -7, dtype=torch.int32, device="cuda")
        assert _call(f, q, qs, k, ks, got) == 0
        assert np.array_equal(host(got), host(want)), f"{name} call differs from the workspace call"


def test_noalloc_refuses_what_the_array_cannot_hold():
    import page_scoring_top_amd as ps
    f = _noalloc()
    N = 65536                                     # 2,048 blocks of records per token (24 KiB)
    assert ps.prefill_topk16_workspace_bytes(2048, N) <= SCRATCH_BYTES
    T = 4096                                      # 96 MiB of records: refused, nothing runs
    assert ps.prefill_topk16_workspace_bytes(T, N) > SCRATCH_BYTES
    # Buffers of the full sizes, so the call would be in bounds even if it ran.
    q = torch.zeros((T, 4, 128), dtype=torch.uint8, device="cuda")
    qs = torch.zeros((T, 4), dtype=torch.float32, device="cuda")
    k = torch.zeros((N, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros(N, dtype=torch.float32, device="cuda")
    out = torch.full((T, 16), -7, dtype=torch.int32, device="cuda")
    announce("noalloc prefill top-16: a batch beyond the array is refused")
    assert _call(f, q, qs, k, ks, out) == ENOSPACE
    torch.cuda.synchronize()
    assert (host(out) == -7).all()
