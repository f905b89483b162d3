"""GPU parity of nvfp4_index_k_dequant: bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu


def _gather(kv, bt, num_pages, offs, max_pages, out_pages):
    import page_scoring_top_amd as ps
    out = torch.full((out_pages, 128, 128), 0xA5, dtype=torch.uint8, device="cuda")
    ps.nvfp4_index_k_dequant(dev(kv), dev(bt), dev(num_pages), dev(offs), max_pages, out)
    return host(out)


def test_every_code_scale_pair():
    """One page in which every (code, scale byte) pair occurs: each group of 16
    holds codes 0..15 and the 1,024 groups cycle through all 256 scale bytes."""
    rng = np.random.default_rng(0)
    page = np.zeros(9216, dtype=np.uint8)
    codes = np.tile(np.arange(16), 8)                   # one token: 8 groups of codes 0..15
    for t in range(128):
        c = np.roll(codes, t)                           # shift so nibble order matters
        page[t * 64:(t + 1) * 64] = c[0::2] | (c[1::2] << 4)
    page[8192:] = rng.permutation(np.tile(np.arange(256), 4)).astype(np.uint8)
    kv = page.reshape(1, 9216)
    announce("dequant every code x scale pair")
    got = _gather(kv, np.zeros((1, 1), np.int32), np.array([1], np.int32),
                  np.array([0], np.int32), 1, 1)
    assert np.array_equal(got[0], oracle.dequant_page(page))


def test_gather_ragged_with_skips_and_canaries():
    rng = np.random.default_rng(1)
    nb = 37
    kv = workloads.random_pages(rng, rng, nb, scale_low=0, scale_high=255)
    R, C = 6, 9
    bt = rng.integers(0, nb, size=(R, C)).astype(np.int32)
    bt[2, 1] = -1                                       # out-of-range ids are skipped
    bt[4, 0] = nb
    num_pages = np.array([3, 0, 9, 12, 2, 5], np.int32)  # 12 > max: cut to the host bound
    max_pages = 9
    offs = np.array([0, 3, 3, 12, 21, 40], np.int32)     # request 5 lands past out_pages: skipped
    out_pages = 24
    announce("dequant ragged gather")
    got = _gather(kv, bt, num_pages, offs, max_pages, out_pages)
    want = np.full((out_pages, 128, 128), 0xA5, np.uint8)
    for r in range(R):
        for j in range(min(num_pages[r], max_pages)):
            o = offs[r] + j
            if 0 <= bt[r, j] < nb and 0 <= o < out_pages:
                want[o] = oracle.dequant_page(kv[bt[r, j]])
    assert np.array_equal(got, want)


def test_gather_mtp_config_every_page():
    """The 16-request, 30,000-token cache: every logical page of every request."""
    d = workloads.mtp_decode()
    R = d.num_reqs
    n = np.full(R, 235, np.int32)
    offs = (np.arange(R) * 235).astype(np.int32)
    announce("dequant mtp config, 3,760 pages")
    got = _gather(d.kv_cache, d.block_table, n, offs, 235, R * 235)
    want = np.empty((R * 235, 128, 128), np.uint8)
    oracle.gather(d.kv_cache, d.block_table, n, offs, 235, want)
    assert np.array_equal(got, want)


def test_gather_long_config_every_page():
    """The 500K-token batch in the benchmark's launch configuration: every
    scored page of the 4 requests (15,624 pages, 256 MB of E4M3 out) against
    the oracle's gather."""
    d = workloads.long_decode()
    R, W = d.num_reqs, d.width
    npages = np.array([min(max((int(s) - 1) // 128, 0), W) for s in d.seq_lens[:R]], np.int32)
    offs = np.concatenate([[0], np.cumsum(npages)[:-1]]).astype(np.int32)
    total = int(npages.sum())
    announce("dequant long config, 15,624 pages")
    got = _gather(d.kv_cache, d.block_table[:R], npages, offs, W, total)
    want = np.empty((total, 128, 128), np.uint8)
    oracle.gather(d.kv_cache, d.block_table[:R], npages, offs, W, want)
    assert np.array_equal(got, want)


def test_nothing_to_do_is_a_no_op():
    import page_scoring_top_amd as ps
    kv = dev(np.zeros((1, 9216), np.uint8))
    out = torch.full((1, 128, 128), 7, dtype=torch.uint8, device="cuda")
    announce("dequant no-op")
    ps.nvfp4_index_k_dequant(kv, dev(np.zeros((1, 1), np.int32)), dev(np.zeros(1, np.int32)),
                             dev(np.zeros(1, np.int32)), 0, out)
    assert (host(out) == 7).all()
