"""GPU parity of topk16_select: bit-identical rows to the oracle on the same
score buffer, including the decode chain on the GPU's own decode scores."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import CANARY_I32, announce, dev, host

pytestmark = pytest.mark.gpu


def gpu_topk(scores, width, valid=None, fb=None, fe=None, ap=None, num_rows=None, out_cols=16):
    import page_scoring_top_amd as ps
    rows = scores.shape[0]
    out = torch.full((rows, out_cols), int(CANARY_I32), dtype=torch.int32, device="cuda")
    s = scores if isinstance(scores, torch.Tensor) else dev(scores)
    ps.topk16_select(s, width, out, None if valid is None else dev(valid),
                     None if fb is None else dev(fb), None if fe is None else dev(fe),
                     None if ap is None else dev(ap), num_rows=num_rows)
    return host(out)


WIDTHS = [1, 2, 15, 16, 17, 63, 64, 65, 100, 255, 768, 769, 1344, 3907, 5000,
          8191, 8193, 32768, 40000]   # two partitions at 8-31 passes, four at 32-63


@pytest.mark.parametrize("width", WIDTHS)
def test_injected_rows(width):
    ti = workloads.injected_rows(seed=width, rows=32, width=width)
    rng = np.random.default_rng(width)
    ap = rng.integers(-1, 4 * width + 2, size=32).astype(np.int32)
    announce(f"topk injected rows width={width}")
    for use_valid in (False, True):
        for use_ap in (False, True):
            kw = dict(valid=ti.valid if use_valid else None, fb=ti.force_begin, fe=ti.force_end,
                      ap=ap if use_ap else None)
            got = gpu_topk(ti.scores, width, **kw)
            want = oracle.topk16(ti.scores, kw["valid"], kw["fb"], kw["fe"], kw["ap"])
            assert np.array_equal(got, want), (use_valid, use_ap,
                                               np.argwhere((got != want).any(1))[:4].ravel())


@pytest.mark.parametrize("width", [300, 5000])
def test_special_bit_patterns(width):
    """Subnormals of both signs next to +-0, NaNs with payloads (quiet and
    signalling, both signs), +-inf and FLT_MAX: the key of each must order as
    its canonical score (NaN as -inf, -0 as +0)."""
    rng = np.random.default_rng(width + 11)
    bits = np.array([0x00000001, 0x80000001, 0x007FFFFF, 0x807FFFFF, 0x00400000, 0x80000000,
                     0x00000000, 0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF,
                     0xFFFFFFFF, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x00800000],
                    dtype=np.uint32)
    rows = 16
    s = rng.standard_normal((rows, width)).astype(np.float32)
    u = s.view(np.uint32)
    for r in range(rows):
        k = int(rng.integers(width // 4, width))           # special patterns over most columns
        cols = rng.choice(width, size=k, replace=False)
        u[r, cols] = bits[rng.integers(0, len(bits), size=k)]
    s[1] = np.where(rng.random(width) < 0.5, np.float32(1e-45), np.float32(-1e-45))
    s[2] = np.float32(-1e-45)                                  # all equal subnormals
    fb = rng.integers(0, width, size=rows).astype(np.int32)
    fe = (fb + rng.integers(0, 4, size=rows)).astype(np.int32)
    announce(f"topk special bit patterns width={width}")
    for kw in (dict(), dict(fb=fb, fe=fe)):
        got = gpu_topk(s, width, **kw)
        want = oracle.topk16(s, None, kw.get("fb"), kw.get("fe"), None)
        assert np.array_equal(got, want), np.argwhere((got != want).any(1))[:4].ravel()


def test_prefill_width_rows():
    """2,048-row x 16,384-column buffer, the prefill score shape, in the benchmark's
    launch configuration (sampled rows compared; all rows are exact by construction)."""
    rng = np.random.default_rng(9)
    s = rng.standard_normal((2048, 16384)).astype(np.float32)
    s[5] = 1.0                             # all-equal row: ties and the fallback
    s[6, ::3] = np.nan
    announce("topk 2048 x 16384")
    got = gpu_topk(s, 16384)
    rows = np.r_[0:16, 2040:2048, rng.choice(2048, 24, replace=False)]
    want = oracle.topk16(s[rows])
    assert np.array_equal(got[rows], want)


def test_long_unsplit_rows():
    """2,048 rows x 65,536 columns: enough rows of at least 64 passes that each
    row stays in one wave.  Special rows among them: all-equal scores, NaN every
    third column, a forced range, a short valid length."""
    rng = np.random.default_rng(10)
    W = 65536
    s = rng.standard_normal((2048, W)).astype(np.float32)
    s[3] = 2.5
    s[4, ::3] = np.nan
    valid = np.full(2048, W, np.int32)
    valid[7] = 1000
    fb = np.zeros(2048, np.int32)
    fe = np.zeros(2048, np.int32)
    fb[9], fe[9] = 40000, 40005
    announce("topk 2048 x 65536 unsplit rows")
    got = gpu_topk(s, W, valid=valid, fb=fb, fe=fe)
    rows = np.r_[0:12, 2040:2048, rng.choice(2048, 12, replace=False)]
    want = oracle.topk16(s[rows], valid[rows], fb[rows], fe[rows])
    assert np.array_equal(got[rows], want)


def test_strides_and_rows_past_num_rows():
    rng = np.random.default_rng(3)
    buf = rng.standard_normal((40, 300)).astype(np.float32)
    announce("topk strided rows, num_rows < buffer rows")
    got = gpu_topk(dev(buf)[:, :250], 250, num_rows=33, out_cols=20)
    want = oracle.topk16(buf[:33, :250])
    assert np.array_equal(got[:33, :16], want)
    assert (got[33:] == CANARY_I32).all() and (got[:, 16:] == CANARY_I32).all()


@pytest.mark.parametrize("cfg", ["tiny", "mtp", "ragged", "long"])
def test_decode_chain_on_gpu_scores(cfg):
    """indexer_score_decode -> topk16_select(valid = own page, append = own page),
    compared with the oracle's top-16 of the GPU's own score buffer."""
    import page_scoring_top_amd as ps
    d = {"tiny": workloads.tiny_decode, "mtp": workloads.mtp_decode,
         "ragged": workloads.ragged_decode, "long": workloads.long_decode}[cfg]()
    R = d.num_reqs
    scores = torch.full((R, 32, d.width), float("nan"), dtype=torch.float32, device="cuda")
    own = torch.empty((R, 32), dtype=torch.int32, device="cuda")
    announce(f"decode chain {cfg}")
    ps.indexer_score_decode(dev(d.kv_cache), dev(d.block_table), dev(d.seq_lens), dev(d.q),
                            dev(d.q_scale), d.qlen, d.width, scores, own, num_reqs=R)
    flat = scores.view(R * 32, d.width)
    own_flat = own.view(R * 32)
    out = torch.full((R * 32, 16), int(CANARY_I32), dtype=torch.int32, device="cuda")
    ps.topk16_select(flat, d.width, out, valid_len=own_flat, append_page=own_flat)
    s_host, own_host, got = host(flat), host(own_flat), host(out)
    want = oracle.topk16(s_host, own_host, None, None, own_host)
    assert np.array_equal(got, want)
    if cfg == "tiny":
        assert (got[28:, 15] == 63).all() and (got[:28] == -1).all()
