"""Pins of the oracle's MXFP8 quantization (vLLM pull request #65508, "How it
works", arithmetic item) against what the page and the formats fix:

* the E8M0 byte equals ceil(log2(amax / 448)) + 127, clamped to [0, 254], for
  every positive finite bf16 magnitude (the identity the page states, here
  computed through a float64 log2 of torch's bf16 value);
* the page's edge blocks: zeros, subnormals, 446/448/450, the 1.75 boundary
  and the value just above it;
* element bytes equal torch's float8_e4m3fn cast (round to nearest even) of
  the element times 2^(127 - sb);
* the reading for non-finite elements (canonical NaN 0x7F)."""

import math

import numpy as np
import torch

import oracle


def bf16_values(bits) -> np.ndarray:
    """Values of bf16 bit patterns through torch (not the oracle)."""
    t = torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).double().numpy()


def expected_scale(amax: float) -> int:
    if amax == 0.0:
        return 0
    return min(max(math.ceil(math.log2(amax / 448.0)) + 127, 0), 254)


def test_bf16_value_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    want = bf16_values(bits)
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got), np.isinf(want))


def test_scale_is_ceil_log2_for_every_magnitude():
    """One element of each positive finite bf16 pattern (and its negative),
    the rest of the block zero."""
    blk = np.zeros(32, dtype=np.uint16)
    vals = bf16_values(np.arange(0, 0x7F80, dtype=np.uint16))
    for bits in range(0, 0x7F80):
        want = expected_scale(float(vals[bits]))
        blk[7] = bits
        assert oracle.mx_block_scale(blk) == want, hex(bits)
        blk[7] = bits | 0x8000
        assert oracle.mx_block_scale(blk) == want, hex(bits | 0x8000)
    blk[7] = 0


def test_page_edge_blocks():
    def scale_of(bits):
        blk = np.zeros(32, dtype=np.uint16)
        blk[31] = bits
        return oracle.mx_block_scale(blk)

    assert scale_of(0x0000) == 0               # all zeros
    assert scale_of(0x0001) == 0               # smallest subnormal
    assert scale_of(0x007F) == 0               # largest subnormal
    assert scale_of(0x43DF) == 127             # 446
    assert scale_of(0x43E0) == 127             # 448 = 1.75 * 2^8: scale 1
    assert scale_of(0x43E1) == 128             # 450: the next value needs scale 2
    for e in range(1, 255):
        assert scale_of((e << 7) | 96) == max(e - 8, 0)      # 1.75 * 2^(e-127)
        assert scale_of((e << 7) | 97) == min(max(e - 7, 0), 254)   # just above it


def test_block_maximum_decides():
    rng = np.random.default_rng(11)
    for _ in range(2000):
        blk = rng.integers(0, 0x7F80, size=32).astype(np.uint16)
        blk |= (rng.integers(0, 2, size=32).astype(np.uint16) << 15)
        amax = float(np.max(np.abs(bf16_values(blk))))
        assert oracle.mx_block_scale(blk) == expected_scale(amax)


def _random_rows(rng, rows, cols, spread):
    """bf16 patterns with per-block magnitudes 2^U(-spread, spread) times N(0,1)."""
    base = rng.standard_normal((rows, cols)).astype(np.float32)
    mag = np.exp2(rng.uniform(-spread, spread, size=(rows, cols // 32, 1))).astype(np.float32)
    x = (base.reshape(rows, cols // 32, 32) * mag).reshape(rows, cols)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_elements_match_torch_rne_cast():
    rng = np.random.default_rng(12)
    x = _random_rows(rng, 64, 2048, 60.0)
    x[0, :32] = 0                                     # a zero block
    x[1, :32] = rng.integers(1, 0x80, size=32)        # a subnormal block
    x[2, :32] = 0x8000                                # negative zeros
    q, s = oracle.mxfp8_quantize(x)
    vals = bf16_values(x).reshape(64, 64, 32)
    amax = np.abs(vals).max(axis=2)
    sb = np.vectorize(expected_scale)(amax)
    assert np.array_equal(s, sb)
    scaled = vals * np.exp2(127.0 - sb)[:, :, None]
    assert np.abs(scaled).max() <= 448.0
    want = torch.from_numpy(scaled.astype(np.float32).reshape(64, 2048)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, want)
    assert (q[2, :32] == 0x80).all()


def test_exact_values_round_trip():
    """Elements that are E4M3 values times a power of two come back exactly."""
    rng = np.random.default_rng(13)
    e4 = np.array([oracle.e4m3_value(b) for b in range(256)])
    finite = np.flatnonzero(np.isfinite(e4))
    for _ in range(200):
        j = int(rng.integers(-100, 100))
        v = e4[rng.choice(finite, size=32)] * 2.0 ** j
        bits = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
        bits = bits.view(np.uint16).reshape(1, 32)
        if not np.array_equal(bf16_values(bits).reshape(-1), v):
            continue                                  # not exact in bf16 at this j
        q, s = oracle.mxfp8_quantize(bits)
        back = np.array([oracle.e4m3_value(b) for b in q[0]]) * 2.0 ** (int(s[0, 0]) - 127)
        assert np.array_equal(back, v)


def test_non_finite_elements():
    blk = np.zeros((1, 32), dtype=np.uint16)
    blk[0, :4] = [0x7F80, 0xFF80, 0x7FC0, 0x3F80]     # +inf, -inf, NaN, 1.0
    q, s = oracle.mxfp8_quantize(blk)
    assert s[0, 0] == 247                             # exponent field 255, fraction 0 / 0.5
    assert list(q[0, :3]) == [0x7F, 0x7F, 0x7F]
    assert q[0, 3] == 0x00                            # 1.0 * 2^-120 rounds to +0
    blk[0, 2] = 0x7FE1                                # NaN with fraction 97/128 > 0.75
    q, s = oracle.mxfp8_quantize(blk)
    assert s[0, 0] == 248
