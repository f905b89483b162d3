"""Seeded synthetic inputs shaped like the workloads on the source pages.

This module only draws random bytes and numbers and lays them out in the
buffers the indexer path consumes.  It holds none of the path's arithmetic:
no dequantization, no scoring, no ordering.  Both the CPU oracle (through the
tests) and the GPU path (through the tests and the benchmark) are fed from
here, so the two sides always see identical inputs.

Shapes follow the pages:
  * packed NVFP4 index-K pages are 9,216 bytes (a ``[128, 72]`` uint8 view):
    8,192 bytes of E2M1 codes (64 per token, two per byte) followed by
    1,024 E4M3 block-scale bytes (8 per token) -- vLLM API page
    ``gather_nvfp4_index_k``, module description;
  * decode queries are ``[R, 8, 4, 128]`` E4M3 (8 query slots, 4 index heads,
    depth 128) -- vLLM API page ``indexer_nvfp4_decode_cp``, module
    description and ``_q_exchange_kernel``;
  * prefill queries are ``[T, H, 128]`` E4M3 and keys ``[N, 128]`` E4M3 with
    per-(token, head) and per-key float scales -- Modular page
    ``sparse_index_fp8_sm100``, module description.

Random streams: one ``numpy.random.Generator`` per buffer, spawned from a
``SeedSequence`` so a buffer's contents do not depend on which other buffers
were drawn.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

PAGE_TOKENS = 128
HEAD_DIM = 128
PAGE_BYTES = 9216          # 128 tokens * (64 code bytes + 8 scale bytes)
CODE_BYTES = 8192
SLOTS = 8
DECODE_HEADS = 4

# Stream indices of the spawned generators.
_S_CODES, _S_SCALES, _S_Q, _S_QSCALE, _S_TABLE, _S_K, _S_KSCALE, _S_SEQ, _S_EXTRA = range(9)


def _streams(seed: int, n: int = 9):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def e4m3_bytes_from_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """E4M3 bytes of N(0,1) draws, produced by torch's float32 -> float8_e4m3fn
    cast after clamping to the finite range (input preparation only)."""
    x = rng.standard_normal(size=shape).astype(np.float32)
    t = torch.from_numpy(x).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def random_pages(rng_codes: np.random.Generator, rng_scales: np.random.Generator,
                 num_pages: int, scale_low: int = 0x01, scale_high: int = 0x7E) -> np.ndarray:
    """``num_pages`` packed pages ``[num_pages, 9216]`` uint8.

    Code bytes are uniform over all 256 values (two uniform 4-bit codes each);
    scale bytes are uniform over ``[scale_low, scale_high]`` (by default the
    positive finite E4M3 encodings, as the pages' random index pages use)."""
    pages = np.empty((num_pages, PAGE_BYTES), dtype=np.uint8)
    pages[:, :CODE_BYTES] = rng_codes.integers(0, 256, size=(num_pages, CODE_BYTES),
                                               dtype=np.uint8)
    pages[:, CODE_BYTES:] = rng_scales.integers(scale_low, scale_high + 1,
                                                size=(num_pages, PAGE_BYTES - CODE_BYTES),
                                                dtype=np.uint8)
    return pages


@dataclasses.dataclass
class DecodeInputs:
    name: str
    kv_cache: np.ndarray      # [num_blocks, 9216] uint8
    block_table: np.ndarray   # [R, bt_cols] int32
    seq_lens: np.ndarray      # [R] int32
    q: np.ndarray             # [R, 8, 4, 128] uint8 (E4M3 bytes)
    q_scale: np.ndarray       # [R, 8, 4] float32
    qlen: int
    width: int
    num_reqs: int             # requests to score; rows past it are padding

    @property
    def num_blocks(self) -> int:
        return self.kv_cache.shape[0]


def decode_inputs(name: str, seed: int, seq_lens, qlen: int, width: int,
                  pad_reqs: int = 0, scale_low: int = 0x01, scale_high: int = 0x7E,
                  pool_pages: int | None = None) -> DecodeInputs:
    """Decode inputs for requests with the given context lengths.

    Each request owns ``ceil(seq_len / 128)`` logical pages mapped through a
    random permutation of a shared physical pool, so consecutive logical pages
    are scattered over the cache as in a paged KV cache.  ``pad_reqs`` extra
    requests are appended to every per-request buffer (with random contents)
    but are not part of ``num_reqs``."""
    st = _streams(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    R = len(seq_lens)
    Rt = R + pad_reqs
    pages_per_req = np.maximum((seq_lens + PAGE_TOKENS - 1) // PAGE_TOKENS, 1)
    bt_cols = int(max(width, int(pages_per_req.max())))
    need = int(pages_per_req.sum())
    nb = need if pool_pages is None else max(pool_pages, need)
    kv = random_pages(st[_S_CODES], st[_S_SCALES], nb, scale_low, scale_high)
    perm = st[_S_TABLE].permutation(nb).astype(np.int32)
    bt = np.zeros((Rt, bt_cols), dtype=np.int32)
    off = 0
    for b in range(R):
        n = int(pages_per_req[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    # Padding requests point at valid pages too, so a kernel that wrongly
    # touched them would still read in bounds and be caught by the canaries.
    for b in range(R, Rt):
        bt[b, :] = st[_S_TABLE].integers(0, nb, size=bt_cols, dtype=np.int32)
    seq_all = np.concatenate([seq_lens, st[_S_SEQ].integers(1, 1 + 128 * bt_cols, size=pad_reqs)])
    q = e4m3_bytes_from_normal(st[_S_Q], (Rt, SLOTS, DECODE_HEADS, HEAD_DIM))
    qs = st[_S_QSCALE].uniform(0.5, 2.0, size=(Rt, SLOTS, DECODE_HEADS)).astype(np.float32)
    return DecodeInputs(name, kv, bt, seq_all.astype(np.int32), q, qs, qlen, width, R)


def tiny_decode(seed: int = 1) -> DecodeInputs:
    """One request, one query token, 64 pages: 8,192 tokens of context, so the
    query's own page is 63 and pages 0..62 are scored."""
    return decode_inputs("tiny", seed, [8192], qlen=1, width=64)


def mtp_decode(seed: int = 2) -> DecodeInputs:
    """16 requests x 8 query slots at 30,000 tokens (235 pages, own page 234)."""
    return decode_inputs("mtp", seed, [30000] * 16, qlen=8, width=235)


def long_decode(seed: int = 3) -> DecodeInputs:
    """4 requests x 8 query slots at 500,000 tokens (3,907 pages, own page
    3,906): the long-context decode whose index-K is streamed once per step."""
    return decode_inputs("long", seed, [500000] * 4, qlen=8, width=3907)


def ragged_decode(seed: int = 5) -> DecodeInputs:
    """64 requests x 8 slots with contexts uniform in 1,000..172,032 tokens
    (172,032 = 1,344 pages of 128), plus 8 padding requests; width 1,344."""
    rng = _streams(seed)[_S_SEQ]
    seq = rng.integers(1000, 172032 + 1, size=64)
    return decode_inputs("ragged", seed, seq, qlen=8, width=1344, pad_reqs=8)


@dataclasses.dataclass
class PrefillInputs:
    name: str
    q: np.ndarray        # [T, H, 128] uint8
    q_scale: np.ndarray  # [T, H] float32
    k: np.ndarray        # [N, 128] uint8
    k_scale: np.ndarray  # [N] float32


def prefill_inputs(name: str, seed: int, T: int, H: int, N: int) -> PrefillInputs:
    st = _streams(seed)
    q = e4m3_bytes_from_normal(st[_S_Q], (T, H, HEAD_DIM))
    k = e4m3_bytes_from_normal(st[_S_K], (N, HEAD_DIM))
    qs = st[_S_QSCALE].uniform(0.5, 2.0, size=(T, H)).astype(np.float32)
    ks = st[_S_KSCALE].uniform(0.5, 2.0, size=(N,)).astype(np.float32)
    return PrefillInputs(name, q, qs, k, ks)


def big_prefill(seed: int = 4) -> PrefillInputs:
    """2,048 query tokens x 64 heads against 16,384 keys."""
    return prefill_inputs("prefill", seed, 2048, 64, 16384)


@dataclasses.dataclass
class Nvfp4PrefillInputs:
    """Prefill queries scored against NVFP4 index-K pages gathered into
    contiguous E4M3 keys (the Q8KV8 prefill of the vLLM API page
    ``gather_nvfp4_index_k``): request ``b`` has ``tokens[b]`` queries (rows
    ``sum(tokens[:b])`` onward of ``q``) and ``context[b]`` keys on its first
    ``ceil(context[b] / 128)`` block-table pages."""
    name: str
    kv_cache: np.ndarray      # [num_blocks, 9216] uint8
    block_table: np.ndarray   # [R, bt_cols] int32
    context: np.ndarray       # [R] int32
    num_pages: np.ndarray     # [R] int32
    page_offsets: np.ndarray  # [R] int32: first gathered page of each request
    tokens: np.ndarray        # [R] int32
    q: np.ndarray             # [sum(tokens), H, 128] uint8 (E4M3 bytes)
    q_scale: np.ndarray       # [sum(tokens), H] float32

    @property
    def total_pages(self) -> int:
        return int(self.num_pages.sum())


def nvfp4_prefill_inputs(name: str, seed: int, tokens, contexts, heads: int = DECODE_HEADS,
                         spare_pages: int = 3) -> Nvfp4PrefillInputs:
    """Each request's pages are a random permutation of a shared physical pool
    (with ``spare_pages`` pages that no request uses)."""
    st = _streams(seed)
    tokens = np.asarray(tokens, dtype=np.int32)
    context = np.asarray(contexts, dtype=np.int32)
    npages = ((context.astype(np.int64) + PAGE_TOKENS - 1) // PAGE_TOKENS).astype(np.int32)
    nb = int(npages.sum()) + spare_pages
    kv = random_pages(st[_S_CODES], st[_S_SCALES], nb)
    perm = st[_S_TABLE].permutation(nb).astype(np.int32)
    bt = np.zeros((len(context), max(int(npages.max()), 1)), dtype=np.int32)
    offs = np.zeros(len(context), dtype=np.int32)
    off = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[off:off + n]
        offs[b] = off
        off += int(n)
    Tt = int(tokens.sum())
    q = e4m3_bytes_from_normal(st[_S_Q], (Tt, heads, HEAD_DIM))
    qs = st[_S_QSCALE].uniform(0.5, 2.0, size=(Tt, heads)).astype(np.float32)
    return Nvfp4PrefillInputs(name, kv, bt, context, npages, offs, tokens, q, qs)


def nvfp4_prefill(seed: int = 6) -> Nvfp4PrefillInputs:
    """One request: a 2,048-token prefill chunk with 4 index heads against a
    65,536-token context (512 NVFP4 pages)."""
    return nvfp4_prefill_inputs("nvfp4-prefill", seed, [2048], [65536])


@dataclasses.dataclass
class RaggedPrefillInputs:
    p: PrefillInputs          # q [T, H, 128], keys of all sequences back to back
    q_start: np.ndarray       # [S + 1] int32
    k_start: np.ndarray       # [S] int32
    k_len: np.ndarray         # [S] int32
    width: int


def ragged_prefill_inputs(name: str, seed: int, q_lens, k_lens, H: int) -> RaggedPrefillInputs:
    """A ragged causal prefill batch: sequence s has q_lens[s] queries (the
    last tokens of its context) and k_lens[s] keys, stored back to back."""
    q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    k_start = np.concatenate([[0], np.cumsum(k_lens)[:-1]]).astype(np.int32)
    p = prefill_inputs(name, seed, int(q_start[-1]), H, int(np.sum(k_lens)))
    return RaggedPrefillInputs(p, q_start, k_start, np.asarray(k_lens, np.int32),
                               int(max(k_lens)))


def ragged_prefill(seed: int = 8) -> RaggedPrefillInputs:
    """Four sequences, each a 512-token prefill chunk at the end of a 4,096 /
    8,192 / 12,288 / 16,384-token context, 64 heads: 2,048 query rows against
    40,960 keys, row width 16,384."""
    return ragged_prefill_inputs("ragged-prefill", seed, [512] * 4, [4096, 8192, 12288, 16384], 64)


def mx_activations(seed: int, rows: int, cols: int, spread: float = 40.0) -> np.ndarray:
    """bf16 bit patterns ``[rows, cols]`` (uint16) of attention-output-like
    activations: N(0,1) values times a per-32-element-block magnitude
    2^U(-spread, spread), so blocks span a wide dynamic range (the ROCm MXFP8
    epilogue's tests use a wide magnitude range).  Rounded to bf16 by torch's
    cast (input preparation only)."""
    rng = _streams(seed)[_S_EXTRA]
    base = rng.standard_normal((rows, cols)).astype(np.float32)
    nb = (cols + 31) // 32
    mag = np.exp2(rng.uniform(-spread, spread, size=(rows, nb))).astype(np.float32)
    x = base * np.repeat(mag, 32, axis=1)[:, :cols]
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


# ---------------------------------------------------------------------------
# Score rows with injected special values, for the top-16 selection.
# ---------------------------------------------------------------------------

FLT_MAX = np.float32(np.finfo(np.float32).max)


@dataclasses.dataclass
class TopkInputs:
    scores: np.ndarray        # [rows, width] float32
    valid: np.ndarray         # [rows] int32
    force_begin: np.ndarray   # [rows] int32
    force_end: np.ndarray     # [rows] int32


def injected_rows(seed: int, rows: int, width: int) -> TopkInputs:
    """Score rows whose pattern cycles with ``row % 8``:

    0 plain N(0,1); 1 all equal (every key ties on score); 2 a mix of -0.0 and
    +0.0 with a few positives; 3 NaN and -inf sprinkled over N(0,1);
    4 real +inf values plus a forced column range; 5 FLT_MAX values plus a
    forced range; 6 large values on columns that are multiples of 64 (many
    lanes hold a large key, so many keys pass a lane-maximum threshold);
    7 N(0,1) with a valid length past the width.
    Valid lengths are otherwise uniform in [0, width]."""
    st = _streams(seed)
    rng = st[_S_EXTRA]
    s = rng.standard_normal(size=(rows, width)).astype(np.float32)
    valid = rng.integers(0, width + 1, size=rows).astype(np.int32)
    fb = np.zeros(rows, dtype=np.int32)
    fe = np.zeros(rows, dtype=np.int32)
    for r in range(rows):
        kind = r % 8
        if kind == 1:
            s[r, :] = np.float32(rng.standard_normal())
        elif kind == 2:
            s[r, :] = np.where(rng.random(width) < 0.5, np.float32(-0.0), np.float32(0.0))
            pos = rng.integers(0, width, size=max(1, width // 97))
            s[r, pos] = rng.random(len(pos)).astype(np.float32)
        elif kind == 3:
            m = rng.random(width)
            s[r, m < 0.05] = np.nan
            s[r, (m >= 0.05) & (m < 0.08)] = -np.inf
        elif kind == 4:
            pos = rng.integers(0, width, size=max(1, width // 50))
            s[r, pos] = np.inf
            a = int(rng.integers(0, width))
            fb[r], fe[r] = a, min(width, a + int(rng.integers(1, 12)))
        elif kind == 5:
            pos = rng.integers(0, width, size=max(1, width // 40))
            s[r, pos] = FLT_MAX
            a = int(rng.integers(0, width))
            fb[r], fe[r] = a, min(width, a + int(rng.integers(1, 6)))
        elif kind == 6:
            cols = np.arange(width)[np.arange(width) % 64 < 8]
            s[r, cols] = np.float32(1000.0) + rng.random(len(cols)).astype(np.float32)
            valid[r] = width
        elif kind == 7:
            valid[r] = width + int(rng.integers(1, 1000))
    return TopkInputs(s, valid, fb, fe)


# ---------------------------------------------------------------------------
# Tiles for the matrix-instruction accuracy probe (tests/probe/).
# ---------------------------------------------------------------------------

def mfma_probe_tiles(seed: int, tiles: int):
    """``(a, b)``, each ``[tiles, 16, 128]`` E4M3 bytes.  Even tiles: a's bytes
    uniform over every finite E4M3 byte of either sign (keys of the whole
    E4M3 range, as block-scaled NVFP4 keys reach), b = e4m3(N(0,1)) (queries).
    Odd tiles cancel: the second half of each row repeats the first with a's
    signs flipped, except for 16 depth positions redrawn at random (positive
    finite bytes), so a dot
    product is a small remainder of large terms."""
    rng = _streams(seed)[_S_EXTRA]
    a = rng.integers(0, 256, size=(tiles, 16, 128), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] ^= 0x01            # no NaN bytes
    b = e4m3_bytes_from_normal(rng, (tiles, 16, 128))
    odd = np.arange(tiles) % 2 == 1
    a[odd, :, 64:] = a[odd, :, :64] ^ 0x80
    b[odd, :, 64:] = b[odd, :, :64]
    for t in np.nonzero(odd)[0]:
        for r in range(16):
            pos = 64 + rng.permutation(64)[:16]
            a[t, r, pos] = rng.integers(0, 0x7F, size=16, dtype=np.uint8)
    return a, b
