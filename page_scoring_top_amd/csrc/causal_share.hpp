// causal_share.hpp -- the balanced schedule of the ragged causal prefill
// (indexer_score_prefill_ragged; Modular page "sparse_index_fp8_sm100",
// module description: causal masking over a batch of sequences, -inf past a
// row's visible keys).  Host and device code: score_prefill.hip runs it in
// every work-group, and a CPU test enumerates it for random batches.
//
// The batch's work is its query groups (eight queries of one sequence, one
// per wave), each computing the 128-key chunks its last query sees.  The
// groups lie end to end on a cost line, in sequence order: group x starts
// at P(x), spends kCostSegment on its set-up, chunk j starts at
// P(x) + kCostSegment + kCostChunk j, and its -inf fill ends the group.
// Work-group b of G owns the chunks that start in [C b / G, C (b + 1) / G),
// C the batch's cost; a group with no visible key belongs to the
// work-group whose share holds the end of its set-up.  Every chunk of every
// group then has exactly one owner, and each share costs C / G within one
// chunk plus the set-up of the group it starts in.
#pragma once

#include <cstdint>

#ifndef PAGESCORE_HD
#define PAGESCORE_HD __host__ __device__
#endif

namespace pagescore {

// Queries per group and keys per chunk of the one-token prefill path.
constexpr int kCausalGroupRows = 8;
constexpr int kCausalChunkKeys = 128;

// The cost model, in units of 1/128 of one chunk's time (128 keys against
// eight queries at 64 heads): kCostChunk per chunk, kCostSegment for the
// set-up of a segment (query rows and scales, the first two key chunks, the
// last tile's drain), and one unit per 2^kCostFillShift columns of -inf
// fill (the width rounded up to a chunk, less the computed columns).
// Fitted to per-work-group timings of 4 x 512 queries at 64 heads over
// 4K-16K keys.
constexpr int64_t kCostChunk = 128;
constexpr int64_t kCostSegment = 242;
constexpr int kCostFillShift = 6;
constexpr int64_t kCostFillPerChunk = kCausalChunkKeys >> kCostFillShift;
static_assert(kCostFillPerChunk * (1 << kCostFillShift) == kCausalChunkKeys,
              "a chunk's columns are whole fill units");

// One sequence as the prefill clamps it: q_len queries, klen keys, at most
// hi = min(klen, width) columns.
struct CausalSeq {
    int32_t q_len, klen, hi;
};

PAGESCORE_HD inline int64_t causal_groups(const CausalSeq &c)
{
    return ((int64_t)c.q_len + kCausalGroupRows - 1) / kCausalGroupRows;
}

// Chunks of query group x: the visible keys of its last query, clamp(klen -
// q_len + last + 1, 0, hi), in 128-key chunks.
PAGESCORE_HD inline int64_t causal_group_chunks(const CausalSeq &c, int64_t x)
{
    const int64_t end = (x + 1) * kCausalGroupRows < c.q_len ? (x + 1) * kCausalGroupRows : c.q_len;
    int64_t v = (int64_t)c.klen - c.q_len + end;
    v = v > c.hi ? c.hi : (v < 0 ? 0 : v);
    return (v + kCausalChunkKeys - 1) / kCausalChunkKeys;
}

// The sum of floor(i / 16) over i in [0, n), n >= 0.
PAGESCORE_HD inline int64_t floor16_sum(int64_t n)
{
    const int64_t a = n >> 4, r = n & 15;
    return 8 * a * (a - 1) + r * a;
}

// Chunks of query groups [0, x), x at most the group count, in closed form.
// A full group i sees v_i = d + 8 (i + 1) keys, d = klen - q_len: none for
// i < i0 (v_i <= 0), hi from i1 on (v_i >= hi), and in between
// ceil(v_i / 128) = floor((m + i) / 16) with m = floor((d + 135) / 8), as
// 8 divides 128.  A partial last group sees klen keys, clamped.
PAGESCORE_HD inline int64_t causal_chunks_before(const CausalSeq &c, int64_t x)
{
    static_assert(kCausalGroupRows == 8 && kCausalChunkKeys == 128, "the closed form assumes 8 | 128");
    const int64_t full = c.q_len / kCausalGroupRows;
    const int64_t xf = x < full ? x : full;
    const int64_t d = (int64_t)c.klen - c.q_len;
    int64_t i0 = ((-d - kCausalGroupRows) >> 3) + 1;                 // floor((-d - 8) / 8) + 1
    i0 = i0 < 0 ? 0 : (i0 > xf ? xf : i0);
    int64_t i1 = -((d + kCausalGroupRows - c.hi) >> 3);              // ceil((hi - d - 8) / 8)
    i1 = i1 < i0 ? i0 : (i1 > xf ? xf : i1);
    const int64_t m = (d + kCausalGroupRows + kCausalChunkKeys - 1) >> 3;
    int64_t n = (xf - i1) * ((c.hi + kCausalChunkKeys - 1) / kCausalChunkKeys);
    n += floor16_sum(m + i1) - floor16_sum(m + i0);
    if (x > full)
        n += causal_group_chunks(c, full);
    return n;
}

// Fill units of a whole row: the width rounded up to a chunk.
PAGESCORE_HD inline int64_t causal_fill_units(int32_t width)
{
    return ((int64_t)width + kCausalChunkKeys - 1) / kCausalChunkKeys * kCostFillPerChunk;
}

// Cost of query groups [0, x) of a sequence.
PAGESCORE_HD inline int64_t causal_cost_before(const CausalSeq &c, int64_t x, int64_t fill_units)
{
    return x * (kCostSegment + fill_units) + (kCostChunk - kCostFillPerChunk) * causal_chunks_before(c, x);
}

// The group of sequence c (placed at cost `base`) holding cost lo, which
// the sequence holds: the last x with base + cost(x) <= lo.
PAGESCORE_HD inline int64_t causal_group_at(const CausalSeq &c, int64_t base, int64_t lo, int64_t fill_units)
{
    int64_t a = 0, z = causal_groups(c) - 1;
    while (a < z) {
        const int64_t mid = (a + z + 1) >> 1;
        if (base + causal_cost_before(c, mid, fill_units) <= lo)
            a = mid;
        else
            z = mid - 1;
    }
    return a;
}

// The share [lo, hi) from group x of sequence s (placed at cost `base`):
// unit(x, ja, ke, first) runs chunks [ja, ...) of group x of the current
// sequence over columns [128 ja, ke) -- ke the width for the group's last
// segment, which also fills the row -- and first marks its first chunk.
// next(s) makes sequence s current and returns it (a sequence with no
// queries is skipped); the walk ends past the batch or where a group's
// first chunk starts at or past hi.
template <class Next, class Unit>
PAGESCORE_HD inline void causal_share_walk(int64_t lo, int64_t hi, int s, int num_seqs, int64_t base,
                                           CausalSeq c, int64_t x, int64_t fill_units, int32_t width,
                                           Next &&next, Unit &&unit)
{
    for (;;) {
        const int64_t groups = causal_groups(c);
        for (; x < groups; ++x) {
            const int64_t p = base + causal_cost_before(c, x, fill_units) + kCostSegment;
            if (p >= hi)
                return;
            const int64_t nc = causal_group_chunks(c, x);
            int64_t ja, jb;
            if (nc == 0) {
                ja = 0;
                jb = p >= lo ? 1 : 0;                          // p < hi
            } else {
                ja = lo > p ? (lo - p + kCostChunk - 1) / kCostChunk : 0;
                jb = (hi - p + kCostChunk - 1) / kCostChunk;
                jb = jb < nc ? jb : nc;
            }
            if (ja < jb)
                unit(x, ja, (nc == 0 || jb == nc) ? (int64_t)width : jb * kCausalChunkKeys, ja == 0);
        }
        base += causal_cost_before(c, groups, fill_units);
        do {
            if (++s >= num_seqs)
                return;
            c = next(s);
        } while (c.q_len == 0);
        x = 0;
    }
}

}  // namespace pagescore
