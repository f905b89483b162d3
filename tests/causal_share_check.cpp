// CPU check of the ragged causal prefill's balanced schedule
// (page_scoring_top_amd/csrc/causal_share.hpp), compiled by
// tests/test_causal_share.py.  For random batches it checks
//  * the closed-form chunk prefix against a direct sum over the groups,
//    each group's chunks taken from the causal mask's definition (query i
//    of a sequence sees clamp(k_len - q_len + i + 1, 0, min(k_len, width))
//    keys; a group computes the chunks of 128 keys its queries see);
//  * that the shares of G work-groups cover every chunk of every group
//    exactly once, a group with no visible key exactly once, with the fill
//    (ke = width) on the group's last segment only and `first` on the
//    segment holding chunk 0;
//  * that no share's chunks start outside it.
// Prints "bad 0" and exits 0 when every check holds.
#define PAGESCORE_HD
#include "causal_share.hpp"

#include <cstdio>
#include <map>
#include <random>
#include <vector>

using namespace pagescore;

static long bad = 0;
static void fail(const char *what, long a, long b, long c)
{
    if (bad++ < 20)
        std::printf("FAIL %s: %ld %ld %ld\n", what, a, b, c);
}

// Chunks of group x from the mask's definition, query by query.
static int64_t group_chunks_by_definition(int32_t q_len, int32_t klen, int32_t width, int64_t x)
{
    const int64_t hi = klen < width ? klen : width;
    int64_t most = 0;
    for (int64_t i = x * 8; i < (x + 1) * 8 && i < q_len; ++i) {
        int64_t v = (int64_t)klen - q_len + i + 1;
        v = v < 0 ? 0 : (v > hi ? hi : v);
        most = v > most ? v : most;
    }
    return (most + 127) / 128;
}

int main()
{
    std::mt19937_64 rng(20260);
    long prefixes = 0, grids = 0;
    // Closed form against the definition.
    for (int it = 0; it < 20000; ++it) {
        const int kind = (int)(rng() % 4);
        CausalSeq c;
        c.q_len = kind == 0 ? (int32_t)(rng() % 24) : (int32_t)(rng() % (kind == 3 ? 20000 : 1500));
        c.klen = rng() % 3 == 0 ? (int32_t)(rng() % 40) : (int32_t)(rng() % 60000);
        const int32_t width = 1 + (int32_t)(rng() % 2 == 0 ? rng() % 300 : rng() % 70000);
        c.hi = c.klen < width ? c.klen : width;
        const int64_t groups = causal_groups(c);
        int64_t sum = 0;
        for (int64_t x = 0; x <= groups; ++x) {
            if (groups < 300 || x % 97 == 0 || x == groups || x + 1 == groups) {
                ++prefixes;
                const int64_t got = causal_chunks_before(c, x);
                if (got != sum)
                    fail("chunk prefix", c.q_len, c.klen, (long)x);
            }
            if (x < groups) {
                const int64_t n = group_chunks_by_definition(c.q_len, c.klen, width, x);
                if (n != causal_group_chunks(c, x))
                    fail("group chunks", c.q_len, c.klen, (long)x);
                sum += n;
            }
        }
    }
    // Shares of random batches.
    const int grid_sizes[] = {1, 2, 7, 256, 257, 1024};
    for (int it = 0; it < 2500; ++it) {
        const int num_seqs = 1 + (int)(rng() % (it % 8 == 0 ? 256 : 12));
        const int32_t width = 1 + (int32_t)(rng() % 4 == 0 ? rng() % 500 : rng() % 40000);
        std::vector<CausalSeq> seqs(num_seqs);
        for (auto &c : seqs) {
            const int kind = (int)(rng() % 5);
            c.q_len = kind == 0 ? 0 : (int32_t)(kind == 1 ? rng() % 9 : rng() % 1500);
            c.klen = kind == 2 ? (int32_t)(rng() % 30) : (int32_t)(rng() % 50000);
            c.hi = c.klen < width ? c.klen : width;
        }
        const int64_t fill = causal_fill_units(width);
        std::vector<int64_t> start(num_seqs + 1, 0);
        for (int s = 0; s < num_seqs; ++s)
            start[s + 1] = start[s] + causal_cost_before(seqs[s], causal_groups(seqs[s]), fill);
        const int64_t total = start[num_seqs];
        for (const int G : grid_sizes) {
            ++grids;
            std::map<std::pair<int, int64_t>, std::vector<int>> seen;   // (s, x) -> owners per chunk
            for (int64_t b = 0; b < G; ++b) {
                const int64_t lo = total * b / G, hi = total * (b + 1) / G;
                if (lo >= hi)
                    continue;
                int s = -1;
                for (int t = 0; t < num_seqs; ++t)
                    if (start[t + 1] > start[t] && start[t] <= lo && lo < start[t + 1])
                        s = t;
                if (s < 0) {
                    fail("no sequence holds the share", (long)b, (long)lo, G);
                    continue;
                }
                int cur = s;
                auto next = [&](int t) {
                    cur = t;
                    return seqs[t];
                };
                auto unit = [&](int64_t x, int64_t ja, int64_t ke, bool first) {
                    const CausalSeq &c = seqs[cur];
                    const int64_t nc = causal_group_chunks(c, x);
                    const int64_t jb = ke == width ? (nc == 0 ? 1 : nc) : (ke + 127) / 128;
                    if (ke != width && ke % 128 != 0)
                        fail("segment end inside a chunk", cur, (long)x, (long)ke);
                    if (first != (ja == 0))
                        fail("first flag", cur, (long)x, (long)ja);
                    if (ke == width && nc > 0 && (int64_t)width < nc * 128 - 127)
                        fail("fill before the last chunk", cur, (long)x, (long)ke);
                    // Chunk starts on the cost line lie inside the share.
                    const int64_t p = start[cur] + causal_cost_before(c, x, fill) + kCostSegment;
                    for (int64_t j = ja; j < (nc == 0 ? 1 : jb); ++j) {
                        const int64_t at = p + kCostChunk * j;
                        if (at < lo || at >= hi)
                            fail("chunk outside its share", cur, (long)x, (long)j);
                    }
                    auto &v = seen[{cur, x}];
                    if (v.empty())
                        v.assign(nc == 0 ? 1 : nc, 0);
                    for (int64_t j = ja; j < (nc == 0 ? 1 : jb) && j < (int64_t)v.size(); ++j)
                        ++v[j];
                };
                const CausalSeq c = seqs[s];
                causal_share_walk(lo, hi, s, num_seqs, start[s], c, causal_group_at(c, start[s], lo, fill), fill,
                                  width, next, unit);
            }
            for (int s = 0; s < num_seqs; ++s)
                for (int64_t x = 0; x < causal_groups(seqs[s]); ++x) {
                    const auto f = seen.find({s, x});
                    if (f == seen.end()) {
                        fail("group without owner", s, (long)x, G);
                        continue;
                    }
                    for (size_t j = 0; j < f->second.size(); ++j)
                        if (f->second[j] != 1)
                            fail("chunk owners", s, (long)x, f->second[j]);
                }
        }
    }
    std::printf("prefixes %ld grids %ld bad %ld\n", prefixes, grids, bad);
    return bad != 0;
}
