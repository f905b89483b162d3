// topk16.hip -- K4: exact top-16 column ids per score row.
//
// Order (GitHub pull request wolfcomos/MSA #1, "Changes" and "Behaviour
// changes"): score descending with forced columns as +inf, NaN as -inf and -0
// as +0, then the lower column.  Output row (vLLM API page
// "indexer_nvfp4_decode_cp", module description and _merge_kernel): the k best
// columns in that order (k = 15 when an own page is appended, else 16), then
// the appended page, then -1.
//
// Every candidate gets a distinct 64-bit key: the order-preserving image of its
// canonical score bits in the high word (sign set: all bits flipped; sign
// clear: the sign bit set), and 0xFFFFFFFF - column in the low word, so a
// larger key is a better candidate and no two keys tie.  Real keys are never
// 0, which marks an empty slot.
//
// Work split (the exact merge of the vLLM page's module description: the best
// 16 of a row lie in the union of the best 16 of any partition of its
// columns).  A row is cut into 1, 2 or 4 contiguous partitions, one wave each
// and one per SIMD of the work-group.  A wave holds up to 1,024 of its columns
// in registers (16 per lane) and keeps its best 16 so far, one key per lane in
// lanes 0..15; wider partitions take several such passes.  The row's first
// wave then merges the partitions' sorted results, at most 64 keys, one per
// lane, with the last steps of a bitonic sort.
//
// Selection of the best 16 among a few keys per lane, after the MSA pull
// request's warp scheme, here on 64 lanes: (1) each lane takes the maximum of
// its keys' high words; (2) a bitonic sort of those 64 maxima across the wave
// (DPP row and quad moves and the permlane swaps; no LDS) gives t, the 16th
// largest; (3) every key whose high word reaches t survives -- the 16 lanes
// whose maxima reach t hold 16 distinct keys no smaller than any key below t,
// so the best 16 are among the survivors; (4) the survivors are placed one per
// lane through LDS (each lane counts its own, a DPP prefix sum gives the
// places), and each is ranked by counting the survivors above it, read back
// from LDS; the 16 best are written in rank order.  When more than 64 keys survive (ties in the
// score), the exact 16th key is found by a 64-bit bisection over all the keys
// instead, and exactly 16 survive.
//
// In a pass, a new key whose high word is below that of the wave's current
// 16th key cannot enter its best 16 and is dropped before selection; a pass
// that keeps no new key costs one compare and ballot per slot, and one that
// keeps at most 48 sorts them with the 16 held keys directly, without the
// threshold step.
#include "device_common.hpp"
#include "launch.hpp"
#include "wave_keys.hpp"

namespace pagescore {

namespace {

constexpr int kMaxWavesPerRow = 4;
// Cache policy of the score loads of long rows (at least kStreamPasses
// passes): nontemporal, each score is read once (2,048 x 65,536: 101 -> 93
// us; 2,048 x 16,384: 29.3 -> 28.7 us).  Shorter rows, such as the decode
// rows the score kernel has just written, keep the default policy.
constexpr int kStreamLoad = 2;
constexpr int64_t kStreamPasses = 8;
constexpr int64_t kUnsplitPasses = 64;             // rows this long stay in one wave (see launch)
constexpr int64_t kHalfSplitPasses = 8;            // rows of 8..31 passes take two partitions (see launch)
constexpr int kWideLane = 16;                      // columns per lane and pass (1,024 per wave)
constexpr int kNarrowLane = 4;                     // for rows of at most 256 columns
constexpr int kBlockWaves = 4;                     // one wave per SIMD


// The candidates of one selection: N columns per lane given by their high
// words (0 = empty) at columns base + 64 i + lane, plus up to 16 earlier
// winners (`held`, one full key per lane in lanes 0..15).
template <int N>
struct Candidates {
    uint32_t hi[N];
    int base;
    uint64_t held;
};

// Place the candidates that `keep` selects (slot -1 is the held key) one
// per lane in surv[0..total) and return total; nothing is placed when more
// than 64 are selected.  Each lane counts its own and a prefix sum across
// the wave places them; a lane's unselected candidates go to a spare slot of
// its own, so the stores need no branches.
template <int N, typename Keep>
__device__ __forceinline__ int place_survivors(const Candidates<N> &c, Keep keep, uint64_t *surv,
                                               int lane)
{
    int mine = keep(-1) ? 1 : 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
        mine += keep(i) ? 1 : 0;
    const int before = wave_prefix_sum(mine, lane);
    const int total = __builtin_amdgcn_readlane(before + mine, kWave - 1);
    if (total <= kWave) {
        int pos = before;
        const bool kh = keep(-1);
        surv[kh ? pos : kWave + lane] = c.held;
        pos += kh ? 1 : 0;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const bool k = keep(i);
            surv[k ? pos : kWave + lane] = make_key(c.hi[i], c.base + i * kWave + lane);
            pos += k ? 1 : 0;
        }
    }
    return total;
}

// The 16 largest candidate keys, the r-th largest in lane r < 16 and 0 in
// lanes 16..63 (0 also past the number of candidates).  `surv` is 128 keys
// of the wave's LDS: 64 places for survivors and a spare slot per lane.
template <int N>
__device__ __forceinline__ uint64_t wave_top16(const Candidates<N> &c, uint64_t *surv, int lane)
{
    const uint32_t held_hi = (uint32_t)(c.held >> 32);
    // With 16 keys held, the caller's floor has dropped every key below the
    // 16th: usually only a few are left, and when the held keys and those
    // fit in 64 lanes they are placed and sorted directly, without the
    // threshold step.
    int total = kWave + 1;
    if (readlane_u64(c.held, kTopk - 1) != 0)
        total = place_survivors(
            c, [&](int i) { return i < 0 ? c.held != 0 : c.hi[i] != 0; }, surv, lane);
    if (total > kWave) {
        uint32_t lmax = held_hi;
#pragma unroll
        for (int i = 0; i < N; ++i)
            lmax = c.hi[i] > lmax ? c.hi[i] : lmax;
        uint32_t t = __builtin_amdgcn_readlane(wave_sort_desc<64>(lmax, lane), kTopk - 1);
        t = t > 0 ? t : 1;   // real keys only

        // Survivors: keys whose high word reaches t.
        total = place_survivors(
            c, [&](int i) { return (i < 0 ? held_hi : c.hi[i]) >= t; }, surv, lane);
    }
    if (total > kWave) {
        // Ties on the high word: the exact 16th key (at least 16 keys exist,
        // since more than 64 survived), and exactly 16 survivors.
        uint64_t kth = 0;
        for (int bit = 63; bit >= 0; --bit) {
            const uint64_t cand = kth | (1ull << bit);
            int cnt = lanes_set(__ballot(c.held >= cand));
#pragma unroll
            for (int i = 0; i < N; ++i)
                cnt += lanes_set(__ballot(c.hi[i] != 0 &&
                                          make_key(c.hi[i], c.base + i * kWave + lane) >= cand));
            if (cnt >= kTopk)
                kth = cand;
        }
        total = place_survivors(
            c,
            [&](int i) {
                return i < 0 ? c.held >= kth
                             : (c.hi[i] != 0 && make_key(c.hi[i], c.base + i * kWave + lane) >= kth);
            },
            surv, lane);
    }
    wave_lds_sync();
    // The survivors sit in places 0 .. total-1 (usually about 20), each
    // taken by one lane.  A survivor's rank is the number of survivors above
    // it (real keys are distinct), counted against every place read back
    // two at a time; the 16 best are written to the places of their ranks.
    // Measured against a bitonic sort of the survivors: 4.83 -> 4.70 us at
    // 128 x 3,906 and 29 -> 27 us at 2,048 x 16,384.
    const uint64_t mine = lane < total ? surv[lane] : 0;
    int r0 = 0, r1 = 0;
    const int pairs = __builtin_amdgcn_readfirstlane(total >> 1);
    for (int j = 0; j < pairs; ++j) {
        const uint64_t a = surv[2 * j], b = surv[2 * j + 1];
        r0 += a > mine ? 1 : 0;
        r1 += b > mine ? 1 : 0;
    }
    if (total & 1)
        r0 += surv[total - 1] > mine ? 1 : 0;
    const int rank = r0 + r1;
    wave_lds_sync();   // every place read before the best are rewritten
    if (lane < total && rank < kTopk)
        surv[rank] = mine;
    wave_lds_sync();
    const uint64_t best = lane < (total < kTopk ? total : kTopk) ? surv[lane] : 0;
    wave_lds_sync();   // the scratch may be rewritten by the caller's next selection
    return best;
}

template <int kPerLane, int kLoadPolicy>
__global__ __launch_bounds__(256) void topk16_kernel(
    const float *__restrict__ scores, int64_t row_stride, int32_t num_rows, int32_t width,
    const int32_t *__restrict__ valid_len, const int32_t *__restrict__ force_begin,
    const int32_t *__restrict__ force_end, const int32_t *__restrict__ append_page,
    int32_t waves_per_row, int32_t *__restrict__ out, int64_t out_stride)
{
    constexpr int kPassCols = kPerLane * kWave;
    __shared__ uint64_t surv[kBlockWaves][2 * kWave];
    __shared__ uint64_t part_best[kBlockWaves][kTopk];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int rows_per_block = kBlockWaves / waves_per_row;
    const int row_in_block = wave / waves_per_row;
    const int part = wave % waves_per_row;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + row_in_block;
    const bool live = row < num_rows;   // no early return: the work-group meets at a barrier
    const float *srow = scores + (live ? row : 0) * row_stride;

    // This wave's columns: whole 64-column groups of the width, split evenly;
    // the row's valid length trims them once it is known.  The first pass is
    // requested together with the row's parameters (every lane loads every
    // slot, so the loads issue back to back with no branch between them).
    const int groups = (width + kWave - 1) / kWave;
    const int span = ((groups + waves_per_row - 1) / waves_per_row) * kWave;
    const int c0 = part * span;
    const int cw = live ? (c0 + span < width ? c0 + span : width) : c0;   // loadable end
    // Columns [c0, cw) of the row through a descriptor: a column past cw
    // reads as zero, and the loads of a pass differ only in their immediate
    // offsets.
    const __amdgpu_buffer_rsrc_t rsrc = uniform_rsrc(srow + c0, (uint32_t)(cw - c0) * 4u);
    auto load = [&](int pc, float (&v)[kPerLane]) {
        const uint32_t off = (uint32_t)(pc - c0 + lane) * 4u;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 rsrc, off + i * kWave * 4, 0, kLoadPolicy));
    };
    float v[kPerLane];
    if (c0 < cw)
        load(c0, v);

    int n = 0, fb = 0, fe = 0, ap = -1;
    if (live) {
        n = valid_len ? valid_len[row] : width;
        n = n < 0 ? 0 : (n > width ? width : n);
        fb = force_begin ? force_begin[row] : 0;
        fe = force_end ? force_end[row] : 0;
        ap = append_page ? append_page[row] : -1;
    }
    const int c1 = cw < n ? cw : n;   // this wave's candidates: [c0, c1)
    const uint32_t fspan = fe > fb ? (uint32_t)(fe - fb) : 0u;   // forced columns [fb, fe)

    uint64_t best = 0;   // lane r < 16: this partition's r-th best key so far
    for (int pc = c0; pc < c1; pc += kPassCols) {
        float nv[kPerLane];
        if (pc + kPassCols < c1)
            load(pc + kPassCols, nv);
        Candidates<kPerLane> cand;
        cand.base = pc;
        cand.held = best;
        // Keys whose high word is below the current 16th best cannot enter.
        // Column checks are unsigned ranges: col - fb < fe - fb (forced) and,
        // in the pass that reaches c1, lane < c1 - (pc + 64 i).
        const uint32_t floor_hi = (uint32_t)(readlane_u64(best, kTopk - 1) >> 32);
        const int rel = pc - fb + lane;
        uint32_t hmax = 0;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            uint32_t h = key_hi(v[i], (uint32_t)(rel + i * kWave) < fspan);
            h = h >= floor_hi ? h : 0u;
            cand.hi[i] = h;
        }
        if (pc + kPassCols > c1) {
#pragma unroll
            for (int i = 0; i < kPerLane; ++i)
                cand.hi[i] = lane < c1 - pc - i * kWave ? cand.hi[i] : 0u;
        }
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            hmax = cand.hi[i] > hmax ? cand.hi[i] : hmax;
        if (__any(hmax != 0))
            best = wave_top16(cand, surv[wave], lane);
        if (pc + kPassCols < c1) {
#pragma unroll
            for (int i = 0; i < kPerLane; ++i)
                v[i] = nv[i];
        }
    }

    uint64_t final_best = best;
    if (waves_per_row > 1) {
        if (lane < kTopk)
            part_best[wave][lane] = best;
        __syncthreads();
        if (part == 0) {
            // The partitions' results, at most 4 x 16 = 64 keys, one per
            // lane.  Each list is sorted; with lists 1 and 3 reversed the
            // lanes hold 16-blocks sorted descending and ascending in turn,
            // so the merge steps of a bitonic sort (K = 32, 64) finish it.
            const int p = lane / kTopk, r = lane % kTopk;
            const int src = (p & 1) ? kTopk - 1 - r : r;
            uint64_t x = p < waves_per_row ? part_best[row_in_block * waves_per_row + p][src] : 0;
            x = bitonic_step<32, 16>(x, lane);
            x = bitonic_step<32, 8>(x, lane);
            x = bitonic_step<32, 4>(x, lane);
            x = bitonic_step<32, 2>(x, lane);
            x = bitonic_step<32, 1>(x, lane);
            x = bitonic_step<64, 32>(x, lane);
            x = bitonic_step<64, 16>(x, lane);
            x = bitonic_step<64, 8>(x, lane);
            x = bitonic_step<64, 4>(x, lane);
            x = bitonic_step<64, 2>(x, lane);
            x = bitonic_step<64, 1>(x, lane);
            final_best = x;
        }
    }
    if (!live || part != 0)
        return;

    const int k = append_page ? kTopk - 1 : kTopk;
    const int m = n < k ? n : k;   // columns selected
    int32_t *orow = out + row * out_stride;
    if (lane < m)
        orow[lane] = key_col(final_best);
    else if (lane < kTopk)
        orow[lane] = (lane == m && ap >= 0) ? ap : -1;
}

}  // namespace

hipError_t launch_topk16(const float *scores, int64_t row_stride, int32_t num_rows, int32_t width,
                         const int32_t *valid_len, const int32_t *force_begin,
                         const int32_t *force_end, const int32_t *append_page, int32_t *out,
                         int64_t out_stride, int num_cus, hipStream_t stream)
{
    // Partitions per row: about one pass (1,024 columns) each, 1, 2 or 4;
    // rows share a work-group of 4 waves.  Rows of at most 256 columns take
    // 4 columns per lane.  Rows of 64 passes or more, enough of them to give
    // every SIMD two waves unsplit, are not split: the partitions' merge and
    // extra waves then cost more than they spread (2,048 x 65,536: 109 ->
    // 101 us; 2,048 x 131,072: 200 -> 184 us).  Rows of 8 to 31 passes take
    // two partitions (2,048 x 16,384: 31.1 -> 29.6 us; 8,192 to 24,576
    // columns gain 3-5%), while 32 passes measured 4% slower with two.
    const bool narrow = width <= kNarrowLane * kWave;
    const int64_t pass_cols = (int64_t)kWideLane * kWave;
    const int64_t passes = ((int64_t)width + pass_cols - 1) / pass_cols;
    const int64_t simds = (int64_t)(num_cus > 0 ? num_cus : 256) * 4;
    int wpr = 1;
    if (!(passes >= kUnsplitPasses && num_rows >= 2 * simds)) {
        const int cap = (passes >= kHalfSplitPasses && passes < 4 * kHalfSplitPasses) ? 2 : kMaxWavesPerRow;
        while (wpr < cap && wpr < passes)
            wpr *= 2;
    }
    const int rows_per_block = kBlockWaves / wpr;
    const int64_t blocks = ((int64_t)num_rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    if (narrow)
        hipLaunchKernelGGL((topk16_kernel<kNarrowLane, 0>), dim3((uint32_t)blocks), dim3(kBlockWaves * kWave),
                           0, stream, scores, row_stride, num_rows, width, valid_len, force_begin,
                           force_end, append_page, (int32_t)wpr, out, out_stride);
    else if (passes >= kStreamPasses)
        hipLaunchKernelGGL((topk16_kernel<kWideLane, kStreamLoad>), dim3((uint32_t)blocks),
                           dim3(kBlockWaves * kWave), 0, stream, scores, row_stride, num_rows, width,
                           valid_len, force_begin, force_end, append_page, (int32_t)wpr, out,
                           out_stride);
    else
        hipLaunchKernelGGL((topk16_kernel<kWideLane, 0>), dim3((uint32_t)blocks),
                           dim3(kBlockWaves * kWave), 0, stream, scores, row_stride, num_rows, width,
                           valid_len, force_begin, force_end, append_page, (int32_t)wpr, out,
                           out_stride);
    return hipGetLastError();
}

}  // namespace pagescore
