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
// columns).  A row is cut into 1..16 contiguous partitions, one wave each, in
// one work-group; each wave streams its columns in passes of 256 (4 per lane)
// and keeps its best 16 so far, one key per lane in lanes 0..15.  At the end
// the row's first wave selects the best 16 of the partitions' results.
//
// Selection of the best 16 among a few keys per lane, as the MSA pull request
// describes it for a 32-lane warp, here on 64 lanes: (1) each lane takes the
// maximum of its keys; (2) the largest high word t such that at least 16 lane
// maxima reach it is found by a most-significant-bits-first search whose
// counts are ballots; (3) every key whose high word reaches t survives -- the
// 16 lanes whose maxima reach t hold 16 distinct keys no smaller than any key
// below t, so the best 16 are among the survivors; (4) survivors are compacted
// into LDS (ballot prefix counts) and each is ranked by counting the survivors
// above it.  When more than 64 keys survive (ties in the score), the exact
// 16th key is found by a 64-bit bisection over all the keys instead, and
// exactly 16 survive.
//
// In a pass, a new key at or below the wave's current 16th key cannot enter
// its best 16 and is dropped before selection; a pass that keeps no new key
// costs one compare and ballot per slot.
#include "device_common.hpp"
#include "launch.hpp"

namespace pagescore {

namespace {

constexpr int kMaxWavesPerRow = 16;
constexpr int kPerLane = 4;                        // new keys per lane and pass
constexpr int kPassCols = kPerLane * kWave;        // 256 columns per pass
constexpr int kBlockWaves = 16;                    // waves per work-group (rows x partitions)

__device__ __forceinline__ uint64_t make_key(float s, int col, int fb, int fe)
{
    uint32_t u = __float_as_uint(s);
    if (col >= fb && col < fe)
        u = 0x7F800000u;                       // forced: +inf
    else if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        u = 0xFF800000u;                       // NaN: -inf
    else if (u == 0x80000000u)
        u = 0u;                                // -0: +0
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)col);
}

__device__ __forceinline__ int key_col(uint64_t key)
{
    return (int)(0xFFFFFFFFu - (uint32_t)key);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Set bits of `mask` below this lane.
__device__ __forceinline__ int bits_below(uint64_t mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Orders this wave's LDS accesses before and after (a wave's LDS operations
// execute in order; this stops the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The 16 largest keys among key[0..N) of all 64 lanes (0 = empty slot).
// Returns the r-th largest in lane r < 16 (0 when there are fewer than r + 1
// keys) and 0 in lanes 16..63.  `surv` (64 keys) and `res` (16 keys) are the
// wave's LDS scratch.
template <int N>
__device__ __forceinline__ uint64_t wave_top16(const uint64_t (&key)[N], uint64_t *surv,
                                               uint64_t *res, int lane)
{
    uint64_t lmax = 0;
#pragma unroll
    for (int i = 0; i < N; ++i)
        lmax = key[i] > lmax ? key[i] : lmax;
    const uint32_t lhi = (uint32_t)(lmax >> 32);
    // Two bits per step: the three candidates' counts are independent.
    uint32_t t = 0;
    for (int sh = 30; sh >= 0; sh -= 2) {
        const uint32_t c1 = t | (1u << sh), c2 = t | (2u << sh), c3 = t | (3u << sh);
        const int n1 = __popcll(__ballot(lhi >= c1));
        const int n2 = __popcll(__ballot(lhi >= c2));
        const int n3 = __popcll(__ballot(lhi >= c3));
        t = n3 >= kTopk ? c3 : (n2 >= kTopk ? c2 : (n1 >= kTopk ? c1 : t));
    }
    uint64_t mask[N];
    int total = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        mask[i] = __ballot(key[i] != 0 && (uint32_t)(key[i] >> 32) >= t);
        total += __popcll(mask[i]);
    }
    if (total > kWave) {
        // Exact 16th key (at least 16 keys exist: more than 64 survived).
        uint64_t kth = 0;
        for (int bit = 63; bit >= 0; --bit) {
            const uint64_t cand = kth | (1ull << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < N; ++i)
                cnt += __popcll(__ballot(key[i] >= cand));
            if (cnt >= kTopk)
                kth = cand;
        }
        total = 0;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            mask[i] = __ballot(key[i] >= kth);
            total += __popcll(mask[i]);
        }
    }
    int base = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if ((mask[i] >> lane) & 1ull)
            surv[base + bits_below(mask[i])] = key[i];
        base += __popcll(mask[i]);
    }
    wave_lds_sync();
    if (lane < total) {
        const uint64_t mine = surv[lane];
        int rank = 0;
        for (int j = 0; j < total; ++j)
            rank += surv[j] > mine ? 1 : 0;
        if (rank < kTopk)
            res[rank] = mine;
    }
    wave_lds_sync();
    const int got = total < kTopk ? total : kTopk;
    const uint64_t r = lane < got ? res[lane] : 0;
    wave_lds_sync();   // the scratch may be rewritten by the caller's next selection
    return r;
}

__device__ __forceinline__ void load_pass(const float *srow, int c, int c1, float (&v)[kPerLane])
{
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
        v[i] = c + i * kWave < c1 ? srow[c + i * kWave] : 0.0f;
}

__global__ __launch_bounds__(1024) void topk16_kernel(
    const float *__restrict__ scores, int64_t row_stride, int32_t num_rows, int32_t width,
    const int32_t *__restrict__ valid_len, const int32_t *__restrict__ force_begin,
    const int32_t *__restrict__ force_end, const int32_t *__restrict__ append_page,
    int32_t waves_per_row, int32_t *__restrict__ out, int64_t out_stride)
{
    __shared__ uint64_t surv[kBlockWaves][kWave];
    __shared__ uint64_t res[kBlockWaves][kTopk];
    __shared__ uint64_t part_best[kBlockWaves][kTopk];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int rows_per_block = (int)(blockDim.x / kWave) / waves_per_row;
    const int row_in_block = wave / waves_per_row;
    const int part = wave % waves_per_row;
    const int64_t row = (int64_t)blockIdx.x * rows_per_block + row_in_block;
    const bool live = row < num_rows;   // no early return: the work-group meets at a barrier

    // The row's parameters, all requested at once (the appended page too).
    int n = 0, fb = 0, fe = 0, ap = -1;
    const float *srow = scores;
    if (live) {
        n = valid_len ? valid_len[row] : width;
        n = n < 0 ? 0 : (n > width ? width : n);
        fb = force_begin ? force_begin[row] : 0;
        fe = force_end ? force_end[row] : 0;
        ap = append_page ? append_page[row] : -1;
        srow = scores + row * row_stride;
    }

    // This wave's columns: whole 64-column groups, split evenly.
    const int groups = (n + kWave - 1) / kWave;
    const int span = ((groups + waves_per_row - 1) / waves_per_row) * kWave;
    const int c0 = part * span;
    const int c1 = c0 + span < n ? c0 + span : n;

    uint64_t best = 0;   // lane r < 16: this partition's r-th best key so far
    if (c0 < c1) {
        float v[kPerLane];
        load_pass(srow, c0 + lane, c1, v);
        for (int pc = c0; pc < c1; pc += kPassCols) {
            float nv[kPerLane];
            if (pc + kPassCols < c1)
                load_pass(srow, pc + kPassCols + lane, c1, nv);
            const uint64_t floor_key = readlane_u64(best, kTopk - 1);
            uint64_t key[kPerLane + 1];
            bool any_new = false;
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) {
                const int c = pc + lane + i * kWave;
                uint64_t k = c < c1 ? make_key(v[i], c, fb, fe) : 0;
                k = k > floor_key ? k : 0;
                any_new |= k != 0;
                key[i] = k;
            }
            key[kPerLane] = best;
            if (__any(any_new))
                best = wave_top16(key, surv[wave], res[wave], lane);
            if (pc + kPassCols < c1) {
#pragma unroll
                for (int i = 0; i < kPerLane; ++i)
                    v[i] = nv[i];
            }
        }
    }

    uint64_t final_best = best;
    if (waves_per_row > 1) {
        if (lane < kTopk)
            part_best[wave][lane] = best;
        __syncthreads();
        if (part == 0) {
            // Partition results of this row: waves_per_row * 16 <= 256 keys, 4 per lane.
            const uint64_t *pb = &part_best[wave][0];
            const int cnt = waves_per_row * kTopk;
            uint64_t key[kPerLane];
#pragma unroll
            for (int i = 0; i < kPerLane; ++i)
                key[i] = lane + i * kWave < cnt ? pb[lane + i * kWave] : 0;
            final_best = wave_top16(key, surv[wave], res[wave], lane);
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
                         int64_t out_stride, hipStream_t stream)
{
    // Partitions per row: about one pass (256 columns) each, a power of two
    // up to 16; rows share a work-group of up to 16 waves.
    const int64_t passes = ((int64_t)width + kPassCols - 1) / kPassCols;
    int wpr = 1;
    while (wpr < kMaxWavesPerRow && wpr < passes)
        wpr *= 2;
    int rows_per_block = 4 / wpr;
    rows_per_block = rows_per_block < 1 ? 1 : rows_per_block;
    const int threads = wpr * rows_per_block * kWave;
    const int64_t blocks = ((int64_t)num_rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(topk16_kernel, dim3((uint32_t)blocks), dim3(threads), 0, stream, scores,
                       row_stride, num_rows, width, valid_len, force_begin, force_end,
                       append_page, (int32_t)wpr, out, out_stride);
    return hipGetLastError();
}

}  // namespace pagescore
