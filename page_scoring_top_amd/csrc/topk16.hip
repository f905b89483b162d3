// topk16.hip -- K4: exact top-16 column ids per score row, one wave64 per row.
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
// Selection, as the MSA pull request describes it for a 32-lane warp, here on
// 64 lanes: (1) each lane takes the maximum of its columns' keys (columns
// lane, lane+64, ...); (2) the k-th largest of the 64 lane maxima is found by
// a most-significant-bit-first bisection whose counts are ballots; (3) every
// key at or above it survives -- at least k do, and the k best are among them
// because each of the k lanes whose maximum reaches the threshold contributes
// a distinct key no smaller than it; (4) survivors are compacted into LDS in
// column order (ballot prefix counts, so the result does not depend on
// scheduling) and each is ranked by counting the survivors above it; (5) when
// more than 64 keys survive, k exact rounds of "largest key below the previous
// one" run over the row instead.
#include "device_common.hpp"
#include "launch.hpp"

namespace pagescore {

namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kSurvivorCap = 64;

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

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask)
{
    const uint32_t lo = __shfl_xor((uint32_t)v, mask);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), mask);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = shfl_xor_u64(v, off);
        v = o > v ? o : v;
    }
    return v;
}

// k-th largest of the 64 lane values (k in 1..64).
__device__ __forceinline__ uint64_t wave_kth_largest(uint64_t v, int k)
{
    uint64_t pfx = 0;
    for (int bit = 63; bit >= 0; --bit) {
        const uint64_t cand = pfx | (1ull << bit);
        const int cnt = __popcll(__ballot(v >= cand));
        if (cnt >= k)
            pfx = cand;
    }
    return pfx;
}

__global__ __launch_bounds__(256) void topk16_kernel(
    const float *__restrict__ scores, int64_t row_stride, int32_t num_rows, int32_t width,
    const int32_t *__restrict__ valid_len, const int32_t *__restrict__ force_begin,
    const int32_t *__restrict__ force_end, const int32_t *__restrict__ append_page,
    int32_t *__restrict__ out, int64_t out_stride)
{
    __shared__ uint64_t surv[kRowsPerBlock][kSurvivorCap];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;
    if (row >= num_rows)
        return;

    int n = valid_len ? valid_len[row] : width;
    n = n < 0 ? 0 : (n > width ? width : n);
    const int fb = force_begin ? force_begin[row] : 0;
    const int fe = force_end ? force_end[row] : 0;
    const int k = append_page ? kTopk - 1 : kTopk;
    const int ap = append_page ? append_page[row] : -1;
    const float *srow = scores + row * row_stride;
    int32_t *orow = out + row * out_stride;
    const int m = n < k ? n : k;   // columns that will be selected

    if (n > 0) {
        // (1) lane maxima.
        uint64_t lmax = 0;
        int c = lane;
        for (; c + 3 * kWave < n; c += 4 * kWave) {
            const float s0 = srow[c], s1 = srow[c + kWave], s2 = srow[c + 2 * kWave],
                        s3 = srow[c + 3 * kWave];
            const uint64_t k0 = make_key(s0, c, fb, fe), k1 = make_key(s1, c + kWave, fb, fe);
            const uint64_t k2 = make_key(s2, c + 2 * kWave, fb, fe),
                           k3 = make_key(s3, c + 3 * kWave, fb, fe);
            const uint64_t a = k0 > k1 ? k0 : k1, b = k2 > k3 ? k2 : k3;
            const uint64_t mx = a > b ? a : b;
            lmax = mx > lmax ? mx : lmax;
        }
        for (; c < n; c += kWave) {
            const uint64_t kk = make_key(srow[c], c, fb, fe);
            lmax = kk > lmax ? kk : lmax;
        }
        // (2) threshold; at least 1 so that empty lanes never count.
        uint64_t thr = wave_kth_largest(lmax, k);
        thr = thr > 0 ? thr : 1;
        // (3)+(4) survivors in column order.
        int total = 0;
        for (int base = 0; base < n; base += kWave) {
            const int cc = base + lane;
            const uint64_t kk = cc < n ? make_key(srow[cc], cc, fb, fe) : 0;
            const bool s = kk >= thr;
            const uint64_t mask = __ballot(s);
            if (s) {
                const int slot = total + __popcll(mask & ((1ull << lane) - 1));
                if (slot < kSurvivorCap)
                    surv[wave][slot] = kk;
            }
            total += __popcll(mask);
        }
        if (total <= kSurvivorCap) {
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            if (lane < total) {
                const uint64_t mine = surv[wave][lane];
                int rank = 0;
                for (int i = 0; i < total; ++i)
                    rank += surv[wave][i] > mine ? 1 : 0;
                if (rank < k)
                    orow[rank] = key_col(mine);
            }
        } else {
            // (5) exact rounds.
            uint64_t prev = ~0ull;
            for (int r = 0; r < m; ++r) {
                uint64_t best = 0;
                for (int cc = lane; cc < n; cc += kWave) {
                    const uint64_t kk = make_key(srow[cc], cc, fb, fe);
                    if (kk < prev && kk > best)
                        best = kk;
                }
                best = wave_max_u64(best);
                if (lane == 0)
                    orow[r] = key_col(best);
                prev = best;
            }
        }
    }
    // Tail: the appended page right after the selected columns, then -1.
    if (lane >= m && lane < kTopk)
        orow[lane] = (lane == m && ap >= 0) ? ap : -1;
}

}  // namespace

hipError_t launch_topk16(const float *scores, int64_t row_stride, int32_t num_rows, int32_t width,
                         const int32_t *valid_len, const int32_t *force_begin,
                         const int32_t *force_end, const int32_t *append_page, int32_t *out,
                         int64_t out_stride, hipStream_t stream)
{
    const int64_t blocks = ((int64_t)num_rows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(topk16_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, scores,
                       row_stride, num_rows, width, valid_len, force_begin, force_end,
                       append_page, out, out_stride);
    return hipGetLastError();
}

}  // namespace pagescore
