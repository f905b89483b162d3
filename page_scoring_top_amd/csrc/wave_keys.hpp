// wave_keys.hpp -- 64-bit selection keys and wave-wide sorting helpers shared
// by the top-16 kernels (topk16.hip) and the fused prefill selection
// (score_prefill.hip).
//
// Key order (GitHub pull request wolfcomos/MSA #1, "Changes" and "Behaviour
// changes"): score descending with forced columns as +inf, NaN as -inf and -0
// as +0, then the lower column.  Every candidate gets a distinct 64-bit key:
// the order-preserving image of its canonical score bits in the high word
// and 0xFFFFFFFF - column in the low word, so a larger key is a better
// candidate and no two keys tie.  Real keys are never 0, which marks an
// empty slot.
#pragma once

#include "device_common.hpp"

namespace pagescore {

namespace {

// Order-preserving image of the canonical score (never 0).  Adding +0
// turns -0 into +0 and quiets a NaN, and the IEEE maximum with -inf then
// returns -inf for a NaN and the value itself otherwise; a forced column is
// +inf.  The map sets the sign bit of a positive value and flips every bit
// of a negative one.
__device__ __forceinline__ uint32_t key_hi(float s, bool forced)
{
    const float c = __builtin_fmaxf(s + 0.0f, -__builtin_huge_valf());
    const uint32_t u = forced ? 0x7F800000u : __float_as_uint(c);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(uint32_t hi, int col)
{
    return ((uint64_t)hi << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)col);
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

// Number of lanes set in a ballot, as a 32-bit count (keeps the comparisons
// that follow on the scalar unit).
__device__ __forceinline__ int lanes_set(uint64_t mask)
{
    return __builtin_popcount((uint32_t)mask) + __builtin_popcount((uint32_t)(mask >> 32));
}


// The value of lane (lane ^ J).  J = 1, 2: quad permutes; J = 4: row shift
// left or right by 4; J = 8: row rotate by 8; J = 16, 32: the gfx950 permlane
// swaps, which hand each lane both halves of the exchange.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int lane)
{
    if constexpr (J == 1) {
        return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (J == 2) {
        return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (J == 4) {
        const uint32_t from_above = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0xF, false);  // row_shl:4
        const uint32_t from_below = __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, false);  // row_shr:4
        return (lane & 4) ? from_below : from_above;
    } else if constexpr (J == 8) {
        return __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
    } else if constexpr (J == 16) {
        const auto s = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? s[0] : s[1];
    } else {
        static_assert(J == 32, "xor distance");
        const auto s = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? s[0] : s[1];
    }
}

// One compare-exchange step of a descending bitonic sort over 64 lanes:
// merge blocks of K lanes at distance J.  The lane keeps the larger value of
// the pair when its position in the block says so, else the smaller one
// (equal values are interchangeable).
template <int K, int J, typename T>
__device__ __forceinline__ T bitonic_step(T x, int lane)
{
    T y;
    if constexpr (sizeof(T) == 4) {
        y = xor_lane<J>(x, lane);
    } else {
        const uint32_t ylo = xor_lane<J>((uint32_t)x, lane);
        const uint32_t yhi = xor_lane<J>((uint32_t)(x >> 32), lane);
        y = ((uint64_t)yhi << 32) | ylo;
    }
    const bool keep_max = ((lane & J) == 0) == ((lane & K) == 0 || K == 64);
    return ((y > x) == keep_max) ? y : x;
}

// Descending sort of one value per lane over the first N lanes (16, 32 or
// 64) of the wave: lane 0 ends with the largest.  The lanes past N end in
// some other order.
template <int N, typename T>
__device__ __forceinline__ T wave_sort_desc(T x, int lane)
{
    static_assert(N == 16 || N == 32 || N == 64, "sort width");
    x = bitonic_step<2, 1>(x, lane);
    x = bitonic_step<4, 2>(x, lane);
    x = bitonic_step<4, 1>(x, lane);
    x = bitonic_step<8, 4>(x, lane);
    x = bitonic_step<8, 2>(x, lane);
    x = bitonic_step<8, 1>(x, lane);
    x = bitonic_step<16, 8>(x, lane);
    x = bitonic_step<16, 4>(x, lane);
    x = bitonic_step<16, 2>(x, lane);
    x = bitonic_step<16, 1>(x, lane);
    if constexpr (N >= 32) {
        x = bitonic_step<32, 16>(x, lane);
        x = bitonic_step<32, 8>(x, lane);
        x = bitonic_step<32, 4>(x, lane);
        x = bitonic_step<32, 2>(x, lane);
        x = bitonic_step<32, 1>(x, lane);
    }
    if constexpr (N == 64) {
        x = bitonic_step<64, 32>(x, lane);
        x = bitonic_step<64, 16>(x, lane);
        x = bitonic_step<64, 8>(x, lane);
        x = bitonic_step<64, 4>(x, lane);
        x = bitonic_step<64, 2>(x, lane);
        x = bitonic_step<64, 1>(x, lane);
    }
    return x;
}

// Exclusive prefix sum of x over the lanes below (DPP row shifts within
// each row of 16, then the rows' totals via the permlane swaps).
__device__ __forceinline__ int wave_prefix_sum(int x, int lane)
{
    int v = x;   // inclusive sum within the row
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
        const int y = d == 1 ? __builtin_amdgcn_mov_dpp(v, 0x111, 0xF, 0xF, true)     // row_shr:1
                    : d == 2 ? __builtin_amdgcn_mov_dpp(v, 0x112, 0xF, 0xF, true)     // row_shr:2
                    : d == 4 ? __builtin_amdgcn_mov_dpp(v, 0x114, 0xF, 0xF, true)     // row_shr:4
                             : __builtin_amdgcn_mov_dpp(v, 0x118, 0xF, 0xF, true);    // row_shr:8
        v += (lane & 15) >= d ? y : 0;
    }
    // Row totals: lane 15 of each row.
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    const int below_rows = (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
    return v - x + below_rows;
}

}  // namespace

}  // namespace pagescore
