// score_prefill.hip -- K3: lightning-indexer scores (Modular page
// "sparse_index_fp8_sm100", module description):
//
//   scores[t, n] = k_scale[n] * sum over heads h of relu(q[t,h] . k[n]) * q_scale[t,h]
//
// Mapping to gfx950.  v_mfma_f32_32x32x16_f16 with 32 heads of one token on
// the M side and 32 keys on the N side; the depth of 128 is eight chained K
// steps of 16.  In the 32x32 output a lane holds 16 rows of one column, i.e.
// 16 heads of one (token, key) pair, so relu, the q_scale multiply and most of
// the head sum stay in registers; one cross-lane add joins the two 16-row
// halves.  Every (token, key) score is owned by one wave: nothing is reduced
// across waves or work-groups (the independence the Mojo kernel's design also
// rests on).
//
// Operands are converted from E4M3 to f16 (exact, v_cvt_scalef32_pk_f16_fp8):
// the f16 MFMA sums the exact products with f32 accuracy, which the fp8 MFMA
// does not (its internal sum keeps about 12 bits below the largest product).
// A work-group owns a few tokens, converts their query rows once into LDS and
// streams the keys: each wave takes 32-key tiles, converts them into its B
// registers, and runs every token of the group against them.
#include "device_common.hpp"
#include "launch.hpp"

namespace pagescore {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kWavesPerBlock = 4;
constexpr int kKeysPerTile = 32;
constexpr int kRowHalves = kDepth + 8;   // f16 per LDS query row (padded: 272 bytes)
constexpr int kLdsBytes = 64 * 1024;

__device__ __forceinline__ u32x4 f16_of_8_bytes(uint32_t lo, uint32_t hi)
{
    return u32x4{f16x2_of_e4m3<false>(lo), f16x2_of_e4m3<true>(lo), f16x2_of_e4m3<false>(hi),
                 f16x2_of_e4m3<true>(hi)};
}

__global__ __launch_bounds__(256) void score_prefill_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ q_scale,
    const uint8_t *__restrict__ k, const float *__restrict__ k_scale, int32_t T, int32_t H,
    int32_t N, int32_t tokens_per_block, float *__restrict__ scores, int64_t ld)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int col = lane & 31;          // key of the tile / head row of the A tile
    const int half = lane >> 5;         // 8-element depth slice within a K step of 16
    const int hp = (H + 31) & ~31;      // heads padded to whole M tiles
    const int head_tiles = hp / 32;
    const int64_t t0 = (int64_t)blockIdx.x * tokens_per_block;
    const int tb = (int)((T - t0) < tokens_per_block ? (T - t0) : tokens_per_block);

    _Float16 *qh = reinterpret_cast<_Float16 *>(smem);                    // [tb][hp][kRowHalves]
    float *qsl = reinterpret_cast<float *>(smem + (size_t)tokens_per_block * hp * kRowHalves * 2);

    // Query rows of the group's tokens as f16 (padding heads are zero), and their scales.
    const int rows = tb * hp;
    for (int i = tid; i < rows * (kDepth / 8); i += blockDim.x) {
        const int r = i / (kDepth / 8), c8 = i % (kDepth / 8);
        const int tt = r / hp, h = r % hp;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (h < H) {
            const uint2 b = *reinterpret_cast<const uint2 *>(q + ((t0 + tt) * H + h) * kDepth + 8 * c8);
            v = f16_of_8_bytes(b.x, b.y);
        }
        *reinterpret_cast<u32x4 *>(qh + (size_t)r * kRowHalves + 8 * c8) = v;
    }
    for (int i = tid; i < rows; i += blockDim.x) {
        const int tt = i / hp, h = i % hp;
        qsl[i] = h < H ? q_scale[(t0 + tt) * H + h] : 0.0f;
    }
    __syncthreads();

    const int num_tiles = (N + kKeysPerTile - 1) / kKeysPerTile;
    for (int tile = wave; tile < num_tiles; tile += kWavesPerBlock) {
        const int64_t n = (int64_t)tile * kKeysPerTile + col;
        const bool key_ok = n < N;
        // B operand: key n, depth [16 s + 8 half, +8) for step s = 0..7.
        u32x4 kb[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            uint2 b = make_uint2(0u, 0u);
            if (key_ok)
                b = *reinterpret_cast<const uint2 *>(k + n * kDepth + 16 * s + 8 * half);
            kb[s] = f16_of_8_bytes(b.x, b.y);
        }
        const float ks = key_ok ? k_scale[n] : 0.0f;

        for (int tt = 0; tt < tb; ++tt) {
            float sum = 0.0f;
            for (int ht = 0; ht < head_tiles; ++ht) {
                const _Float16 *arow = qh + ((size_t)tt * hp + 32 * ht + col) * kRowHalves + 8 * half;
                v16f acc = {};
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(arow + 16 * s);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                                __builtin_bit_cast(v8h, kb[s]),
                                                                acc, 0, 0, 0);
                }
                // Lane holds rows 8*(i/4) + 4*half + i%4 (i = 0..15) of its key column.
                // The sum runs on x + |x| = 2 relu(x), one add and one fma per
                // element; scaling by 2 commutes with every rounding, so half
                // of it at the end equals the sum of relu(x) * q_scale.
                const float *qs = qsl + (size_t)tt * hp + 32 * ht + 4 * half;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float x = acc[i];
                    sum = fmaf(x + fabsf(x), qs[8 * (i / 4) + (i % 4)], sum);
                }
            }
            sum += __shfl_xor(sum, 32);
            if (half == 0 && key_ok)
                scores[(t0 + tt) * ld + n] = ks * (0.5f * sum);
        }
    }
}

}  // namespace

static_assert(kPrefillMaxHeads * ((kRowHalves * 2) + 4) <= kLdsBytes,
              "one token of the largest head count must fit the work-group's LDS");

hipError_t launch_score_prefill(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                const float *k_scale, int32_t T, int32_t H, int32_t N,
                                float *scores, int64_t ld, hipStream_t stream)
{
    const int hp = (H + 31) & ~31;
    const size_t per_token = (size_t)hp * (kRowHalves * 2 + 4);
    int tb = (int)(kLdsBytes / per_token);
    if (tb < 1)
        return hipErrorInvalidValue;
    if (tb > 4)
        tb = 4;
    const int64_t blocks = ((int64_t)T + tb - 1) / tb;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const size_t lds = (size_t)tb * per_token;
    hipLaunchKernelGGL(score_prefill_kernel, dim3((uint32_t)blocks), dim3(256), lds, stream, q,
                       q_scale, k, k_scale, T, H, N, tb, scores, ld);
    return hipGetLastError();
}

}  // namespace pagescore
