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

// ---------------------------------------------------------------------------
// Heads <= 64: query rows in registers, keys streamed through LDS.
//
// A wave owns two tokens and keeps their query rows as MFMA A operands in
// VGPRs for the whole key range (two 32-head tiles x eight 16-deep K steps x
// two tokens = 128 VGPRs), so each B operand read from LDS feeds four MFMAs.
// The work-group's four waves convert the keys to f16 together, 128 keys at
// a time, into one of two LDS buffers while they compute on the other; one
// barrier per 128 keys.  A work-group covers 8 tokens and a contiguous range
// of keys (the key range is split so the grid fills the chip).  Rows of the key buffer are padded to 272 bytes so
// the 32 keys a B read touches fall on distinct banks.
// ---------------------------------------------------------------------------
constexpr int kTokPerWave = 2;
constexpr int kTokPerGroup = kWavesPerBlock * kTokPerWave;   // 8
constexpr int kChunkKeys = 128;
constexpr int kKeyRowBytes = kRowHalves * 2;                  // 272
constexpr int kSmallHeads = 64;

__global__ __launch_bounds__(256, 2) void score_prefill_h64_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ q_scale,
    const uint8_t *__restrict__ k, const float *__restrict__ k_scale, int32_t T, int32_t H,
    int32_t N, int32_t keys_per_group, float *__restrict__ scores, int64_t ld)
{
    __shared__ __align__(16) uint8_t kbuf[2][kChunkKeys * kKeyRowBytes];
    __shared__ __align__(16) float qs_lds[kTokPerGroup][kSmallHeads];
    __shared__ float ks_lds[2][kChunkKeys];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t tg = (int64_t)blockIdx.x * kTokPerGroup;
    const int kb = blockIdx.y * keys_per_group;
    const int ke = kb + keys_per_group < N ? kb + keys_per_group : N;

    // Query rows of this wave's two tokens as f16 A operands: head 32 ht +
    // col, depth 16 s + 8 half .. +8 (zero past H or T).
    u32x4 a[kTokPerWave][2][8];
#pragma unroll
    for (int tk = 0; tk < kTokPerWave; ++tk) {
        const int64_t t = tg + wave * kTokPerWave + tk;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const int h = 32 * ht + col;
            const bool ok = t < T && h < H;
            const uint8_t *src = q + ((ok ? t : 0) * H + (ok ? h : 0)) * kDepth + 8 * half;
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                uint2 b = make_uint2(0u, 0u);
                if (ok)
                    b = *reinterpret_cast<const uint2 *>(src + 16 * st);
                a[tk][ht][st] = f16_of_8_bytes(b.x, b.y);
            }
        }
    }
    for (int i = tid; i < kTokPerGroup * kSmallHeads; i += blockDim.x) {
        const int tt = i / kSmallHeads, h = i % kSmallHeads;
        const int64_t t = tg + tt;
        qs_lds[tt][h] = (t < T && h < H) ? q_scale[t * H + h] : 0.0f;
    }

    // Key conversion: thread -> key tid / 2 of the chunk, depth half tid % 2
    // (64 elements: four 16-byte loads, 32 conversions, eight 16-byte
    // stores).  The loads of chunk i+1 are issued before chunk i is computed
    // and converted after it, so their latency hides behind the MFMAs.
    const int ck = tid >> 1, cd = (tid & 1) * 64;
    struct Raw {
        u32x4 v[4];
        float ks;
    };
    auto load_chunk = [&](int chunk_base, Raw &r) {
        const int n = chunk_base + ck;
        const bool ok = n < ke;
        const int64_t nn = ok ? n : kb;   // a valid key; its values are not used
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.v[i] = *reinterpret_cast<const u32x4 *>(k + nn * kDepth + cd + 16 * i);
        r.ks = k_scale[nn];
        if (!ok) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                r.v[i] = u32x4{0u, 0u, 0u, 0u};
            r.ks = 0.0f;
        }
    };
    auto store_chunk = [&](const Raw &r, int buf) {
        uint8_t *dst = &kbuf[buf][ck * kKeyRowBytes + cd * 2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<u32x4 *>(dst + 32 * i) = f16_of_8_bytes(r.v[i][0], r.v[i][1]);
            *reinterpret_cast<u32x4 *>(dst + 32 * i + 16) = f16_of_8_bytes(r.v[i][2], r.v[i][3]);
        }
        if ((tid & 1) == 0)
            ks_lds[buf][ck] = r.ks;
    };

    if (kb < ke) {
        Raw r0;
        load_chunk(kb, r0);
        store_chunk(r0, 0);
    }
    __syncthreads();

    int buf = 0;
    for (int cb = kb; cb < ke; cb += kChunkKeys, buf ^= 1) {
        const bool has_next = cb + kChunkKeys < ke;
        Raw nxt;
        if (has_next)
            load_chunk(cb + kChunkKeys, nxt);

        const uint8_t *kt_base = &kbuf[buf][0];
#pragma unroll 1
        for (int kt = 0; kt < kChunkKeys / 32; ++kt) {
            const int n = cb + kt * 32 + col;
            if (cb + kt * 32 >= ke)
                break;
            v16f acc[kTokPerWave][2];
#pragma unroll
            for (int tk = 0; tk < kTokPerWave; ++tk)
#pragma unroll
                for (int ht = 0; ht < 2; ++ht)
                    acc[tk][ht] = v16f{};
            const uint8_t *brow = kt_base + (kt * 32 + col) * kKeyRowBytes + 16 * half;
#pragma unroll
            for (int st = 0; st < 8; ++st) {
                const v8h b = __builtin_bit_cast(v8h, *reinterpret_cast<const u32x4 *>(brow + 32 * st));
#pragma unroll
                for (int tk = 0; tk < kTokPerWave; ++tk)
#pragma unroll
                    for (int ht = 0; ht < 2; ++ht)
                        acc[tk][ht] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(v8h, a[tk][ht][st]), b, acc[tk][ht], 0, 0, 0);
            }
            const float ks = ks_lds[buf][kt * 32 + col];
#pragma unroll
            for (int tk = 0; tk < kTokPerWave; ++tk) {
                const int tt = wave * kTokPerWave + tk;
                float sum = 0.0f;
#pragma unroll
                for (int ht = 0; ht < 2; ++ht) {
                    // Lane holds heads 32 ht + 8 (i/4) + 4 half + i%4, i = 0..15.
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 qs4 = *reinterpret_cast<const float4 *>(
                            &qs_lds[tt][32 * ht + 8 * g + 4 * half]);
                        const float qv[4] = {qs4.x, qs4.y, qs4.z, qs4.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float x = acc[tk][ht][4 * g + r];
                            sum = fmaf(x + fabsf(x), qv[r], sum);
                        }
                    }
                }
                sum += __shfl_xor(sum, 32);
                const int64_t t = tg + tt;
                if (half == 0 && n < ke && t < T)
                    scores[t * ld + n] = ks * (0.5f * sum);
            }
        }
        // The other buffer's readers finished before the previous barrier.
        if (has_next)
            store_chunk(nxt, buf ^ 1);
        __syncthreads();
    }
}

}  // namespace

static_assert(kPrefillMaxHeads * ((kRowHalves * 2) + 4) <= kLdsBytes,
              "one token of the largest head count must fit the work-group's LDS");

hipError_t launch_score_prefill(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                const float *k_scale, int32_t T, int32_t H, int32_t N,
                                float *scores, int64_t ld, hipStream_t stream)
{
    if (H <= kSmallHeads) {
        // Token groups of 8; the keys are split so that the grid holds about
        // two work-groups per compute unit, in whole chunks of 128 keys.
        const int64_t groups = ((int64_t)T + kTokPerGroup - 1) / kTokPerGroup;
        if (groups > 0x7FFFFFFF)
            return hipErrorInvalidValue;
        const int64_t chunks = ((int64_t)N + kChunkKeys - 1) / kChunkKeys;
        int64_t splits = (512 + groups - 1) / groups;
        splits = splits < 1 ? 1 : (splits > chunks ? chunks : splits);
        const int64_t keys_per_group = ((chunks + splits - 1) / splits) * kChunkKeys;
        splits = ((int64_t)N + keys_per_group - 1) / keys_per_group;
        hipLaunchKernelGGL(score_prefill_h64_kernel, dim3((uint32_t)groups, (uint32_t)splits),
                           dim3(256), 0, stream, q, q_scale, k, k_scale, T, H, N,
                           (int32_t)keys_per_group, scores, ld);
        return hipGetLastError();
    }
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
