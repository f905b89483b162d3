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
//
// Two kernels.  Up to 64 heads (the indexer's shape) a wave keeps its
// tokens' query rows in registers and streams keys through LDS, with the
// epilogue of each key tile interleaved into the next tile's MFMAs: one
// token per wave, or up to four heads of 8 or 16 tokens packed into the
// MFMA rows (the module description packs (token, head) pairs the same way,
// on the other operand).  The same per-unit code runs the ragged causal batch
// of indexer_score_prefill_ragged, either one unit per work-group of a grid
// or, for up to 256 sequences with one token per wave, as a balanced
// schedule: one work-group per compute unit, each taking an equal share of
// the batch's estimated cost (causal_share.hpp).  It also runs the first pass of the fused top-16
// (indexer_prefill_topk16), keeping per-block records instead of storing
// scores; the second pass, prefill_topk_rescore_kernel, selects from them
// (see the section near the end).  More heads take the general kernel: a
// work-group converts a few tokens' query rows once into LDS, and each wave
// takes 32-key tiles, converts them into its B registers and runs every
// token of the group against them.
#include "device_common.hpp"
#include "causal_share.hpp"
#include "launch.hpp"
#include "wave_keys.hpp"

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
// Heads <= 64: a wave's query rows and scales in registers, keys streamed
// through LDS, the epilogue of one key tile run between the MFMAs of the
// next.
//
// A wave holds its token's query rows as f16 A operands (kHT = 1 or 2
// 32-head tiles x eight 16-deep K steps = 32 kHT VGPRs) and the q_scale of
// the heads its accumulator lanes hold (16 kHT VGPRs); up to 32 heads take
// one tile and half the MFMAs of 64.  The work-group's eight waves (two
// per SIMD) convert the keys to f16 together, 128 keys at a time, into three
// rotating LDS buffers; one barrier per 128 keys.  Rows of the key buffer
// are padded to 272 bytes so the 32 keys a B read touches fall on distinct
// banks.
//
// The epilogue ((x + |x|) * q_scale summed over the heads, two VALU per
// element) is independent of the next tile's MFMAs, so the two are
// interleaved in one instruction stream, a few VALU after each MFMA: the
// SIMD issues them while the matrix core executes, instead of after it.
// Every load and store of the loop is a buffer access against a descriptor
// that bounds it (keys past the range read as zero, scores past it are
// dropped), so the loop body has no branches and the interleaving spans
// whole chunks.
// ---------------------------------------------------------------------------

// Ragged causal batch description (unused by the dense launch).
struct RaggedBatch {
    const int32_t *q_start;   // [num_seqs + 1]
    const int32_t *k_start;   // [num_seqs]
    const int32_t *k_len;     // [num_seqs]
    int32_t *row_len;         // [T] or null
    int32_t width;            // score columns per row
};

// Sequence s of a ragged batch cut to the buffers: query rows
// [row0, row0 + q_len) of [0, T) and keys [k0, k0 + klen) of [0, N) (a key
// slice leaving the buffer keeps the part inside it; one starting outside
// it has no keys).
struct SeqSlice {
    int32_t row0, q_len, k0, klen;
};

// The slice of a sequence whose batch entries are q_start = qa, qb (its
// own and the next), k_start = k0 and k_len = kl.
__device__ __forceinline__ SeqSlice slice_of(int32_t qa, int32_t qb, int32_t k0, int32_t kl, int32_t T,
                                             int32_t N)
{
    int64_t a0 = qa, a1 = qb;
    a0 = a0 < 0 ? 0 : (a0 > T ? T : a0);
    a1 = a1 < a0 ? a0 : (a1 > T ? T : a1);
    const bool inside = k0 >= 0 && k0 <= N;
    const int64_t room = (int64_t)N - k0;
    const int64_t n = !inside ? 0 : (kl > room ? room : (kl < 0 ? 0 : kl));
    return SeqSlice{(int32_t)a0, (int32_t)(a1 - a0), inside ? k0 : 0, (int32_t)n};
}

__device__ __forceinline__ SeqSlice seq_slice(const RaggedBatch &rb, int s, int32_t T, int32_t N)
{
    return slice_of(rb.q_start[s], rb.q_start[s + 1], rb.k_start[s], rb.k_len[s], T, N);
}

constexpr int kH64Waves = 8;                                  // waves per work-group
constexpr int kChunkKeys = 128;
constexpr int kChunkBufs = 3;
constexpr int kTilesPerChunk = kChunkKeys / kKeysPerTile;     // 4
constexpr int kKeyRowBytes = kRowHalves * 2;                  // 272
constexpr int kSmallHeads = 64;
constexpr int kMaxKeysPerGroup = 1 << 20;                     // keeps descriptor sizes in 32 bits
constexpr uint32_t kDropped = 0x80000000u;                    // an offset past every descriptor
constexpr uint32_t kKeyDropped = 0x40000000u;                 // added to a row offset: past it too
constexpr int kPackHeads = 4;                                 // heads per token, packed
// Cache policy of the packed path's score stores: nontemporal (the "nt"
// bit).  Its 16 score rows per wave are written at four bytes per key and
// never read back by the kernel; measured 11% faster than default stores
// at 2,048 tokens x 65,536 keys.
constexpr int kStreamingStore = 2;
constexpr int64_t kPackMaxLd = 1 << 24;                       // 16 rows of scores <= 2^30 bytes
// Block-maximum mode (the first pass of the fused top-16): a block is one
// lane's column of 32 consecutive key tiles, i.e. the 32 keys
// 1024 j + c + 32 i (i = 0..31) of block 32 j + c, so a row of N keys has
// 32 ceil(N / 1024) blocks and a lane keeps its block's record in three
// registers: the largest score, the tile i where it first occurs, and the
// second largest (the largest again on a tie).
constexpr int kBlockTiles = 32;
constexpr int kBlockKeys = kBlockTiles * kKeysPerTile;        // 1,024


// kPack: up to four heads, a wave takes 8 kHT tokens and row 4 u + h of its
// A tile ht is head h of token 8 ht + u.  In the accumulator, element i of
// tile ht is then head i % 4 of token 8 ht + 2 (i / 4) + half, so the head
// sum of a (token, key) score is four elements of one lane, and a lane
// stores 4 kHT scores per tile.
// kCausal: a ragged batch of sequences (sl), each query row masked
// causally and its row filled with -inf past its visible keys.  Sequence s
// owns query rows [q_start[s], q_start[s+1]) and keys k_start[s] ..
// + k_len[s]; its queries are the last q_len tokens of its context, so
// query i sees count(i) = clamp(k_len - q_len + i + 1, 0, min(k_len, width))
// keys.  Score columns are relative to the sequence's first key; a
// work-group computes only the key chunks some of its queries see and fills
// the rest of its column range with -inf.
typedef uint8_t KeyChunks[kChunkBufs][kChunkKeys * kKeyRowBytes];
typedef float KeyScales[kChunkBufs][kChunkKeys];

// One unit of work-group work: the queries [tb, tb + kTokPerGroup) of
// sequence sl (the whole batch when not causal) against columns [kb, ke)
// (ke clamped to the row width); first_split: the unit holding column 0
// writes row_len.  kbuf / ks_lds: the work-group's LDS key chunks.  Every
// thread of the work-group calls it with the same arguments.
// kBlockMax (dense only): instead of the scores, `scores` receives the
// block records, three planes of T rows of ld blocks: the largest score,
// the second largest and (as int32) the tile of the largest, ranked as the
// key order ranks (-0 as +0, NaN lowest: a block of NaN scores records
// -inf); keys past the range count as NaN.  The work-group's first key kb must then be a
// multiple of kBlockKeys.
template <int kHT, bool kPack, bool kCausal, bool kBlockMax = false>
__device__ __forceinline__ void prefill_unit(
    KeyChunks &kbuf, KeyScales &ks_lds, const uint8_t *__restrict__ q,
    const float *__restrict__ q_scale, const uint8_t *__restrict__ k,
    const float *__restrict__ k_scale, int32_t T, int32_t H, int32_t N,
    float *__restrict__ scores, int64_t ld, const RaggedBatch &rb, const SeqSlice &sl, int tb, int kb,
    int64_t ke_in, bool first_split)
{
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int col = lane & 31;
    const int half = lane >> 5;
    constexpr int kTokPerWave = kPack ? 8 * kHT : 1;
    constexpr int kTokPerGroup = kH64Waves * kTokPerWave;
    // Query rows [row0, row_end) and keys [0, klen) of k / k_scale from here
    // on; the work-group's tokens start at row0 + tb and its columns are
    // [kb, ke), of which [kb, kc) are computed.
    int64_t row0 = 0, row_end = T;
    int32_t klen = N, width = N;
    if constexpr (kCausal) {
        row0 = __builtin_amdgcn_readfirstlane(sl.row0);
        row_end = row0 + __builtin_amdgcn_readfirstlane(sl.q_len);
        klen = __builtin_amdgcn_readfirstlane(sl.klen);
        width = rb.width;
        const int64_t k0 = __builtin_amdgcn_readfirstlane(sl.k0);
        k += k0 * kDepth;
        k_scale += k0;
    }
    const int q_len = (int)(row_end - row0);
    if (tb >= q_len)
        return;
    const int iw = tb + wave * kTokPerWave;                 // the wave's first query of the sequence
    const int64_t t = row0 + iw;
    const int tok_rows = iw >= q_len ? 0 : (q_len - iw < kTokPerWave ? q_len - iw : kTokPerWave);
    const bool tok_ok = tok_rows > 0;
    const int ke = (int)(ke_in < width ? ke_in : width);
    // Visible keys of query i of the sequence (all of them without the mask).
    auto visible = [&](int i) {
        if constexpr (!kCausal)
            return klen;
        const int64_t c = (int64_t)klen - q_len + i + 1;
        const int hi = klen < width ? klen : width;
        return (int)(c > hi ? hi : (c < 0 ? 0 : c));
    };
    int kc = ke;
    if constexpr (kCausal) {
        const int last = tb + kTokPerGroup < q_len ? tb + kTokPerGroup - 1 : q_len - 1;
        const int cmax = visible(last);
        kc = cmax < kb ? kb : (cmax < ke ? cmax : ke);
        if (first_split && rb.row_len != nullptr && lane < tok_rows)
            rb.row_len[t + lane] = visible(iw + lane);
    }
    const int chunks = (kc - kb + kChunkKeys - 1) / kChunkKeys;

    // Key conversion: thread -> key tid / 4 of the chunk, 32 depth bytes at
    // 32 (tid % 4): two 16-byte loads, then four pieces of four conversions
    // and one 16-byte LDS store each.
    const int ck = tid >> 2, cd = (tid & 3) * 32;
    struct Raw {
        u32x4 v[2];
        float ks;
    };
    auto load_chunk = [&](int c, Raw &r) {
        // Keys [kb + 128 c, kc): a chunk past the range has no records.
        const int base = kb + c * kChunkKeys;
        const int live = c < chunks ? (kc - base < kChunkKeys ? kc - base : kChunkKeys) : 0;
        const __amdgpu_buffer_rsrc_t kr = uniform_rsrc(k + (int64_t)(c < chunks ? base : 0) * kDepth,
                                                       (uint32_t)live * kDepth);
        const __amdgpu_buffer_rsrc_t sr = uniform_rsrc(k_scale + (c < chunks ? base : 0),
                                                       (uint32_t)live * 4);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, ck * kDepth + cd + 16 * i, 0, 0);
        r.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, 4 * ck, 0, 0));
        if constexpr (kBlockMax)
            r.ks = ck < live ? r.ks : __builtin_nanf("");
    };
    // Piece j (0..3) of a chunk's conversion; piece 3 also stores the key
    // scale (the key's four threads store the same value).
    auto store_piece = [&](const Raw &r, int buf, int j) {
        uint8_t *dst = &kbuf[buf][ck * kKeyRowBytes + cd * 2 + 16 * j];
        const u32x4 &v = r.v[j / 2];
        *reinterpret_cast<u32x4 *>(dst) = f16_of_8_bytes(v[2 * (j % 2)], v[2 * (j % 2) + 1]);
        if (j == 3)
            ks_lds[buf][ck] = r.ks;
    };

    // Every load the unit starts with -- its query rows, their scales and
    // the first two key chunks -- is issued before any of them is used, so
    // the unit waits for memory once.
    // Query rows as f16 A operands: head 32 ht + col, depth 16 st + 8 half
    // .. +8 (zero past H, and for a token past T); kHT head tiles of 32.
    // The rows and their scales are read through descriptors spanning the
    // wave's tokens, so a lane outside them reads zero without a branch.
    const int64_t row_q = tok_ok ? t : 0;
    const __amdgpu_buffer_rsrc_t qr =
        uniform_rsrc(q + row_q * H * kDepth, tok_ok ? (uint32_t)(tok_rows * H * kDepth) : 0u);
    const __amdgpu_buffer_rsrc_t qsr = uniform_rsrc(q_scale + row_q * H, tok_ok ? (uint32_t)(tok_rows * H * 4) : 0u);
    uint2 q_raw[kHT][8];
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht) {
        const int h = kPack ? col % 4 : 32 * ht + col;
        const int u = kPack ? 8 * ht + col / 4 : 0;
        const uint32_t off = (u < tok_rows && h < H) ? (uint32_t)((u * H + h) * kDepth + 8 * half) : kDropped;
#pragma unroll
        for (int st = 0; st < 8; ++st)
            q_raw[ht][st] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(qr, off + 16 * st, 0, 0));
    }
    // Scales of the heads the lane's accumulators hold: element i of tile ht
    // is head 32 ht + 8 (i / 4) + 4 half + i % 4 (packed: head i % 4 of
    // token 8 ht + 2 (i / 4) + half).
    float qs[kHT][16];
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = kPack ? i % 4 : 32 * ht + 8 * (i / 4) + 4 * half + i % 4;
            const int u = kPack ? 8 * ht + 2 * (i / 4) + half : 0;
            const uint32_t off = (u < tok_rows && h < H) ? (uint32_t)((u * H + h) * 4) : kDropped;
            qs[ht][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qsr, off, 0, 0));
        }
    Raw r0, r1;
    load_chunk(0, r0);
    load_chunk(1, r1);
    u32x4 a[kHT][8];
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht)
#pragma unroll
        for (int st = 0; st < 8; ++st)
            a[ht][st] = f16_of_8_bytes(q_raw[ht][st].x, q_raw[ht][st].y);

    // Scores of this wave's tokens for keys [kb, ke); a wave past T has no
    // records.  Packed, the descriptor spans the wave's rows (at most 2^30
    // bytes), and a store's offset is row_off[g], the byte offset of the
    // lane's row of token 8 (g / 4) + 2 (g % 4) + half (kDropped for a token
    // past T), plus the key's offset (plus kKeyDropped for a key past ke):
    // every dropped offset lies past the records, and none wraps.
    // Block-maximum mode: the work-group's blocks start at column kb / 32.
    const int out_col0 = kBlockMax ? kb / kBlockKeys * kKeysPerTile : kb;
    const int out_cols = kBlockMax ? (ke - kb + kBlockKeys - 1) / kBlockKeys * kKeysPerTile : ke - kb;
    const uint32_t out_bytes = tok_ok ? (uint32_t)(((int64_t)(tok_rows - 1) * ld + out_cols) * 4) : 0u;
    float *const out_base = scores + (tok_ok ? t : 0) * ld + out_col0;
    const __amdgpu_buffer_rsrc_t out = uniform_rsrc(out_base, out_bytes);
    // Block-maximum mode: the second and third record planes.
    const int64_t plane = kBlockMax ? (int64_t)T * ld : 0;
    const __amdgpu_buffer_rsrc_t out2 = uniform_rsrc(out_base + plane, kBlockMax ? out_bytes : 0u);
    const __amdgpu_buffer_rsrc_t out3 = uniform_rsrc(out_base + 2 * plane, kBlockMax ? out_bytes : 0u);
    const int key_count = ke - kb;
    uint32_t row_off[kPack ? 4 * kHT : 1];
    // Causal: a store of column kb + n writes -inf unless n < vis_rel (the
    // row's visible keys relative to kb).
    int vis_rel[kPack ? 4 * kHT : 1];
    if constexpr (kPack) {
#pragma unroll
        for (int g = 0; g < 4 * kHT; ++g) {
            const int u = 8 * (g / 4) + 2 * (g % 4) + half;
            row_off[g] = u < tok_rows ? (uint32_t)(u * ld * 4) : kDropped;
            vis_rel[g] = visible(iw + u) - kb;
        }
    } else {
        vis_rel[0] = visible(iw) - kb;
    }

    // The drain of a tile's accumulators is cut into 8 kHT slices, one per
    // MFMA of the next tile.  Element e (0 .. 16 kHT - 1) is row e % 16 of
    // head tile e / 16;
    // its doubled relu y = x + |x| is formed one slice before its fma, so no
    // VALU instruction waits on the one just before it, and the fma goes to
    // partial sum e % 4 (packed: the sum of its token, e / 4).  A sum's first
    // term is a multiply.
    constexpr int kElems = 16 * kHT;
    constexpr int kParts = kPack ? 4 * kHT : 4;
    v16f acc[2][kHT];
    float y[4];
    float part[kParts];
    // Block-maximum mode: running maxima of the lane's current block, one
    // per score the lane produces per tile.
    constexpr int kRecs = kPack ? kParts : 1;
    float bm1[kRecs], bm2[kRecs];
    int bat[kRecs];
#pragma unroll
    for (int g = 0; g < kRecs; ++g) {
        bm1[g] = -__builtin_huge_valf();
        bm2[g] = -__builtin_huge_valf();
        bat[g] = 0;
    }
    // Fold score v of tile `tile` (of its block) into record g.  With
    // bm2 <= bm1, the new second largest is the median of (bm2, bm1, v)
    // (bm1 again on a tie), one v_med3_f32; the IEEE compare and maximum
    // already rank as the key order does: -0 equals +0, a NaN never wins,
    // and v_med3_f32 with a NaN operand returns the minimum of the others
    // (bm2 here).  Strict > keeps the earlier (lower) column on a tie.
    auto record = [&](int g, float v, int tile) {
        const bool gt = v > bm1[g];
        bm2[g] = __builtin_amdgcn_fmed3f(bm2[g], bm1[g], v);
        bm1[g] = __builtin_fmaxf(bm1[g], v);
        bat[g] = gt ? tile : bat[g];
    };
    auto part_of = [](int e) { return kPack ? e / 4 : e % 4; };
    auto first_of_part = [](int e) { return kPack ? e % 4 == 0 : e < 4; };
    auto add_term = [&](int e) {
        const float v = y[e % 4];
        const float w = qs[e / 16][e % 16];
        part[part_of(e)] = first_of_part(e) ? v * w : fmaf(v, w, part[part_of(e)]);
    };
    auto drain_slice = [&](const v16f (&c)[kHT], int m) {
        if (m > 0) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                add_term(2 * (m - 1) + j);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = 2 * m + j;
            const float x = c[e / 16][e % 16];
            y[e % 4] = x + fabsf(x);
        }
    };
    // The last two fmas, the head sum across the lane halves, the k_scale
    // and the store (by the first half; n_rel is the tile's first key
    // relative to kb, and a negative one drops the store).
    auto drain_tail = [&](float ks, int n_rel) {
#pragma unroll
        for (int e = kElems - 2; e < kElems; ++e)
            add_term(e);
        if constexpr (kPack) {
            const int n = n_rel + col;
            const uint32_t key_off = (n_rel >= 0 && n < key_count) ? (uint32_t)n * 4u : kKeyDropped;
            const float hks = 0.5f * ks;
#pragma unroll
            for (int g = 0; g < kParts; ++g) {
                float v = hks * part[g];
                if constexpr (kBlockMax) {
                    record(g, v, (n_rel / kKeysPerTile) % kBlockTiles);
                    continue;
                }
                if constexpr (kCausal)
                    v = n < vis_rel[g] ? v : -INFINITY;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), out, row_off[g] + key_off, 0,
                                                      kStreamingStore);
            }
            return;
        }
        const float sum = (part[0] + part[1]) + (part[2] + part[3]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum),
                                                         false, false);
        const float total = sum + __uint_as_float(sw[1]);   // lanes 0..31: the other half's sum
        const uint32_t off = (half == 0 && n_rel >= 0) ? (uint32_t)(n_rel + col) * 4u : kDropped;
        float v = ks * (0.5f * total);
        if constexpr (kBlockMax) {
            record(0, v, (n_rel / kKeysPerTile) % kBlockTiles);
            return;
        }
        if constexpr (kCausal)
            v = n_rel + col < vis_rel[0] ? v : -INFINITY;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), out, off, 0, 0);
    };
    // Block-maximum mode: store the records of the block holding the tile
    // whose first key is n_rel, and start the next block.
    auto flush_blocks = [&](int n_rel) {
        const uint32_t boff = (uint32_t)(n_rel / kBlockKeys * kKeysPerTile + col) * 4u;
#pragma unroll
        for (int g = 0; g < kRecs; ++g) {
            const uint32_t off = kPack ? row_off[g] + boff : (half == 0 ? boff : kDropped);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bm1[g]), out, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bm2[g]), out2, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)bat[g], out3, off, 0, 0);
            bm1[g] = -__builtin_huge_valf();
            bm2[g] = -__builtin_huge_valf();
            bat[g] = 0;
        }
    };

    // B operand of tile kt, K step st of the chunk in buffer buf.
    auto read_b = [&](int buf, int kt, int st) {
        return *reinterpret_cast<const u32x4 *>(
            &kbuf[buf][(kt * kKeysPerTile + col) * kKeyRowBytes + 16 * half + 32 * st]);
    };

    // Three chunk buffers: while chunk c is computed, chunk c + 1 is ready
    // (its first B operands are read during chunk c's last tile) and chunk
    // c + 2 is converted into the third.  One barrier per chunk covers both
    // hazards: chunk c + 2 visible before chunk c + 1's last tile reads it,
    // and buffer c % 3 read out before chunk c + 3 is written into it.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        store_piece(r0, 0, j);
        store_piece(r1, 1, j);
    }
    __syncthreads();

    // acc[p]: the tile being accumulated and the tile being drained swap
    // roles every tile.  The drain before the first tile stores nothing.
#pragma unroll
    for (int ht = 0; ht < kHT; ++ht)
        acc[1][ht] = v16f{};
    float ks_prev = 0.0f;
    int n_prev = -1;
    u32x4 b_carry[2] = {read_b(0, 0, 0), read_b(0, 0, 1)};
    int buf = 0;

    for (int c = 0; c < chunks; ++c) {
        const int nbuf = buf == kChunkBufs - 1 ? 0 : buf + 1;
        const int wbuf = nbuf == kChunkBufs - 1 ? 0 : nbuf + 1;
        Raw nxt;
        load_chunk(c + 2, nxt);
        // B operands in flight two K steps ahead, across tiles and chunks.
        u32x4 b[kTilesPerChunk][8];
        b[0][0] = b_carry[0];
        b[0][1] = b_carry[1];
#pragma unroll
        for (int kt = 0; kt < kTilesPerChunk; ++kt) {
            v16f (&cur)[kHT] = acc[kt & 1];
            const v16f (&prev)[kHT] = acc[(kt & 1) ^ 1];
            const float ks = ks_lds[buf][kt * kKeysPerTile + col];
#pragma unroll
            for (int st = 0; st < 8; ++st) {
#pragma unroll
                for (int ht = 0; ht < kHT; ++ht) {
                    const int m = kHT * st + ht;
                    cur[ht] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(v8h, a[ht][st]), __builtin_bit_cast(v8h, b[kt][st]),
                        st == 0 ? v16f{} : cur[ht], 0, 0, 0);
                    drain_slice(prev, m);
                    if (ht == 0) {
                        if (st + 2 < 8)
                            b[kt][st + 2] = read_b(buf, kt, st + 2);
                        else if (kt + 1 < kTilesPerChunk)
                            b[kt + 1][st - 6] = read_b(buf, kt + 1, st - 6);
                        else
                            b_carry[st - 6] = read_b(nbuf, 0, st - 6);
                    }
                    // The last tile converts chunk c + 2, one piece per
                    // K step.
                    if (kt == kTilesPerChunk - 1 && ht == kHT - 1 && st < 4)
                        store_piece(nxt, wbuf, st);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (kBlockMax) {
                // The drain before the first tile has no scores; a block
                // ends with its 32nd tile.
                if (n_prev >= 0) {
                    drain_tail(ks_prev, n_prev);
                    if ((n_prev / kKeysPerTile) % kBlockTiles == kBlockTiles - 1)
                        flush_blocks(n_prev);
                }
            } else {
                drain_tail(ks_prev, n_prev);
            }
            ks_prev = ks;
            n_prev = c * kChunkKeys + kt * kKeysPerTile;
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        buf = nbuf;
    }
    // Drain the last tile.
#pragma unroll
    for (int m = 0; m < 8 * kHT; ++m)
        drain_slice(acc[(kTilesPerChunk - 1) & 1], m);
    if constexpr (kBlockMax) {
        // The last tile's block (complete or not).
        if (n_prev >= 0) {
            drain_tail(ks_prev, n_prev);
            flush_blocks(n_prev);
        }
    } else {
        drain_tail(ks_prev, n_prev);
    }
    if constexpr (kCausal) {
        // The -inf tail past the computed chunks: columns [kb + 128 chunks, ke)
        // of the wave's rows, 16 bytes per lane from the row's first 16-byte
        // boundary on (single columns before it and after the last whole
        // quad).
        const int fill0 = chunks * kChunkKeys, fill1 = ke - kb;
        const uint32_t ninf = __float_as_uint(-INFINITY);
        const u32x4 ninf4 = {ninf, ninf, ninf, ninf};
        for (int u = 0; u < tok_rows && fill0 < fill1; ++u) {
            const uint32_t row = (uint32_t)(u * ld * 4);
            const int mis = (int)(((uintptr_t)out_base / 4 + (uintptr_t)u * ld + fill0) & 3);
            const int lead = (4 - mis) & 3;
            const int head = lead < fill1 - fill0 ? lead : fill1 - fill0;
            const int a0 = fill0 + head;
            const int quads = (fill1 - a0) >> 2;
            const int t0 = a0 + 4 * quads;
            if (lane < head)
                __builtin_amdgcn_raw_buffer_store_b32(ninf, out, row + (uint32_t)(fill0 + lane) * 4u, 0,
                                                      kStreamingStore);
            for (int qd = lane; qd < quads; qd += kWave)
                __builtin_amdgcn_raw_buffer_store_b128(ninf4, out, row + (uint32_t)(a0 + 4 * qd) * 4u, 0,
                                                       kStreamingStore);
            if (lane < fill1 - t0)
                __builtin_amdgcn_raw_buffer_store_b32(ninf, out, row + (uint32_t)(t0 + lane) * 4u, 0,
                                                      kStreamingStore);
        }
    }
}

// One unit per work-group: grid (token groups, key splits, sequences).
template <int kHT, bool kPack, bool kCausal, bool kBlockMax = false>
__global__ __launch_bounds__(kH64Waves * kWave, 2) void score_prefill_h64_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ q_scale,
    const uint8_t *__restrict__ k, const float *__restrict__ k_scale, int32_t T, int32_t H,
    int32_t N, int32_t keys_per_group, float *__restrict__ scores, int64_t ld, RaggedBatch rb)
{
    __shared__ __align__(16) KeyChunks kbuf;
    __shared__ KeyScales ks_lds;
    constexpr int kTokPerGroup = kH64Waves * (kPack ? 8 * kHT : 1);
    const int kb = blockIdx.y * keys_per_group;
    const SeqSlice sl = kCausal ? seq_slice(rb, blockIdx.z, T, N) : SeqSlice{0, T, 0, N};
    prefill_unit<kHT, kPack, kCausal, kBlockMax>(kbuf, ks_lds, q, q_scale, k, k_scale, T, H, N, scores,
                                                 ld, rb, sl, blockIdx.x * kTokPerGroup, kb,
                                                 (int64_t)kb + keys_per_group, blockIdx.y == 0);
}

// The ragged causal batch with a balanced schedule (one token per wave; the
// schedule itself is causal_share.hpp's): work-group b runs its share of the
// batch's cost line as a few segments of consecutive chunks of one query
// group, each a prefill_unit over the segment's columns (the group's last
// segment also fills its rows with -inf up to the width).  The share is
// found without walking the batch: each lane costs four sequences in closed
// form, a wave scan and a ballot give the sequence holding the share's
// start, and a binary search the group.  Every thread computes the same
// walk, so the work-group's barriers match.
template <int kHT>
__global__ __launch_bounds__(kH64Waves * kWave, 2) void score_prefill_balanced_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ q_scale,
    const uint8_t *__restrict__ k, const float *__restrict__ k_scale, int32_t T, int32_t H,
    int32_t N, int32_t num_seqs, float *__restrict__ scores, int64_t ld, RaggedBatch rb)
{
    static_assert(kCausalGroupRows == kH64Waves && kCausalChunkKeys == kChunkKeys,
                  "the schedule's groups and chunks are the unit's");
    __shared__ __align__(16) KeyChunks kbuf;
    __shared__ KeyScales ks_lds;
    const int lane = threadIdx.x % kWave;
    auto causal = [&](const SeqSlice &sl) {
        return CausalSeq{sl.q_len, sl.klen, sl.klen < rb.width ? sl.klen : rb.width};
    };
    auto uniform64 = [](int64_t v) {
        return (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v));
    };
    const int64_t fill_units = causal_fill_units(rb.width);

    // Lane l costs sequences 4 l .. 4 l + 3; an exclusive scan over the
    // lanes places them on the cost line.  Every lane loads its four
    // sequences' entries (a lane past the batch rereads the last one) before
    // any is used, so the wave waits for memory once: the empty asm
    // statements take the loaded values as they are, which keeps the
    // compiler from moving a load behind a branch.
    int32_t qa[4], qb[4], ka[4], kn[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s = 4 * lane + i < num_seqs ? 4 * lane + i : num_seqs - 1;
        qa[i] = rb.q_start[s];
        qb[i] = rb.q_start[s + 1];
        ka[i] = rb.k_start[s];
        kn[i] = rb.k_len[s];
    }
    SeqSlice mine[4];
    int64_t cost[4], lane_cost = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        asm volatile("" : "+v"(qa[i]), "+v"(qb[i]), "+v"(ka[i]), "+v"(kn[i]));
        const SeqSlice sl = slice_of(qa[i], qb[i], ka[i], kn[i], T, N);
        mine[i] = 4 * lane + i < num_seqs ? sl : SeqSlice{0, 0, 0, 0};
        const CausalSeq c = causal(mine[i]);
        cost[i] = causal_cost_before(c, causal_groups(c), fill_units);
        lane_cost += cost[i];
    }
    int64_t excl = lane_cost;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int64_t y = __shfl_up(excl, d);
        excl += lane >= d ? y : 0;
    }
    const int64_t total = uniform64(__shfl(excl, kWave - 1));
    excl -= lane_cost;
    const int64_t G = gridDim.x, b = blockIdx.x;
    const int64_t lo = total * b / G, hi = total * (b + 1) / G;
    if (lo >= hi)
        return;
    // The sequence holding cost lo (lo < total: exactly one lane has it).
    int found = -1;
    int64_t found_base = 0;
    SeqSlice found_sl{0, 0, 0, 0};
    {
        int64_t base = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (cost[i] > 0 && base <= lo && lo < base + cost[i]) {
                found = 4 * lane + i;
                found_base = base;
                found_sl = mine[i];
            }
            base += cost[i];
        }
    }
    const int src = (int)__builtin_ctzll(__ballot(found >= 0));
    const int s = __builtin_amdgcn_readlane(found, src);
    const int64_t base =
        (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)((uint64_t)found_base >> 32), src) << 32) |
                  (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)found_base, src));
    SeqSlice sl{__builtin_amdgcn_readlane(found_sl.row0, src), __builtin_amdgcn_readlane(found_sl.q_len, src),
                __builtin_amdgcn_readlane(found_sl.k0, src), __builtin_amdgcn_readlane(found_sl.klen, src)};
    const CausalSeq c = causal(sl);
    auto next = [&](int t) {
        sl = seq_slice(rb, t, T, N);
        sl.row0 = __builtin_amdgcn_readfirstlane(sl.row0);
        sl.q_len = __builtin_amdgcn_readfirstlane(sl.q_len);
        sl.k0 = __builtin_amdgcn_readfirstlane(sl.k0);
        sl.klen = __builtin_amdgcn_readfirstlane(sl.klen);
        return causal(sl);
    };
    auto unit = [&](int64_t x, int64_t ja, int64_t ke, bool first) {
        prefill_unit<kHT, false, true>(kbuf, ks_lds, q, q_scale, k, k_scale, T, H, N, scores, ld, rb, sl,
                                       (int)(x * kH64Waves), (int)(ja * kChunkKeys), ke, first);
        __syncthreads();   // the next unit rewrites the LDS chunks
    };
    causal_share_walk(lo, hi, s, num_seqs, base, c, causal_group_at(c, base, lo, fill_units), fill_units,
                      rb.width, next, unit);
}

// ---------------------------------------------------------------------------
// Fused top-16 of prefill score rows (indexer_prefill_topk16), without the
// score matrix.  Two passes:
//  1. the score kernel in block-maximum mode writes each token's block
//     records (kBlockKeys): largest score, its tile, second largest;
//  2. this kernel takes a bar every key of the best 16 reaches -- the 16th
//     largest of its lanes' maxima of the blocks' largest scores -- and
//     keeps every key scoring at least the bar: a block can hold one only if
//     its largest score reaches the bar; if its second largest does not,
//     that key is the largest, known from the record; otherwise the block's
//     keys are recomputed with the score kernel's arithmetic.  The kept keys
//     are sorted by the full key order.
// Recomputing gives the very bits the score kernel computes: the same f16
// operands in the same MFMA (each accumulator element depends only on its
// own row and column), eight K steps in the same order, and the same
// epilogue operations in the same order.
// ---------------------------------------------------------------------------
constexpr int kRescoreWaves = 4;
constexpr int kSurvCap = 256;    // survivors a token holds before compacting to its best 16
constexpr int kCandCap = 1024;   // candidate blocks listed before they are settled

// Wave maximum of a 64-bit value (butterfly over the lane distances).
template <int J>
__device__ __forceinline__ uint64_t max_with_lane_xor(uint64_t x, int lane)
{
    const uint32_t lo = xor_lane<J>((uint32_t)x, lane);
    const uint32_t hi = xor_lane<J>((uint32_t)(x >> 32), lane);
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    return y > x ? y : x;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x, int lane)
{
    x = max_with_lane_xor<1>(x, lane);
    x = max_with_lane_xor<2>(x, lane);
    x = max_with_lane_xor<4>(x, lane);
    x = max_with_lane_xor<8>(x, lane);
    x = max_with_lane_xor<16>(x, lane);
    return max_with_lane_xor<32>(x, lane);
}

// The best 16 of the first `count` (at most kSurvCap) keys of a wave's LDS
// list, descending in lanes 0..15 (0 where there are fewer).  Up to 64 keys:
// one bitonic sort; more: sixteen rounds of taking the wave's largest key.
__device__ __forceinline__ uint64_t best16_of_list(const uint64_t *list, int count, int lane)
{
    if (count <= kWave)
        return wave_sort_desc<kWave>(lane < count ? list[lane] : 0ull, lane);
    constexpr int kPer = kSurvCap / kWave;
    uint64_t v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        v[j] = lane + kWave * j < count ? list[lane + kWave * j] : 0ull;
    uint64_t res = 0;
    for (int r = 0; r < kTopk; ++r) {
        uint64_t m = v[0];
#pragma unroll
        for (int j = 1; j < kPer; ++j)
            m = v[j] > m ? v[j] : m;
        m = wave_max_u64(m, lane);
        res = lane == r ? m : res;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            v[j] = v[j] == m ? 0ull : v[j];   // keys are distinct: one lane drops it
    }
    return res;
}

// One token per wave.  kHT, kPack: the score kernel's variant (packed, the
// token sits in rows 0..3 of a one-tile group; otherwise kHT 32-head tiles).
template <int kHT, bool kPack>
__global__ __launch_bounds__(kRescoreWaves * kWave) void prefill_topk_rescore_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ q_scale,
    const uint8_t *__restrict__ k, const float *__restrict__ k_scale, int32_t T, int32_t H,
    int32_t N, const float *__restrict__ bmax, int32_t nblocks, int32_t *__restrict__ out,
    int64_t out_stride)
{
    __shared__ uint64_t surv[kRescoreWaves][kSurvCap];
    __shared__ int32_t cand[kRescoreWaves][kCandCap];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int64_t t = (int64_t)blockIdx.x * kRescoreWaves + wave;
    if (t >= T)
        return;   // no work-group barrier follows
    uint64_t *list = surv[wave];
    int32_t *cl = cand[wave];

    constexpr int kTiles = kPack ? 1 : kHT;
    u32x4 a[kTiles][8];
    float qs[kTiles][16];
#pragma unroll
    for (int ht = 0; ht < kTiles; ++ht) {
        const int h = kPack ? col % 4 : 32 * ht + col;
        const bool ok = (!kPack || col < 4) && h < H;
        const uint8_t *src = q + (t * H + (ok ? h : 0)) * kDepth + 8 * half;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            uint2 b = make_uint2(0u, 0u);
            if (ok)
                b = *reinterpret_cast<const uint2 *>(src + 16 * st);
            a[ht][st] = f16_of_8_bytes(b.x, b.y);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int hh = kPack ? i % 4 : 32 * ht + 8 * (i / 4) + 4 * half + i % 4;
            const bool mine = !kPack || (i < 4 && half == 0);
            qs[ht][i] = (mine && hh < H) ? q_scale[t * H + hh] : 0.0f;
        }
    }
    // The score of key `n` of lane col (lanes 0..31): the score kernel's
    // epilogue, term for term.
    auto score_of = [&](const uint2 (&kr)[8], float ks) __attribute__((always_inline)) {
        v16f acc[kTiles];
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const u32x4 bop = f16_of_8_bytes(kr[st].x, kr[st].y);
#pragma unroll
            for (int ht = 0; ht < kTiles; ++ht)
                acc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a[ht][st]),
                                                                 __builtin_bit_cast(v8h, bop),
                                                                 st == 0 ? v16f{} : acc[ht], 0, 0, 0);
        }
        if constexpr (kPack) {
            float part = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = acc[0][e];
                const float y = x + fabsf(x);
                part = e == 0 ? y * qs[0][e] : fmaf(y, qs[0][e], part);
            }
            const float hks = 0.5f * ks;
            return hks * part;
        } else {
            float part[4];
#pragma unroll
            for (int e = 0; e < 16 * kTiles; ++e) {
                const float x = acc[e / 16][e % 16];
                const float y = x + fabsf(x);
                part[e % 4] = e < 4 ? y * qs[e / 16][e % 16] : fmaf(y, qs[e / 16][e % 16], part[e % 4]);
            }
            const float sum = (part[0] + part[1]) + (part[2] + part[3]);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum),
                                                             false, false);
            const float total = sum + __uint_as_float(sw[1]);
            return ks * (0.5f * total);
        }
    };

    // Block records of the token: largest score, second largest, tile of the
    // largest (three planes of [T, nblocks]).
    const int64_t plane = (int64_t)T * nblocks;
    const float *m1row = bmax + t * nblocks;
    const float *m2row = m1row + plane;
    const int32_t *atrow = reinterpret_cast<const int32_t *>(m1row + 2 * plane);
    const uint32_t kNegInfHi = key_hi(-__builtin_huge_valf(), false);

    // The bar: the 16th largest of the 64 lanes' maxima of the blocks'
    // largest scores (in key order; lane l holds blocks l, l + 64, ...).
    // The 16 lanes reaching it hold 16 distinct blocks, hence 16 distinct
    // keys, scoring at least that much, so no key below it is among the
    // best 16 (a row has at least 32 blocks, so the 16 lanes are real).
    // Rows of up to kWin windows keep their largest scores in registers
    // for the candidate scan below; longer rows read them again.
    // Lane l holds blocks base + 256 w + 4 l + j (j < 4), loaded 16 bytes at
    // a time (nblocks is a multiple of 32, so a group of four is whole).
    constexpr int kWin = kTiles == 2 ? 2 : 8;
    constexpr int kStep = kWin * 4 * kWave;
    const bool one_step = nblocks <= kStep;
    uint32_t rh[kWin][4];
    uint32_t lmax = 0;   // below every key's high word
    auto load_step = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int w = 0; w < kWin; ++w) {
            const int b = base + w * 4 * kWave + 4 * lane;
            float4 v = make_float4(-__builtin_huge_valf(), 0.f, 0.f, 0.f);
            if (b < nblocks)
                v = *reinterpret_cast<const float4 *>(m1row + b);
            const bool in = b < nblocks;
            rh[w][0] = in ? key_hi(v.x, false) : 0u;
            rh[w][1] = in ? key_hi(v.y, false) : 0u;
            rh[w][2] = in ? key_hi(v.z, false) : 0u;
            rh[w][3] = in ? key_hi(v.w, false) : 0u;
        }
    };
    for (int base = 0; base < nblocks; base += kStep) {
        load_step(base);
#pragma unroll
        for (int w = 0; w < kWin; ++w)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                lmax = rh[w][j] > lmax ? rh[w][j] : lmax;
    }
    uint32_t thr = __builtin_amdgcn_readlane(wave_sort_desc<kWave>(lmax, lane), kTopk - 1);
    int count = 0;

    // Append the keys of the lanes with `keep` to the survivor list,
    // compacting it to its best 16 first if they would not fit (the bar then
    // rises to the 16th).
    auto append = [&](bool keep, uint64_t key) __attribute__((always_inline)) {
        const uint64_t km = __ballot(keep);
        const int nkeep = lanes_set(km);
        if (count + nkeep > kSurvCap) {
            wave_lds_sync();
            const uint64_t best = best16_of_list(list, count, lane);
            wave_lds_sync();
            if (lane < kTopk)
                list[lane] = best;
            const uint32_t hi16 = __builtin_amdgcn_readlane((uint32_t)(best >> 32), kTopk - 1);
            thr = hi16 > thr ? hi16 : thr;
            count = kTopk;
            wave_lds_sync();
        }
        if (keep)
            list[count + __builtin_amdgcn_mbcnt_hi((uint32_t)(km >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u))] = key;
        count += nkeep;
    };

    // Keys of candidate blocks cl[j0 .. j0 + kBatch) (lane col: the block's
    // key 1024 (b / 32) + b % 32 + 32 col; n = N past the list or the keys).
    constexpr int kBatch = 2;
    struct Batch {
        uint2 kr[kBatch][8];
        float ks[kBatch];
        int64_t n[kBatch];
    };
    auto load_batch = [&](int j0, int nc, Batch &bt) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < kBatch; ++cb) {
            const int blk = j0 + cb < nc ? cl[j0 + cb] : -1;
            const int64_t n = blk >= 0 ? (int64_t)(blk / kKeysPerTile) * kBlockKeys + blk % kKeysPerTile +
                                             (int64_t)kKeysPerTile * col
                                       : (int64_t)N;
            const bool live = n < N;
            bt.n[cb] = n;
            const uint2 *src = reinterpret_cast<const uint2 *>(k + (live ? n : 0) * kDepth + 8 * half);
#pragma unroll
            for (int st = 0; st < 8; ++st)
                bt.kr[cb][st] = live ? src[2 * st] : make_uint2(0u, 0u);
            bt.ks[cb] = live ? k_scale[n] : __builtin_nanf("");
        }
    };
    // Score a loaded batch and keep the keys that reach the bar.
    auto run_batch = [&](int j0, int nc, const Batch &bt) __attribute__((always_inline)) {
#pragma unroll
        for (int cb = 0; cb < kBatch; ++cb) {
            if (j0 + cb >= nc)
                break;
            const float v = score_of(bt.kr[cb], bt.ks[cb]);
            const uint32_t hi = key_hi(v, false);
            append(half == 0 && bt.n[cb] < N && hi >= thr, make_key(hi, (int)bt.n[cb]));
        }
    };
    // The blocks listed in cl[0, nc), two batches in flight: the next
    // batch's keys load while this one is scored.
    auto rescore = [&](int nc) __attribute__((always_inline)) {
        Batch x, y;
        load_batch(0, nc, x);
        for (int j0 = 0; j0 < nc; j0 += 2 * kBatch) {
            load_batch(j0 + kBatch, nc, y);
            run_batch(j0, nc, x);
            if (j0 + kBatch >= nc)
                break;
            load_batch(j0 + 2 * kBatch, nc, x);
            run_batch(j0 + kBatch, nc, y);
        }
    };

    // A block whose largest score reaches the bar is a candidate.  If its
    // second largest is below the bar, its only key that can count is the
    // largest, whose score and column the record gives: it joins the
    // survivors directly.  Otherwise (two or more keys at the bar, or a
    // block of -inf / NaN scores) its keys are rescored.  Candidates are
    // listed in cl and settled (their other two records read, the direct
    // ones kept, the others compacted to the front of cl and rescored)
    // when the list could overflow and at the end.
    auto settle = [&](int nc) __attribute__((always_inline)) {
        int na = 0;
        for (int g0 = 0; g0 < nc; g0 += kWave) {
            const bool in = g0 + lane < nc;
            const int b = in ? cl[g0 + lane] : 0;
            const float r1 = m1row[b], r2 = m2row[b];
            const int at = atrow[b];
            wave_lds_sync();   // cl is read before it is rewritten below
            const uint32_t h1 = key_hi(r1, false);
            const bool direct = in && h1 > kNegInfHi && key_hi(r2, false) < thr;
            const int64_t colk = (int64_t)(b / kKeysPerTile) * kBlockKeys + b % kKeysPerTile +
                                 (int64_t)kKeysPerTile * at;
            append(direct, make_key(h1, (int)colk));
            const bool again = in && !direct;
            const uint64_t mask = __ballot(again);
            if (again)
                cl[na + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u))] = b;
            na += lanes_set(mask);
            wave_lds_sync();
        }
        if (na > 0)
            rescore(na);
        wave_lds_sync();
    };
    int nc = 0;
    for (int base = 0; base < nblocks; base += kStep) {
        if (!one_step)
            load_step(base);
#pragma unroll
        for (int w = 0; w < kWin; ++w) {
            if (nc > kCandCap - 4 * kWave) {
                settle(nc);
                nc = 0;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool is_cand = rh[w][j] >= thr;   // 0 (no block) never reaches the bar
                const uint64_t mask = __ballot(is_cand);
                if (is_cand)
                    cl[nc + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u))] =
                        base + w * 4 * kWave + 4 * lane + j;
                nc += lanes_set(mask);
            }
            wave_lds_sync();
        }
    }
    if (nc > 0)
        settle(nc);
    const uint64_t best = best16_of_list(list, count, lane);
    if (lane < kTopk)
        out[t * out_stride + lane] = best != 0 ? key_col(best) : -1;
}

}  // namespace

static_assert(kPrefillMaxHeads * ((kRowHalves * 2) + 4) <= kLdsBytes,
              "one token of the largest head count must fit the work-group's LDS");

namespace {

// Launch of the small-head kernel over `token_groups` x key splits x
// `num_seqs` work-groups, with columns [0, width) split in whole chunks of
// 128 keys (at most 2^20 per work-group) so the grid holds about one
// work-group per compute unit.
// Sequences up to which a causal launch of the one-token path takes the
// balanced schedule (each lane of a work-group's waves costs four of them).
constexpr int32_t kBalancedMaxSeqs = 256;
// Work-groups a causal launch of the one-token path aims at (about four
// per compute unit) when it takes the grid instead.
constexpr int64_t kCausalTargetGroups = 1024;

template <bool kCausal>
hipError_t launch_h64(const uint8_t *q, const float *q_scale, const uint8_t *k, const float *k_scale,
                      int32_t T, int32_t H, int32_t N, float *scores, int64_t ld, int64_t max_q,
                      int32_t width, int32_t num_seqs, const RaggedBatch &rb, hipStream_t stream)
{
    // Up to four heads, 16 tokens per wave (8 for a short prefill); one
    // token per wave otherwise.  Eight waves per work-group.
    const bool pack = H <= kPackHeads && ld <= kPackMaxLd;
    // Dense work is even, so about one work-group per compute unit.  Causal
    // rows see different key counts: the one-token path oversubscribes the
    // grid four times and lets the hardware balance it (measured 11% faster
    // at 4 x 512 queries over 4K-16K keys); the packed path, whose work per
    // key is small, keeps one work-group per compute unit.
    const int64_t target_groups = (kCausal && !pack) ? kCausalTargetGroups : 256;
    const int pack_tiles = max_q > 8 * kH64Waves ? 2 : 1;
    const int64_t tokens_per_group = (int64_t)kH64Waves * (pack ? 8 * pack_tiles : 1);
    const int64_t groups = (max_q + tokens_per_group - 1) / tokens_per_group;
    if (groups > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const int64_t busy = ((int64_t)T + tokens_per_group - 1) / tokens_per_group + num_seqs - 1;
    const int64_t chunks = ((int64_t)width + kChunkKeys - 1) / kChunkKeys;
    int64_t splits = (target_groups + busy - 1) / busy;
    const int64_t min_splits = ((int64_t)width + kMaxKeysPerGroup - 1) / kMaxKeysPerGroup;
    splits = splits < min_splits ? min_splits : splits;
    splits = splits < 1 ? 1 : (splits > chunks ? chunks : splits);
    const int64_t keys_per_group = ((chunks + splits - 1) / splits) * kChunkKeys;
    splits = ((int64_t)width + keys_per_group - 1) / keys_per_group;
    if (splits > 65535)
        return hipErrorInvalidValue;
    const dim3 grid((uint32_t)groups, (uint32_t)splits, (uint32_t)num_seqs), block(kH64Waves * kWave);
    // Packed tokens up to four heads; otherwise one 32-head MFMA tile up to
    // 32 heads, two up to 64.
    if (pack && pack_tiles == 2)
        hipLaunchKernelGGL((score_prefill_h64_kernel<2, true, kCausal>), grid, block, 0, stream, q,
                           q_scale, k, k_scale, T, H, N, (int32_t)keys_per_group, scores, ld, rb);
    else if (pack)
        hipLaunchKernelGGL((score_prefill_h64_kernel<1, true, kCausal>), grid, block, 0, stream, q,
                           q_scale, k, k_scale, T, H, N, (int32_t)keys_per_group, scores, ld, rb);
    else if (H <= 32)
        hipLaunchKernelGGL((score_prefill_h64_kernel<1, false, kCausal>), grid, block, 0, stream, q,
                           q_scale, k, k_scale, T, H, N, (int32_t)keys_per_group, scores, ld, rb);
    else
        hipLaunchKernelGGL((score_prefill_h64_kernel<2, false, kCausal>), grid, block, 0, stream, q,
                           q_scale, k, k_scale, T, H, N, (int32_t)keys_per_group, scores, ld, rb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_score_prefill_ragged(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                       const float *k_scale, int32_t T, int32_t H, int32_t N,
                                       int32_t num_seqs, const int32_t *q_start,
                                       const int32_t *k_start, const int32_t *k_len, int32_t max_q,
                                       int32_t width, float *scores, int64_t ld, int32_t *row_len,
                                       int num_cus, hipStream_t stream)
{
    static_assert(kRaggedMaxHeads == kSmallHeads, "the ragged batch runs the small-head kernel only");
    if (H > kSmallHeads || num_seqs > 65535)
        return hipErrorInvalidValue;
    const RaggedBatch rb{q_start, k_start, k_len, row_len, width};
    // One token per wave over a few sequences: the balanced schedule, one
    // work-group per compute unit (the kernel's registers allow one).
    const bool pack = H <= kPackHeads && ld <= kPackMaxLd;
    if (!pack && num_seqs <= kBalancedMaxSeqs) {
        const dim3 grid((uint32_t)(num_cus > 0 ? num_cus : 256)), block(kH64Waves * kWave);
        if (H <= 32)
            hipLaunchKernelGGL(score_prefill_balanced_kernel<1>, grid, block, 0, stream, q, q_scale,
                               k, k_scale, T, H, N, num_seqs, scores, ld, rb);
        else
            hipLaunchKernelGGL(score_prefill_balanced_kernel<2>, grid, block, 0, stream, q, q_scale,
                               k, k_scale, T, H, N, num_seqs, scores, ld, rb);
        return hipGetLastError();
    }
    return launch_h64<true>(q, q_scale, k, k_scale, T, H, N, scores, ld, max_q, width, num_seqs, rb,
                            stream);
}

int64_t prefill_topk16_blocks(int32_t N)
{
    return ((int64_t)N + kBlockKeys - 1) / kBlockKeys * kKeysPerTile;
}

hipError_t launch_prefill_topk16(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                 const float *k_scale, int32_t T, int32_t H, int32_t N, int32_t *out,
                                 int64_t out_stride, float *bmax, hipStream_t stream)
{
    if (H > kSmallHeads || T < 1 || N < 1)
        return hipErrorInvalidValue;
    const int64_t nblocks = prefill_topk16_blocks(N);
    // Pass 1: block records, with the score kernel's launch shape (about one
    // work-group per compute unit), key splits in whole blocks of 1,024.
    const int64_t ld = nblocks;                              // record planes of [T, nblocks]
    const bool pack = H <= kPackHeads && ld <= kPackMaxLd;
    const int pack_tiles = T > 8 * kH64Waves ? 2 : 1;
    const int64_t tokens_per_group = (int64_t)kH64Waves * (pack ? 8 * pack_tiles : 1);
    const int64_t groups = ((int64_t)T + tokens_per_group - 1) / tokens_per_group;
    if (groups > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const int64_t block_groups = nblocks / kKeysPerTile;
    int64_t splits = (256 + groups - 1) / groups;
    const int64_t min_splits = ((int64_t)N + kMaxKeysPerGroup - 1) / kMaxKeysPerGroup;
    splits = splits < min_splits ? min_splits : splits;
    splits = splits < 1 ? 1 : (splits > block_groups ? block_groups : splits);
    const int64_t keys_per_group = ((block_groups + splits - 1) / splits) * kBlockKeys;
    splits = ((int64_t)N + keys_per_group - 1) / keys_per_group;
    if (splits > 65535)
        return hipErrorInvalidValue;
    const dim3 grid((uint32_t)groups, (uint32_t)splits, 1u), block(kH64Waves * kWave);
    const RaggedBatch none{};
    if (pack && pack_tiles == 2)
        hipLaunchKernelGGL((score_prefill_h64_kernel<2, true, false, true>), grid, block, 0, stream, q,
                           q_scale, k, k_scale, T, H, N, (int32_t)keys_per_group, bmax, ld, none);
    else if (pack)
        hipLaunchKernelGGL((score_prefill_h64_kernel<1, true, false, true>), grid, block, 0, stream, q,
                           q_scale, k, k_scale, T, H, N, (int32_t)keys_per_group, bmax, ld, none);
    else if (H <= 32)
        hipLaunchKernelGGL((score_prefill_h64_kernel<1, false, false, true>), grid, block, 0, stream, q,
                           q_scale, k, k_scale, T, H, N, (int32_t)keys_per_group, bmax, ld, none);
    else
        hipLaunchKernelGGL((score_prefill_h64_kernel<2, false, false, true>), grid, block, 0, stream, q,
                           q_scale, k, k_scale, T, H, N, (int32_t)keys_per_group, bmax, ld, none);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // Pass 2: the bar, the candidates, rescoring where needed and the exact
    // selection.
    const dim3 g3((uint32_t)(((int64_t)T + kRescoreWaves - 1) / kRescoreWaves)), b3(kRescoreWaves * kWave);
    if (pack)
        hipLaunchKernelGGL((prefill_topk_rescore_kernel<1, true>), g3, b3, 0, stream, q, q_scale, k,
                           k_scale, T, H, N, bmax, (int32_t)nblocks, out, out_stride);
    else if (H <= 32)
        hipLaunchKernelGGL((prefill_topk_rescore_kernel<1, false>), g3, b3, 0, stream, q, q_scale, k,
                           k_scale, T, H, N, bmax, (int32_t)nblocks, out, out_stride);
    else
        hipLaunchKernelGGL((prefill_topk_rescore_kernel<2, false>), g3, b3, 0, stream, q, q_scale, k,
                           k_scale, T, H, N, bmax, (int32_t)nblocks, out, out_stride);
    return hipGetLastError();
}

hipError_t launch_score_prefill(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                const float *k_scale, int32_t T, int32_t H, int32_t N,
                                float *scores, int64_t ld, hipStream_t stream)
{
    if (H <= kSmallHeads)
        return launch_h64<false>(q, q_scale, k, k_scale, T, H, N, scores, ld, T, N, 1, RaggedBatch{},
                                 stream);
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
