// score_decode.hip -- K2: fused NVFP4 dequantization + decode page scores.
//
// Semantics (vLLM API page "indexer_nvfp4_decode_cp": module description for
// the Q8KV4 scorer contract, Nvfp4DecodeCPPlan for the [B, 8*H, W] score
// layout with row = slot*H + head, _local_topk_push_kernel for a query's own
// page; Modular page "sparse_index_fp8_sm100" for relu(q.k)*q_scale; vLLM API
// page "gather_nvfp4_index_k" for the key values):
//
//   scores[b, row, j] = max over tokens t of page j of relu(q[b,row] . k[t]) * q_scale[b,row]
//
// stored for pages j below the row's own page.  The page maximum is taken on
// the raw dot products and relu and q_scale are applied once per page: for
// q_scale >= 0 both are monotone, so this equals the maximum of the products.
//
// Mapping to gfx950.  The request's 32 query rows (8 slots x 4 heads) are the
// N side of v_mfma_f32_16x16x32_f16 (two 16-row halves held in registers for
// the whole request); a page's 128 tokens are eight 16-token M tiles; the
// depth of 128 is four chained K steps of 32.  Lane l = (m = l%16, g = l/16)
// owns token 16*tile + m, depth chunk g (32 elements = 16 code bytes + 2 scale
// bytes): per code word (8 elements, one K step), two v_perm_b32 lookups in
// the scale's table give the E4M3 magnitudes of the even and odd elements,
// the code sign bits are OR-ed in, and four v_cvt_scalef32_pk_f16_fp8 turn
// the bytes into the f16 pairs (0,2) (4,6) (1,3) (5,7).  The query rows are
// converted to f16 in the same depth order when a request is loaded; a dot
// product does not depend on the order of the depth index as long as both
// operands use the same one.
//
// Why f16 and not the fp8 MFMA: every E4M3 value is exact in f16, so both
// operands are the exact key and query values.  The f16 MFMA sums the exact
// products with f32 accuracy, while the fp8 MFMA's internal sum keeps only
// about 12 bits below its largest product (measured on this GPU), which is an
// error of order 1e-4 relative on these dot products.
//
// Each output lane of a 16x16 tile holds 4 tokens of one query row, so the
// page maximum is a running per-lane max over the 8 tiles, then 2 cross-lane
// steps.  The kernel is persistent: the (request, page) pairs of the batch are
// flattened and every wave takes one contiguous range, so ragged batches
// balance; a wave prefetches the next page's 9 KiB while it scores the
// current one.  Page ids come from a per-lane cache of the next 64
// block-table entries.
//
// NaN: the MFMA's NaN handling is not relied on.  A NaN scale byte makes every
// dot of its token NaN, so it marks the whole page NaN; a NaN byte in a query
// row marks the row NaN.  Both are tracked as flags and applied at the store.
#include "device_common.hpp"
#include "launch.hpp"

namespace pagescore {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kWavesPerBlock = 4;

struct PageRegs {
    u32x4 codes[8];   // per tile: 16 code bytes of token 16*tile + m, chunk g
    uint32_t sc[8];   // per tile: the 2 scale bytes of that chunk
};

__device__ __forceinline__ void fetch_page(PageRegs &p, const uint8_t *src, int m, int g)
{
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int tok = 16 * t + m;
        p.codes[t] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(src + tok * 64 + 16 * g));
        p.sc[t] = *reinterpret_cast<const uint16_t *>(src + kCodeBytes + tok * 8 + 2 * g);
    }
}

// E4M3 bytes [0,2,4,6] and [1,3,5,7] of a word -> the four f16 pairs (0,2) (4,6) (1,3) (5,7).
__device__ __forceinline__ u32x4 f16_word(uint32_t even, uint32_t odd)
{
    return u32x4{f16x2_of_e4m3<false>(even), f16x2_of_e4m3<true>(even),
                 f16x2_of_e4m3<false>(odd), f16x2_of_e4m3<true>(odd)};
}

// One 8-element query group (bytes q[0..7] in lo, hi) -> f16 pairs in the
// order the key words use.
__device__ __forceinline__ u32x4 q_word_f16(uint32_t lo, uint32_t hi)
{
    return f16_word(byte_perm(hi, lo, 0x06040200u), byte_perm(hi, lo, 0x07050301u));
}

__device__ __forceinline__ bool has_nan_byte(uint32_t w)
{
    // A byte is NaN iff its low 7 bits are all ones.
    const uint32_t x = w & 0x7F7F7F7Fu;
    return ((x + 0x01010101u) & 0x80808080u) != 0;
}

__device__ __forceinline__ int decode_own(int32_t seq, int32_t qlen, int slot)
{
    const int i = slot - (kSlots - qlen);
    if (i < 0)
        return -1;
    const int64_t pos = (int64_t)seq - qlen + i;
    return pos < 0 ? -1 : (int)(pos / kPageTokens);
}

__device__ __forceinline__ int32_t pages_scored(int32_t seq, int32_t width)
{
    const int32_t n = seq >= 1 ? (seq - 1) / kPageTokens : 0;
    return n < width ? n : width;
}

struct RequestRegs {
    u32x4 qa[4], qb[4];  // B operands (f16): query rows m and 16+m, chunk g, per code word
    int own;          // lanes 0..31: own page of row `lane`
    float qs;         // lanes 0..31: q_scale of row `lane`
    bool qnan;        // lanes 0..31: row `lane` has a NaN query byte
};

__device__ __forceinline__ void load_request(RequestRegs &rq, const uint8_t *__restrict__ q,
                                             const float *__restrict__ q_scale,
                                             const int32_t *__restrict__ seq_lens, int32_t qlen,
                                             int b, int lane, int m, int g)
{
    const int32_t seq = seq_lens[b];
    bool nan_half[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int row = 16 * hf + m;
        const int slot = row / kDecodeHeads;
        u32x4 *dst = hf == 0 ? rq.qa : rq.qb;
        bool nan = false;
        if (slot >= kSlots - qlen) {
            const uint4 *src =
                reinterpret_cast<const uint4 *>(q + ((int64_t)b * kDecodeRows + row) * kDepth + 32 * g);
            const uint4 u0 = src[0], u1 = src[1];
            const uint32_t raw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                dst[k] = q_word_f16(raw[2 * k], raw[2 * k + 1]);
                nan |= has_nan_byte(raw[2 * k]) | has_nan_byte(raw[2 * k + 1]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                dst[k] = u32x4{0u, 0u, 0u, 0u};
        }
        // A row is NaN when any of its four depth chunks (lanes m, m+16, m+32, m+48) is.
        int f = nan ? 1 : 0;
        f |= __shfl_xor(f, 16);
        f |= __shfl_xor(f, 32);
        nan_half[hf] = f != 0;
    }
    if (lane < kDecodeRows) {
        rq.own = decode_own(seq, qlen, lane / kDecodeHeads);
        rq.qs = rq.own >= 0 ? q_scale[(int64_t)b * kDecodeRows + lane] : 0.0f;
        rq.qnan = lane < 16 ? nan_half[0] : nan_half[1];
    } else {
        rq.own = -1;
        rq.qs = 0.0f;
        rq.qnan = false;
    }
}

// Score one page for the 32 rows of the current request; returns the page-NaN flag
// through `page_nan` and the per-lane maxima in r0 (row m) and r1 (row 16+m).
__device__ __forceinline__ void score_page(const PageRegs &p, const uint64_t *lut,
                                           const RequestRegs &rq, float &r0, float &r1,
                                           bool &page_nan)
{
    const float ninf = -__builtin_huge_valf();
    v4f mx0 = {ninf, ninf, ninf, ninf};
    v4f mx1 = mx0;
    bool nan = false;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t w[4] = {p.codes[t][0], p.codes[t][1], p.codes[t][2], p.codes[t][3]};
        v4f c0 = {0.f, 0.f, 0.f, 0.f};
        v4f c1 = c0;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint32_t s = (p.sc[t] >> (8 * hh)) & 0xFFu;
            const uint64_t e = lut[s];
            const uint32_t flip = scale_sign_flip(s);
            nan |= scale_is_nan(s);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                uint32_t ev, od;
                dequant_word(w[2 * hh + k] ^ flip, uint32_t(e >> 32), uint32_t(e), ev, od);
                const v8h av = __builtin_bit_cast(v8h, f16_word(ev, od));
                c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    av, __builtin_bit_cast(v8h, rq.qa[2 * hh + k]), c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    av, __builtin_bit_cast(v8h, rq.qb[2 * hh + k]), c1, 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mx0[i] = fmaxf(mx0[i], c0[i]);
            mx1[i] = fmaxf(mx1[i], c1[i]);
        }
    }
    float m0 = fmaxf(fmaxf(mx0[0], mx0[1]), fmaxf(mx0[2], mx0[3]));
    float m1 = fmaxf(fmaxf(mx1[0], mx1[1]), fmaxf(mx1[2], mx1[3]));
    m0 = fmaxf(m0, __shfl_xor(m0, 16));
    m0 = fmaxf(m0, __shfl_xor(m0, 32));
    m1 = fmaxf(m1, __shfl_xor(m1, 16));
    m1 = fmaxf(m1, __shfl_xor(m1, 32));
    r0 = m0;
    r1 = m1;
    page_nan = __any(nan);
}

__global__ __launch_bounds__(256) void score_decode_kernel(
    const uint8_t *__restrict__ kv, int64_t page_stride, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ seq_lens, const uint8_t *__restrict__ q,
    const float *__restrict__ q_scale, int32_t num_reqs, int32_t qlen, int32_t width,
    float *__restrict__ scores, int32_t *__restrict__ row_own)
{
    __shared__ uint64_t lut[256];
    __shared__ int32_t partial[256];
    extern __shared__ int32_t prefix[];   // num_reqs + 1 entries
    const int tid = threadIdx.x;
    load_lut_to_lds(lut);

    // Own page of every row of every request (-1 for rows without a query).
    if (row_own) {
        for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < (int64_t)num_reqs * kDecodeRows;
             i += (int64_t)gridDim.x * 256)
            row_own[i] = decode_own(seq_lens[i / kDecodeRows], qlen,
                                    (int)(i % kDecodeRows) / kDecodeHeads);
    }

    // Exclusive prefix sum of the pages scored per request.
    const int per = (num_reqs + 255) / 256;
    const int rb = tid * per;
    const int re = rb + per < num_reqs ? rb + per : num_reqs;
    int local = 0;
    for (int r = rb; r < re; ++r)
        local += pages_scored(seq_lens[r], width);
    partial[tid] = local;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int v = tid >= off ? partial[tid - off] : 0;
        __syncthreads();
        partial[tid] += v;
        __syncthreads();
    }
    int run = partial[tid] - local;
    for (int r = rb; r < re; ++r) {
        prefix[r] = run;
        run += pages_scored(seq_lens[r], width);
    }
    if (tid == 255)
        prefix[num_reqs] = partial[255];
    __syncthreads();

    const int64_t total = prefix[num_reqs];
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int m = lane & 15;
    const int g = lane >> 4;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    const int64_t base = total / nwaves, rem = total % nwaves;
    int64_t p = w * base + (w < rem ? w : rem);
    const int64_t pend = p + base + (w < rem ? 1 : 0);
    if (p >= pend)
        return;

    // Request holding flattened page p: prefix[b] <= p < prefix[b + 1].
    auto find_req = [&](int64_t pp) {
        int lo = 0, hi = num_reqs;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (prefix[mid] <= pp)
                lo = mid;
            else
                hi = mid;
        }
        return lo;
    };
    // Lane i caches the page id of flattened page cache_base + i.
    int64_t cache_base = p;
    auto fill_cache = [&](int64_t cb) {
        const int64_t pl = cb + lane;
        int32_t id = -1;
        if (pl < pend) {
            const int bl = find_req(pl);
            id = block_table[(int64_t)bl * bt_stride + (pl - prefix[bl])];
        }
        return id;
    };
    int32_t id_cache = fill_cache(cache_base);
    auto page_id = [&](int64_t pp) -> int64_t {
        return (int64_t)__shfl(id_cache, (int)(pp - cache_base));
    };

    int b = find_req(p);
    int64_t bend = prefix[b + 1];
    RequestRegs rq;
    load_request(rq, q, q_scale, seq_lens, qlen, b, lane, m, g);

    PageRegs cur, nxt;
    int64_t id = page_id(p);
    bool cur_ok = id >= 0 && id < num_blocks;
    if (cur_ok)
        fetch_page(cur, kv + id * page_stride, m, g);

    for (;;) {
        const int64_t pn = p + 1;
        const bool has_next = pn < pend;
        bool nxt_ok = false;
        if (has_next) {
            if (pn - cache_base >= kWave) {
                cache_base = pn;
                id_cache = fill_cache(cache_base);
            }
            const int64_t idn = page_id(pn);
            nxt_ok = idn >= 0 && idn < num_blocks;
            if (nxt_ok)
                fetch_page(nxt, kv + idn * page_stride, m, g);
        }
        if (cur_ok) {
            float r0, r1;
            bool page_nan;
            score_page(cur, lut, rq, r0, r1, page_nan);
            const int j = (int)(p - prefix[b]);
            if (lane < kDecodeRows && j < rq.own) {
                const float v = lane < 16 ? r0 : r1;
                float s = (v + fabsf(v)) * 0.5f * rq.qs;
                if (page_nan || rq.qnan)
                    s = __builtin_nanf("");
                scores[((int64_t)b * kDecodeRows + lane) * width + j] = s;
            }
        }
        if (!has_next)
            break;
        p = pn;
        if (p >= bend) {
            b = find_req(p);
            bend = prefix[b + 1];
            load_request(rq, q, q_scale, seq_lens, qlen, b, lane, m, g);
        }
        cur = nxt;
        cur_ok = nxt_ok;
    }
}

}  // namespace

hipError_t launch_score_decode(const uint8_t *kv, int64_t page_stride, int64_t num_blocks,
                               const int32_t *block_table, int64_t bt_stride,
                               const int32_t *seq_lens, const uint8_t *q, const float *q_scale,
                               int32_t num_reqs, int32_t qlen, int32_t width, float *scores,
                               int32_t *row_own, int num_cus, hipStream_t stream)
{
    // Enough waves to cover the upper bound of the pages at two per wave, at
    // most two blocks (eight waves, the occupancy the kernel's registers allow) per
    // compute unit.
    const int64_t max_pages = (int64_t)num_reqs * width;
    int64_t blocks = (max_pages + 2 * kWavesPerBlock - 1) / (2 * kWavesPerBlock);
    const int64_t cap = (int64_t)(num_cus > 0 ? num_cus : 256) * 2;
    if (blocks > cap)
        blocks = cap;
    if (blocks < 1)
        blocks = 1;
    const size_t lds = sizeof(int32_t) * ((size_t)num_reqs + 1);
    hipLaunchKernelGGL(score_decode_kernel, dim3((uint32_t)blocks), dim3(256), lds, stream, kv,
                       page_stride, num_blocks, block_table, bt_stride, seq_lens, q, q_scale,
                       num_reqs, qlen, width, scores, row_own);
    return hipGetLastError();
}

}  // namespace pagescore
