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
// steps.  A wave cannot issue VALU work while its own MFMAs run, and the
// VALU of a second wave on the SIMD runs at about half rate meanwhile
// (measured), so the per-page cost is close to the sum of both: the
// dequantization keeps to 12 VALU operations per 8 elements, the MFMA
// results stay in VGPRs, and tiles are taken in pairs -- a burst of
// dequantization for two tiles, then their 16 MFMAs -- so that the two waves
// of a SIMD can overlap one's VALU burst with the other's MFMA burst.  The
// table is signed (a negative scale's entry carries the sign bit and the
// code's sign is XOR-ed in), so negative scales need no extra work and every
// page takes the same path.
//
// Scheduling: work-group (x, b) covers request b; each of its waves owns a run
// of `chunk` consecutive pages (chosen on the host from the batch size).  A
// batch too large for one round of such runs (ragged batches, whose upper
// bound of requests x width is far above their real pages) takes the flat
// schedule instead: the real pages are split evenly over all waves
// (score_decode_flat_kernel).  A
// wave issues its first loads -- the request's length, the run's page ids and
// the query rows -- all at once, so a single memory round trip precedes the
// first page fetch.  Then it scores the run from one set of page registers
// that is refilled as it is consumed: the next page's scale block as soon as
// this page's is staged, and the next page's codes of each tile right after
// the tile is scored, so every load is issued one page-time before its use
// (past the run's end the loads go through an empty descriptor and cost
// nothing).  Runs past a request's last page exit at once, and the hardware
// dispatcher back-fills the compute units, which balances ragged batches.
//
// NaN propagates through the arithmetic itself: a NaN scale byte gives its
// group NaN keys (the table entry of a NaN scale is all 0x7F), a NaN query
// byte a NaN query element, the f16 MFMA carries a NaN operand into every dot
// it enters, and the page maximum is taken with v_maximum3_f32, which
// propagates NaN (IEEE 754-2019 maximum).  So a NaN scale makes its token's
// dots, and the page score, NaN; a NaN query byte makes its row NaN.
#include "device_common.hpp"
#include "launch.hpp"
#include "wave_keys.hpp"

namespace pagescore {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kWavesPerBlock = 4;
constexpr int kXcds = 8;   // accelerator complex dies of an MI355X, each with its own L2
// Batches of up to this many requests take the flat schedule (each wave
// walks the request list once to find its share).
constexpr int32_t kFlatMaxReqs = 4096;

struct PageRegs {
    u32x4 codes[8];   // per tile: 16 code bytes of token 16*tile + m, chunk g
    u32x4 scales;     // bytes 16*lane .. 16*lane+15 of the page's 1 KiB of scales
};

// One page: one coalesced 16-byte load per lane of the scale block and eight
// 16-byte code loads per lane (1 KiB per wave each), as buffer loads against
// a descriptor that covers only this page.  A descriptor with no records
// makes every load return zeros without touching memory, so a wave issues
// the same loads for every page, whether it exists or not.
constexpr int kStreamLoad = 2;   // cache policy: nontemporal (streamed once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t *page, bool live)
{
    return uniform_rsrc(page, live ? kPageBytes : 0u);
}

// The scale block first, as the page loop refills it: the first page's loads
// then stand in the same order as every later page's, and the compiler can
// wait for each load by the same count (anything else merges to a full wait
// at the loop head).
__device__ __forceinline__ void fetch_page(PageRegs &p, __amdgpu_buffer_rsrc_t src, int lane, int m,
                                           int g)
{
    p.scales = __builtin_amdgcn_raw_buffer_load_b128(src, kCodeBytes + 16 * lane, 0, kStreamLoad);
#pragma unroll
    for (int t = 0; t < 8; ++t)
        p.codes[t] = __builtin_amdgcn_raw_buffer_load_b128(src, (16 * t + m) * 64 + 16 * g, 0,
                                                           kStreamLoad);
}

// The 2 scale bytes of tile t for this lane (token 16*t + m, groups 2g and
// 2g+1), gathered through the wave's 1 KiB LDS staging area.
__device__ __forceinline__ void unpack_scales(const PageRegs &p, uint8_t *stage, int lane, int m,
                                              int g, uint32_t sc[8])
{
    *reinterpret_cast<u32x4 *>(stage + 16 * lane) = p.scales;
    wave_lds_sync();   // other lanes' bytes are read next
#pragma unroll
    for (int t = 0; t < 8; ++t)
        sc[t] = *reinterpret_cast<const uint16_t *>(stage + (16 * t + m) * 8 + 2 * g);
    wave_lds_sync();   // before the next page's block overwrites the area
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

// The score row a lane stores once a page's maxima are joined across lanes:
// lanes 0..15 rows 0..15, lanes 32..47 rows 16..31, others none (-1).
__device__ __forceinline__ int store_row(int lane)
{
    return lane < 16 ? lane : (lane >= 32 && lane < 48 ? lane - 16 : -1);
}

struct RequestRegs {
    u32x4 qa[4], qb[4];  // B operands (f16): query rows m and 16+m, chunk g, per code word
    int own;             // own page of row store_row(lane) (-1 for other lanes)
    float qs;            // q_scale of that row
};

// Raw query bytes (rows m and 16+m, depth chunk g) and the q_scale of row
// store_row(lane), as loaded; slots without a query are not read.
struct RequestRaw {
    uint32_t bytes[2][8];
    float qs;
};

__device__ __forceinline__ void load_request_raw(RequestRaw &r, const uint8_t *__restrict__ q,
                                                 const float *__restrict__ q_scale, int32_t qlen,
                                                 int b, int lane, int m, int g)
{
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int row = 16 * hf + m;
        uint4 u0 = make_uint4(0u, 0u, 0u, 0u), u1 = u0;
        if (row / kDecodeHeads >= kSlots - qlen) {
            const uint4 *src =
                reinterpret_cast<const uint4 *>(q + ((int64_t)b * kDecodeRows + row) * kDepth + 32 * g);
            u0 = src[0];
            u1 = src[1];
        }
        const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r.bytes[hf][i] = w[i];
    }
    r.qs = 0.0f;
    const int row = store_row(lane);
    if (row >= 0 && row / kDecodeHeads >= kSlots - qlen)
        r.qs = q_scale[(int64_t)b * kDecodeRows + row];
}

__device__ __forceinline__ void finish_request(RequestRegs &rq, const RequestRaw &r, int32_t seq,
                                               int32_t qlen, int lane)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        rq.qa[k] = q_word_f16(r.bytes[0][2 * k], r.bytes[0][2 * k + 1]);
        rq.qb[k] = q_word_f16(r.bytes[1][2 * k], r.bytes[1][2 * k + 1]);
    }
    const int row = store_row(lane);
    rq.own = row >= 0 ? decode_own(seq, qlen, row / kDecodeHeads) : -1;
    rq.qs = row >= 0 ? r.qs : 0.0f;
}

// Dequantize the 8 E2M1 codes of one word against a signed table entry
// (byte c = E4M3 of code magnitude c times the scale, sign bit = the
// scale's): the code's sign bit is XOR-ed in, so the result's sign is the
// product of both signs (zeros included).
__device__ __forceinline__ void dequant_word_signed(uint32_t codes, uint32_t lut_hi, uint32_t lut_lo,
                                                    uint32_t &even, uint32_t &odd)
{
    const uint32_t mag_e = byte_perm(lut_hi, lut_lo, codes & 0x07070707u);
    const uint32_t mag_o = byte_perm(lut_hi, lut_lo, (codes >> 4) & 0x07070707u);
    even = mag_e ^ ((codes << 4) & 0x80808080u);
    odd = mag_o ^ (codes & 0x80808080u);
}

__device__ __forceinline__ float max3(float a, float b, float c)
{
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Score one page for the request's 32 rows: rmax is the page maximum of the
// raw dot products of row store_row(lane).  Each tile's code registers are
// refilled from nsrc (the next page) once the tile is scored.
__device__ __forceinline__ void score_page(PageRegs &p, const uint32_t sc[8],
                                           const uint64_t *lut, const RequestRegs &rq,
                                           __amdgpu_buffer_rsrc_t nsrc, int lane, int m, int g,
                                           float &rmax)
{
    const float ninf = -__builtin_huge_valf();
    v4f mx0 = {ninf, ninf, ninf, ninf};
    v4f mx1 = mx0;
#pragma unroll
    for (int tp = 0; tp < 4; ++tp) {
        // The fence keeps the compiler from hoisting the selector arithmetic
        // of later tiles to the top of the page, which would hold dozens of
        // registers live at once.
        __builtin_amdgcn_sched_barrier(0);
        v8h av[2][4];   // A operands (f16 keys) of tiles 2tp and 2tp+1, per code word
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int t = 2 * tp + u;
            const uint32_t w[4] = {p.codes[t][0], p.codes[t][1], p.codes[t][2], p.codes[t][3]};
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const uint64_t e = lut[(sc[t] >> (8 * hh)) & 0xFFu];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    uint32_t ev, od;
                    dequant_word_signed(w[2 * hh + k], uint32_t(e >> 32), uint32_t(e), ev, od);
                    av[u][2 * hh + k] = __builtin_bit_cast(v8h, f16_word(ev, od));
                }
            }
        }
        v4f c[2][2];    // [tile][query half]
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            c[u][0] = v4f{0.f, 0.f, 0.f, 0.f};
            c[u][1] = c[u][0];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                c[u][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    av[u][k], __builtin_bit_cast(v8h, rq.qa[k]), c[u][0], 0, 0, 0);
                c[u][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    av[u][k], __builtin_bit_cast(v8h, rq.qb[k]), c[u][1], 0, 0, 0);
            }
            // This tile's code registers are free: they take the next page's.
            const int t = 2 * tp + u;
            p.codes[t] = __builtin_amdgcn_raw_buffer_load_b128(nsrc, (16 * t + m) * 64 + 16 * g, 0,
                                                               kStreamLoad);
        }
        // Issue order: the four table reads, the dequantization of both
        // tiles, then their 16 MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 200, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mx0[i] = max3(mx0[i], c[0][0][i], c[1][0][i]);
            mx1[i] = max3(mx1[i], c[0][1][i], c[1][1][i]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    const float m0 = max3(mx0[0], mx0[1], __builtin_elementwise_maximum(mx0[2], mx0[3]));
    const float m1 = max3(mx1[0], mx1[1], __builtin_elementwise_maximum(mx1[2], mx1[3]));
    // Join the four depth-chunk lanes of each row with two lane swaps: the
    // 32-lane swap pairs m0's halves in lanes 0..31 and m1's in 32..63, the
    // 16-lane swap finishes both.  Lane m then holds row m and lane 32 + m
    // row 16 + m (see store_row).
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(m0), __float_as_uint(m1), false,
                                                    false);
    float x = __builtin_elementwise_maximum(__uint_as_float(h[0]), __uint_as_float(h[1]));
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = __builtin_elementwise_maximum(x, __uint_as_float((lane & 16) ? q[0] : q[1]));
    rmax = x;
}

__global__ __launch_bounds__(256, 2) void score_decode_kernel(
    const uint8_t *__restrict__ kv, int64_t page_stride, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ seq_lens, const uint8_t *__restrict__ q,
    const float *__restrict__ q_scale, int32_t qlen, int32_t width, int32_t chunk,
    float *__restrict__ scores, int32_t *__restrict__ row_own)
{
    __shared__ uint64_t lut[256];
    __shared__ __align__(16) uint8_t scale_stage[kWavesPerBlock][1024];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int m = lane & 15;
    const int g = lane >> 4;
    // XCD-aware block order.  Work-groups are dispatched round-robin over the
    // eight XCDs, each with its own L2.  Renumbering so that every XCD gets a
    // contiguous range of (request, run) blocks keeps the columns a row's
    // 128-byte score lines share inside one L2, which then writes whole lines
    // back instead of four partial ones from four XCDs.
    const int gx = gridDim.x;
    const int total = gx * gridDim.y;
    const int lin = blockIdx.x + blockIdx.y * gx;
    const int xcd = lin % kXcds, slot = lin / kXcds;
    const int per = total / kXcds, extra = total % kXcds;
    const int logical = xcd < extra ? xcd * (per + 1) + slot : extra * (per + 1) + (xcd - extra) * per + slot;
    const int b = logical / gx;
    // The run [j0, j1) is uniform; read through readfirstlane, the per-page
    // bounds and page addresses stay in scalar registers.
    const int j0 = __builtin_amdgcn_readfirstlane(((logical % gx) * kWavesPerBlock + wave) * chunk);
    uint8_t *stage = scale_stage[wave];

    // First round of loads, all independent: the request's length, the run's
    // page ids (in bounds whatever the length: columns below the width), the
    // table and the query rows.  The first page is requested as soon as the
    // length and the ids are in; the table, the query conversion and the
    // barrier come after, while that page is in flight.
    const int32_t seq = __builtin_amdgcn_readfirstlane(seq_lens[b]);
    int32_t id_lane = -1;
    if (lane < chunk && j0 + lane < width)
        id_lane = block_table[(int64_t)b * bt_stride + j0 + lane];
    const uint64_t lut_entry_g = kNvfp4Lut.entry[tid];
    RequestRaw qraw;
    load_request_raw(qraw, q, q_scale, qlen, b, lane, m, g);

    const int np = pages_scored(seq, width);
    const int j1 = __builtin_amdgcn_readfirstlane(j0 + chunk < np ? j0 + chunk : np);
    // A work-group past the request's last page leaves as soon as the length
    // is in (the first work-group of a request stays: it writes row_own).
    // Ragged batches launch many such groups.
    if (logical % gx != 0 && (logical % gx) * kWavesPerBlock * chunk >= np)
        return;

    // Descriptor of page j: empty past the run and for an id out of range
    // (such a page is not scored).  The id is read with v_readlane, so the
    // page base is a scalar and every load uses it with a constant per-lane
    // offset.
    // Page ids are 32-bit, so the bound is compared in 32 bits (scalar ALU).
    const int32_t nb32 = num_blocks > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)num_blocks;
    auto page_src = [&](int j, bool &ok) -> __amdgpu_buffer_rsrc_t {
        const int32_t id = __builtin_amdgcn_readlane(id_lane, j - j0);
        ok = j < j1 && id >= 0 && id < nb32;
        return page_rsrc(kv + (int64_t)(ok ? id : 0) * page_stride, ok);
    };
    // The first page is requested without a branch (an empty run gets an
    // empty descriptor): after a conditional load the compiler could not
    // count the loads in flight and would wait for the page before the
    // query conversion below.
    PageRegs pr;
    bool cur_ok = false;
    fetch_page(pr, page_src(j0, cur_ok), lane, m, g);

    // Signed table: a negative scale's entry carries the sign bit.
    lut[tid] = lut_entry_g | ((tid & 0x80) ? 0x8080808080808080ull : 0ull);
    RequestRegs rq;
    finish_request(rq, qraw, seq, qlen, lane);
    if (logical % gx == 0 && wave == 0 && row_own && store_row(lane) >= 0)
        row_own[(int64_t)b * kDecodeRows + store_row(lane)] = rq.own;
    __syncthreads();
    if (j0 >= j1)
        return;

    // One set of page registers, refilled as it is consumed: the next page's
    // scale block is requested once this page's is staged, and its codes
    // tile by tile as this page's tiles are scored.  Past the run's last
    // page the descriptor is empty and the loads cost nothing.
    for (int j = j0; j < j1; ++j) {
        bool nxt_ok;
        const __amdgpu_buffer_rsrc_t nsrc = page_src(j + 1 < j1 ? j + 1 : j1, nxt_ok);
        uint32_t sc[8];
        unpack_scales(pr, stage, lane, m, g, sc);
        pr.scales = __builtin_amdgcn_raw_buffer_load_b128(nsrc, kCodeBytes + 16 * lane, 0, kStreamLoad);
        float v;
        score_page(pr, sc, lut, rq, nsrc, lane, m, g, v);
        // Lanes without a row have own = -1 and store nothing.
        if (cur_ok && j < rq.own) {
            const float s = (v + fabsf(v)) * 0.5f * rq.qs;
            scores[((int64_t)b * kDecodeRows + store_row(lane)) * width + j] = s;
        }
        cur_ok = nxt_ok;
    }
}

// The pages [ja, jb) of request b (length seq): its query rows, then runs of
// up to 64 pages, each run's ids loaded at once and its pages scored through
// the one set of page registers as in score_decode_kernel.
__device__ __forceinline__ void score_segment(
    const uint8_t *__restrict__ kv, int64_t page_stride, int32_t nb32,
    const int32_t *__restrict__ block_table, int64_t bt_stride, const uint8_t *__restrict__ q,
    const float *__restrict__ q_scale, int32_t qlen, int32_t width, float *__restrict__ scores,
    const uint64_t *lut, uint8_t *stage, int b, int32_t seq, int ja, int jb, int lane, int m, int g)
{
    RequestRaw qraw;
    load_request_raw(qraw, q, q_scale, qlen, b, lane, m, g);
    int32_t id_lane = lane < jb - ja ? block_table[(int64_t)b * bt_stride + ja + lane] : -1;
    RequestRegs rq;
    finish_request(rq, qraw, seq, qlen, lane);
    for (int j0 = ja; j0 < jb; j0 += kWave) {
        const int j1 = __builtin_amdgcn_readfirstlane(j0 + kWave < jb ? j0 + kWave : jb);
        if (j0 > ja)
            id_lane = lane < j1 - j0 ? block_table[(int64_t)b * bt_stride + j0 + lane] : -1;
        // (j = j1 after a full run of 64 reads lane 0 back; the page is not scored.)
        auto page_src = [&](int j, bool &ok) -> __amdgpu_buffer_rsrc_t {
            const int32_t id = __builtin_amdgcn_readlane(id_lane, (j - j0) & (kWave - 1));
            ok = j < j1 && id >= 0 && id < nb32;
            return page_rsrc(kv + (int64_t)(ok ? id : 0) * page_stride, ok);
        };
        PageRegs pr;
        bool cur_ok = false;
        fetch_page(pr, page_src(j0, cur_ok), lane, m, g);
        for (int j = j0; j < j1; ++j) {
            bool nxt_ok;
            const __amdgpu_buffer_rsrc_t nsrc = page_src(j + 1 < j1 ? j + 1 : j1, nxt_ok);
            uint32_t sc[8];
            unpack_scales(pr, stage, lane, m, g, sc);
            pr.scales = __builtin_amdgcn_raw_buffer_load_b128(nsrc, kCodeBytes + 16 * lane, 0, kStreamLoad);
            float v;
            score_page(pr, sc, lut, rq, nsrc, lane, m, g, v);
            if (cur_ok && j < rq.own) {
                const float s = (v + fabsf(v)) * 0.5f * rq.qs;
                scores[((int64_t)b * kDecodeRows + store_row(lane)) * width + j] = s;
            }
            cur_ok = nxt_ok;
        }
    }
}

// Flat schedule: the batch's real pages, listed request by request, are
// split into equal shares over every wave of the grid (P w / W onward for
// wave w of W), whatever the requests' lengths.  A share is one or a few
// segments of consecutive pages of one request.  Requests are numbered over
// the waves for their row_own.  A ragged batch then runs in one even round
// instead of a grid over requests x width whose work-groups past a
// request's last page exit at once, leaving the real pages in uneven
// rounds.
__global__ __launch_bounds__(256, 2) void score_decode_flat_kernel(
    const uint8_t *__restrict__ kv, int64_t page_stride, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ seq_lens, const uint8_t *__restrict__ q,
    const float *__restrict__ q_scale, int32_t num_reqs, int32_t qlen, int32_t width,
    float *__restrict__ scores, int32_t *__restrict__ row_own)
{
    __shared__ uint64_t lut[256];
    __shared__ __align__(16) uint8_t scale_stage[kWavesPerBlock][1024];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int m = lane & 15;
    const int g = lane >> 4;
    // Work-groups numbered so that every XCD holds a contiguous range of
    // shares (score lines shared by neighbouring columns stay in one L2).
    const int G = gridDim.x;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int per = G / kXcds, extra = G % kXcds;
    const int logical = xcd < extra ? xcd * (per + 1) + slot : extra * (per + 1) + (xcd - extra) * per + slot;
    const int64_t W = (int64_t)G * kWavesPerBlock;
    const int64_t w = (int64_t)logical * kWavesPerBlock + wave;
    lut[tid] = kNvfp4Lut.entry[tid] | ((tid & 0x80) ? 0x8080808080808080ull : 0ull);
    uint8_t *stage = scale_stage[wave];

    // The batch's pages (the host keeps num_reqs x width below 2^31).
    int32_t total = 0;
    for (int b0 = 0; b0 < num_reqs; b0 += kWave)
        total += b0 + lane < num_reqs ? pages_scored(seq_lens[b0 + lane], width) : 0;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1)
        total += __shfl_xor(total, d);
    total = __builtin_amdgcn_readfirstlane(total);
    const int64_t s0 = (int64_t)total * w / W, s1 = (int64_t)total * (w + 1) / W;
    if (row_own != nullptr && store_row(lane) >= 0) {
        for (int64_t b = w; b < num_reqs; b += W)
            row_own[b * kDecodeRows + store_row(lane)] = decode_own(seq_lens[b], qlen, store_row(lane) / kDecodeHeads);
    }
    __syncthreads();   // the table is in LDS
    if (s0 >= s1)
        return;

    // The request holding page s0: windows of 64 requests and the inclusive
    // sums of their page counts.
    int64_t pos = 0;
    int b = num_reqs;
    for (int b0 = 0; b0 < num_reqs; b0 += kWave) {
        const int bb = b0 + lane;
        const int n = bb < num_reqs ? pages_scored(seq_lens[bb], width) : 0;
        const int excl = wave_prefix_sum(n, lane);
        const int win = __builtin_amdgcn_readlane(excl + n, kWave - 1);
        if (pos + win <= s0) {
            pos += win;
            continue;
        }
        const uint64_t mask = __ballot(bb < num_reqs && pos + excl + n > s0);
        const int first = (int)__builtin_ctzll(mask);
        b = b0 + first;
        pos += __builtin_amdgcn_readlane(excl, first);
        break;
    }
    const int32_t nb32 = num_blocks > 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)num_blocks;
    for (; b < num_reqs && pos < s1; ++b) {
        const int32_t seq = __builtin_amdgcn_readfirstlane(seq_lens[b]);
        const int np = pages_scored(seq, width);
        const int ja = (int)(s0 > pos ? s0 - pos : 0);
        const int jb = (int)(s1 - pos < np ? s1 - pos : np);
        if (ja < jb)
            score_segment(kv, page_stride, nb32, block_table, bt_stride, q, q_scale, qlen, width, scores,
                          lut, stage, b, seq, ja, jb, lane, m, g);
        pos += np;
    }
}

}  // namespace

hipError_t launch_score_decode(const uint8_t *kv, int64_t page_stride, int64_t num_blocks,
                               const int32_t *block_table, int64_t bt_stride,
                               const int32_t *seq_lens, const uint8_t *q, const float *q_scale,
                               int32_t num_reqs, int32_t qlen, int32_t width, float *scores,
                               int32_t *row_own, int num_cus, hipStream_t stream)
{
    // Pages per wave: the batch's upper bound of pages spread over about eight
    // waves per compute unit (two resident work-groups of four), 1..8.  Past
    // 8, ragged batches (whose upper bound is far above their real pages)
    // lose more to the last runs than they save on per-run set-up.
    const int64_t max_pages = (int64_t)num_reqs * width;
    const int64_t waves = (int64_t)(num_cus > 0 ? num_cus : 256) * 8;
    // The grid holds at most 8 pages per wave; a batch whose upper bound of
    // pages exceeds one round of that (ragged or very large batches) takes
    // the flat schedule, which splits the real pages evenly instead.
    if (max_pages > waves * 8 && num_reqs <= kFlatMaxReqs && max_pages <= 0x7FFFFFFF) {
        const dim3 grid((uint32_t)((num_cus > 0 ? num_cus : 256) * 2));
        hipLaunchKernelGGL(score_decode_flat_kernel, grid, dim3(256), 0, stream, kv, page_stride,
                           num_blocks, block_table, bt_stride, seq_lens, q, q_scale, num_reqs, qlen,
                           width, scores, row_own);
        return hipGetLastError();
    }
    int64_t chunk = (max_pages + waves - 1) / waves;
    chunk = chunk < 1 ? 1 : (chunk > 8 ? 8 : chunk);
    const int64_t gx = ((int64_t)width + chunk * kWavesPerBlock - 1) / (chunk * kWavesPerBlock);
    hipLaunchKernelGGL(score_decode_kernel, dim3((uint32_t)gx, (uint32_t)num_reqs), dim3(256), 0,
                       stream, kv, page_stride, num_blocks, block_table, bt_stride, seq_lens, q,
                       q_scale, qlen, width, (int32_t)chunk, scores, row_own);
    return hipGetLastError();
}

}  // namespace pagescore
