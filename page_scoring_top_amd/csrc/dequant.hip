// dequant.hip -- K1: gather packed NVFP4 index-K pages into contiguous E4M3 pages.
//
// Semantics: vLLM API page "gather_nvfp4_index_k", function
// minimax_m3_gather_nvfp4_index_k_fp8 (which pages go where) and the module
// description (page format; element = e4m3_rn_satfinite(e2m1 * scale)).
//
// A wave dequantizes a run of pages, one at a time.  Per round i (0..7) of a
// page it reads 1 KiB of codes (16 tokens x 64 B, one 16-byte load per lane,
// contiguous across the wave) and 128 B of scales (two bytes per lane), and
// writes 2 KiB of E4M3 output (two 16-byte stores per lane, contiguous).
// Lane l works on token 16i + l/4, elements 32*(l%4) .. 32*(l%4) + 31
// (block-scale groups 2*(l%4) and +1).  The page's 9 KiB in and 16 KiB out
// are each touched once: the kernel is bound by HBM at 25,604 algorithmic
// bytes per page (with its block-table entry).
#include "device_common.hpp"
#include "launch.hpp"

namespace pagescore {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesPerBlock = 4;
constexpr int kStreamLoad = 2;    // buffer cache policy: nontemporal (read once)

// A descriptor covering one page; with no records, loads through it return
// zeros without touching memory, so a wave issues the same loads for every
// page of its run, whether the page exists or not.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t *page, bool live)
{
    return uniform_rsrc(page, live ? kPageBytes : 0u);
}

// One page in registers: round i (tokens 16 i .. 16 i + 15) is 1 KiB of
// codes, 16 bytes per lane, and the round's 128 scale bytes, 2 per lane
// (lane l: token 16 i + l / 4, groups 2 (l % 4) and 2 (l % 4) + 1).
struct PageIn {
    u32x4 codes[8];
    uint32_t sc[8];
};

__device__ __forceinline__ void load_page(PageIn &p, __amdgpu_buffer_rsrc_t src, int lane)
{
#pragma unroll
    for (int i = 0; i < 8; ++i)
        p.codes[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(src, 1024 * i + 16 * lane, 0, kStreamLoad));
#pragma unroll
    for (int i = 0; i < 8; ++i)
        p.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(src, kCodeBytes + 128 * i + 2 * lane, 0,
                                                       kStreamLoad);
}

// Dequantize a page held in registers and write the 16 KiB of E4M3 out:
// per round, two 16-byte stores per lane (32 output bytes: the lane's 32
// elements of its token), contiguous across the wave.  Plain stores: the
// nontemporal form measured about a quarter slower here.
__device__ __forceinline__ void store_page(const PageIn &p, const uint64_t *lut, uint8_t *dst, int lane)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t w[4] = {p.codes[i][0], p.codes[i][1], p.codes[i][2], p.codes[i][3]};
        uint32_t o[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint32_t s = (p.sc[i] >> (8 * hh)) & 0xFFu;
            const uint64_t t = lut[s];
            const uint32_t flip = scale_sign_flip(s);
            const bool nan = scale_is_nan(s);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                uint32_t even, odd;
                dequant_word(w[2 * hh + k] ^ flip, uint32_t(t >> 32), uint32_t(t), even, odd);
                // Re-interleave to element order: e0 o0 e1 o1 | e2 o2 e3 o3.
                uint32_t a = byte_perm(odd, even, 0x05010400u);
                uint32_t b = byte_perm(odd, even, 0x07030602u);
                if (nan)
                    a = b = 0x7F7F7F7Fu;
                o[4 * hh + 2 * k] = a;
                o[4 * hh + 2 * k + 1] = b;
            }
        }
        u32x4 *d = reinterpret_cast<u32x4 *>(dst + 2048 * i + 32 * lane);
        d[0] = u32x4{o[0], o[1], o[2], o[3]};
        d[1] = u32x4{o[4], o[5], o[6], o[7]};
    }
}

// Work-group (x, r) covers request r; each wave owns a run of `run` logical
// pages.  The run's page ids, the request's page count and output offset
// and the table are requested at once; the first page follows as soon as
// the ids are in, and each page's successor is in flight while it is
// dequantized and stored.
__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(
    const uint8_t *__restrict__ kv, int64_t page_stride, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ num_pages, const int32_t *__restrict__ page_offsets,
    int32_t max_num_pages, int32_t run, uint8_t *__restrict__ out, int64_t out_pages)
{
    __shared__ uint64_t lut[256];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int r = blockIdx.y;
    const int j0 = (blockIdx.x * kWavesPerBlock + wave) * run;

    int n = num_pages[r];
    const int64_t off = page_offsets[r];
    int32_t id_lane = -1;
    if (lane < run && j0 + lane < max_num_pages)
        id_lane = block_table[(int64_t)r * bt_stride + j0 + lane];
    const uint64_t lut_entry = kNvfp4Lut.entry[tid];
    n = n < max_num_pages ? n : max_num_pages;
    const int j1 = j0 + run < n ? j0 + run : n;

    // Page j is dequantized when its id is in range and its output page is
    // inside `out`; otherwise nothing is read or written for it.
    auto page_src = [&](int j, bool &ok) -> __amdgpu_buffer_rsrc_t {
        const int64_t id = __builtin_amdgcn_readlane(id_lane, j - j0);
        const int64_t opage = off + j;
        ok = j < j1 && id >= 0 && id < num_blocks && opage >= 0 && opage < out_pages;
        return page_rsrc(kv + (ok ? id : 0) * page_stride, ok);
    };
    PageIn pa, pb;
    bool ok_a = false, ok_b = false;
    load_page(pa, page_src(j0, ok_a), lane);   // unconditional: empty descriptor for an empty run
    lut[tid] = lut_entry;
    __syncthreads();
    if (j0 >= j1)
        return;

    int j = j0;
    auto step = [&](const PageIn &cur, bool cur_ok, PageIn &nxt, bool &nxt_ok) -> bool {
        load_page(nxt, page_src(j + 1 < j1 ? j + 1 : j1, nxt_ok), lane);
        if (cur_ok)
            store_page(cur, lut, out + (off + j) * (kPageTokens * kDepth), lane);
        return ++j < j1;
    };
    for (;;) {
        if (!step(pa, ok_a, pb, ok_b))
            break;
        if (!step(pb, ok_b, pa, ok_a))
            break;
    }
}

}  // namespace

hipError_t launch_nvfp4_dequant(const uint8_t *kv, int64_t page_stride, int64_t num_blocks,
                                const int32_t *block_table, int64_t bt_stride,
                                const int32_t *num_pages, const int32_t *page_offsets,
                                int32_t num_reqs, int32_t max_num_pages, uint8_t *out,
                                int64_t out_pages, hipStream_t stream)
{
    // Pages per wave: the batch's upper bound spread over about 16 waves per
    // compute unit, 1..8 (a run's ids fit one wave's lanes).
    const int64_t max_pages = (int64_t)num_reqs * max_num_pages;
    int64_t run = (max_pages + 256 * 16 - 1) / (256 * 16);
    run = run < 1 ? 1 : (run > 8 ? 8 : run);
    const int64_t gx = ((int64_t)max_num_pages + run * kWavesPerBlock - 1) / (run * kWavesPerBlock);
    if (gx > 0x7FFFFFFF || num_reqs > 65535)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3((uint32_t)gx, (uint32_t)num_reqs), dim3(256), 0,
                       stream, kv, page_stride, num_blocks, block_table, bt_stride, num_pages,
                       page_offsets, max_num_pages, (int32_t)run, out, out_pages);
    return hipGetLastError();
}

}  // namespace pagescore
