// dequant.hip -- K1: gather packed NVFP4 index-K pages into contiguous E4M3 pages.
//
// Semantics: vLLM API page "gather_nvfp4_index_k", function
// minimax_m3_gather_nvfp4_index_k_fp8 (which pages go where) and the module
// description (page format; element = e4m3_rn_satfinite(e2m1 * scale)).
//
// One wave per output page.  Per round i (0..7) the wave reads 1 KiB of codes
// (16 tokens x 64 B, one 16-byte load per lane, contiguous across the wave)
// and 128 B of scales (two bytes per lane), and writes 2 KiB of E4M3 output
// (two 16-byte stores per lane, contiguous).  Lane l works on token 16i + l/4,
// elements 32*(l%4) .. 32*(l%4) + 31 (block-scale groups 2*(l%4) and +1).
// The page's 9 KiB in and 16 KiB out are each touched once: the kernel is
// bound by HBM at 25,600 algorithmic bytes per page.
#include "device_common.hpp"
#include "launch.hpp"

namespace pagescore {

namespace {

constexpr int kPagesPerBlock = 4;  // one wave per page

__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(
    const uint8_t *__restrict__ kv, int64_t page_stride, int64_t num_blocks,
    const int32_t *__restrict__ block_table, int64_t bt_stride,
    const int32_t *__restrict__ num_pages, const int32_t *__restrict__ page_offsets,
    int32_t max_num_pages, int32_t blocks_per_req, uint8_t *__restrict__ out, int64_t out_pages)
{
    __shared__ uint64_t lut[256];
    load_lut_to_lds(lut);
    __syncthreads();

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int r = blockIdx.x / blocks_per_req;
    const int j = (blockIdx.x % blocks_per_req) * kPagesPerBlock + wave;
    int n = num_pages[r];
    n = n < max_num_pages ? n : max_num_pages;
    if (j >= n)
        return;
    const int64_t pid = block_table[(int64_t)r * bt_stride + j];
    const int64_t opage = (int64_t)page_offsets[r] + j;
    if (pid < 0 || pid >= num_blocks || opage < 0 || opage >= out_pages)
        return;
    const uint8_t *src = kv + pid * page_stride;
    uint8_t *dst = out + opage * (kPageTokens * kDepth);

    const int chunk = lane & 3;      // 32-element chunk of the token
    const int tok_in_round = lane >> 2;

    uint4 codes[8];
    uint32_t sc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        codes[i] = *reinterpret_cast<const uint4 *>(src + 1024 * i + 16 * lane);
        sc[i] = *reinterpret_cast<const uint16_t *>(src + kCodeBytes + (16 * i + tok_in_round) * 8 +
                                                    2 * chunk);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t w[4] = {codes[i].x, codes[i].y, codes[i].z, codes[i].w};
        uint32_t o[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint32_t s = (sc[i] >> (8 * hh)) & 0xFFu;
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
        uint4 *d = reinterpret_cast<uint4 *>(dst + 2048 * i + 32 * lane);
        d[0] = make_uint4(o[0], o[1], o[2], o[3]);
        d[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

}  // namespace

hipError_t launch_nvfp4_dequant(const uint8_t *kv, int64_t page_stride, int64_t num_blocks,
                                const int32_t *block_table, int64_t bt_stride,
                                const int32_t *num_pages, const int32_t *page_offsets,
                                int32_t num_reqs, int32_t max_num_pages, uint8_t *out,
                                int64_t out_pages, hipStream_t stream)
{
    const int32_t blocks_per_req = (max_num_pages + kPagesPerBlock - 1) / kPagesPerBlock;
    const int64_t grid = (int64_t)blocks_per_req * num_reqs;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, kv,
                       page_stride, num_blocks, block_table, bt_stride, num_pages, page_offsets,
                       max_num_pages, blocks_per_req, out, out_pages);
    return hipGetLastError();
}

}  // namespace pagescore
