// api.hip -- the exported C ABI (declared in include/pagescore.h): host-side
// argument checks, then stream-ordered launches.  Nothing here synchronizes
// with the host or allocates memory (the allocation-free prefill top-16 uses
// a static device array, below).
#include <hip/hip_runtime.h>
#include <cstdint>
#include <mutex>

#include "launch.hpp"
#include "pagescore.h"

namespace {

thread_local int g_last_hip_error = 0;

int launch_status(hipError_t e)
{
    if (e == hipSuccess)
        return PAGESCORE_OK;
    g_last_hip_error = (int)e;
    return PAGESCORE_ELAUNCH;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// Workspace of indexer_prefill_topk16_noalloc: one array per GPU, held by the
// loaded code object until the process ends.  Host code never uses its name
// as an address (it is a host-side stand-in there); the device address comes
// from hipGetSymbolAddress, once per device, in noalloc_scratch().
static __device__ __align__(256) uint8_t scratch[PAGESCORE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (nullptr and the HIP
// error in *err if it cannot be had).
void *noalloc_scratch(hipError_t *err)
{
    static std::mutex mu;
    static void *addr[kMaxDevices] = {nullptr};
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess)
            return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

// Compute units of the current device, queried once per device.
int current_device_cus()
{
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

bool page_args_ok(const uint8_t *kv, int64_t page_stride, int64_t num_blocks)
{
    return kv && aligned16(kv) && page_stride >= PAGESCORE_PAGE_BYTES && (page_stride % 16) == 0 &&
           num_blocks >= 1;
}

}  // namespace

extern "C" {

int nvfp4_index_k_dequant(const uint8_t *kv_cache, int64_t page_stride_bytes, int64_t num_blocks,
                          const int32_t *block_table, int64_t bt_stride, const int32_t *num_pages,
                          const int32_t *page_offsets, int32_t num_reqs, int32_t max_num_pages,
                          uint8_t *out, int64_t out_pages, void *stream)
{
    if (num_reqs < 0 || num_reqs > pagescore::kDequantMaxReqs || max_num_pages < 0)
        return PAGESCORE_EINVAL;
    if (num_reqs == 0 || max_num_pages == 0)
        return PAGESCORE_OK;
    if (!page_args_ok(kv_cache, page_stride_bytes, num_blocks) || !block_table || !num_pages ||
        !page_offsets || !out || !aligned16(out) || out_pages < 0 || bt_stride < max_num_pages)
        return PAGESCORE_EINVAL;
    return launch_status(pagescore::launch_nvfp4_dequant(
        kv_cache, page_stride_bytes, num_blocks, block_table, bt_stride, num_pages, page_offsets,
        num_reqs, max_num_pages, out, out_pages, (hipStream_t)stream));
}

int indexer_score_decode(const uint8_t *kv_cache, int64_t page_stride_bytes, int64_t num_blocks,
                         const int32_t *block_table, int64_t bt_stride, const int32_t *seq_lens,
                         const uint8_t *q, const float *q_scale, int32_t num_reqs, int32_t qlen,
                         int32_t width, float *scores, int32_t *row_own, void *stream)
{
    if (num_reqs < 0 || num_reqs > pagescore::kDecodeMaxReqs || qlen < 1 ||
        qlen > PAGESCORE_SLOTS || width < 1)
        return PAGESCORE_EINVAL;
    if (num_reqs == 0)
        return PAGESCORE_OK;
    if (!page_args_ok(kv_cache, page_stride_bytes, num_blocks) || !block_table ||
        bt_stride < width || !seq_lens || !q || !aligned16(q) || !q_scale || !scores)
        return PAGESCORE_EINVAL;
    return launch_status(pagescore::launch_score_decode(
        kv_cache, page_stride_bytes, num_blocks, block_table, bt_stride, seq_lens, q, q_scale,
        num_reqs, qlen, width, scores, row_own, current_device_cus(), (hipStream_t)stream));
}

int indexer_score_prefill(const uint8_t *q, const float *q_scale, const uint8_t *k,
                          const float *k_scale, int32_t T, int32_t H, int32_t N, float *scores,
                          int64_t ld, void *stream)
{
    if (T < 0 || N < 0 || H < 1 || H > pagescore::kPrefillMaxHeads)
        return PAGESCORE_EINVAL;
    if (T == 0 || N == 0)
        return PAGESCORE_OK;
    if (!q || !aligned16(q) || !q_scale || !k || !aligned16(k) || !k_scale || !scores || ld < N)
        return PAGESCORE_EINVAL;
    return launch_status(pagescore::launch_score_prefill(q, q_scale, k, k_scale, T, H, N, scores, ld,
                                                         (hipStream_t)stream));
}

int indexer_score_prefill_ragged(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                 const float *k_scale, int32_t T, int32_t H, int32_t N,
                                 int32_t num_seqs, const int32_t *q_start, const int32_t *k_start,
                                 const int32_t *k_len, int32_t max_q, int32_t width, float *scores,
                                 int64_t ld, int32_t *row_len, void *stream)
{
    static_assert(PAGESCORE_RAGGED_MAX_HEADS == pagescore::kRaggedMaxHeads, "header and kernel agree");
    if (T < 0 || N < 0 || H < 1 || H > PAGESCORE_RAGGED_MAX_HEADS || num_seqs < 0 ||
        num_seqs > PAGESCORE_RAGGED_MAX_SEQS || max_q < 0 || width < 1)
        return PAGESCORE_EINVAL;
    if (T == 0 || num_seqs == 0 || max_q == 0)
        return PAGESCORE_OK;
    if (!q || !aligned16(q) || !q_scale || !k || !aligned16(k) || !k_scale || !q_start || !k_start ||
        !k_len || !scores || ld < width)
        return PAGESCORE_EINVAL;
    return launch_status(pagescore::launch_score_prefill_ragged(
        q, q_scale, k, k_scale, T, H, N, num_seqs, q_start, k_start, k_len, max_q, width, scores, ld,
        row_len, current_device_cus(), (hipStream_t)stream));
}

// Workspace of indexer_prefill_topk16: the block records, three planes of
// [T, blocks] (float32 largest and second largest score, int32 tile); -1
// for arguments out of range.
int64_t indexer_prefill_topk16_workspace(int32_t T, int32_t N)
{
    if (T < 0 || N < 1)
        return -1;
    return (int64_t)T * 3 * pagescore::prefill_topk16_blocks(N) * 4;
}

int indexer_prefill_topk16(const uint8_t *q, const float *q_scale, const uint8_t *k,
                           const float *k_scale, int32_t T, int32_t H, int32_t N, int32_t *out,
                           int64_t out_stride, void *workspace, int64_t workspace_bytes,
                           void *stream)
{
    if (T < 0 || N < 1 || H < 1 || H > PAGESCORE_PREFILL_TOPK_MAX_HEADS)
        return PAGESCORE_EINVAL;
    if (T == 0)
        return PAGESCORE_OK;
    if (!q || !aligned16(q) || !q_scale || !k || !aligned16(k) || !k_scale || !out ||
        out_stride < PAGESCORE_TOPK || !workspace || ((uintptr_t)workspace & 255u) != 0 ||
        workspace_bytes < indexer_prefill_topk16_workspace(T, N))
        return PAGESCORE_EINVAL;
    return launch_status(pagescore::launch_prefill_topk16(q, q_scale, k, k_scale, T, H, N, out,
                                                          out_stride, static_cast<float *>(workspace),
                                                          (hipStream_t)stream));
}

int indexer_prefill_topk16_noalloc(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                   const float *k_scale, int32_t T, int32_t H, int32_t N,
                                   int32_t *out, int64_t out_stride, void *stream)
{
    if (T < 0 || N < 1 || H < 1 || H > PAGESCORE_PREFILL_TOPK_MAX_HEADS)
        return PAGESCORE_EINVAL;
    if (T == 0)
        return PAGESCORE_OK;
    if (!q || !aligned16(q) || !q_scale || !k || !aligned16(k) || !k_scale || !out ||
        out_stride < PAGESCORE_TOPK)
        return PAGESCORE_EINVAL;
    if (indexer_prefill_topk16_workspace(T, N) > (int64_t)PAGESCORE_NOALLOC_SCRATCH_BYTES)
        return PAGESCORE_ENOSPACE;
    hipError_t err = hipSuccess;
    void *ws = noalloc_scratch(&err);
    if (ws == nullptr)
        return launch_status(err);
    return launch_status(pagescore::launch_prefill_topk16(q, q_scale, k, k_scale, T, H, N, out,
                                                          out_stride, static_cast<float *>(ws),
                                                          (hipStream_t)stream));
}

int topk16_select(const float *scores, int64_t row_stride, int32_t num_rows, int32_t width,
                  const int32_t *valid_len, const int32_t *force_begin, const int32_t *force_end,
                  const int32_t *append_page, int32_t *out, int64_t out_stride, void *stream)
{
    if (num_rows < 0 || width < 1 || width > pagescore::kTopkMaxWidth)
        return PAGESCORE_EINVAL;
    if (num_rows == 0)
        return PAGESCORE_OK;
    if (!scores || row_stride < width || !out || out_stride < PAGESCORE_TOPK ||
        (force_begin == nullptr) != (force_end == nullptr))
        return PAGESCORE_EINVAL;
    return launch_status(pagescore::launch_topk16(scores, row_stride, num_rows, width, valid_len,
                                                   force_begin, force_end, append_page, out,
                                                   out_stride, current_device_cus(),
                                                   (hipStream_t)stream));
}

int mxfp8_e4m3_quantize(const uint16_t *x, int64_t x_stride, int32_t rows, int32_t cols, uint8_t *q,
                        int64_t q_stride, uint8_t *scales, int64_t scale_stride, void *stream)
{
    if (rows < 0 || cols < 0 || cols % 32 != 0)
        return PAGESCORE_EINVAL;
    if (rows == 0 || cols == 0)
        return PAGESCORE_OK;
    if (!x || !aligned16(x) || x_stride < cols || x_stride % 8 != 0 || !q || !aligned16(q) ||
        q_stride < cols || q_stride % 16 != 0 || !scales || scale_stride < cols / 32)
        return PAGESCORE_EINVAL;
    return launch_status(pagescore::launch_mxfp8_quant(x, x_stride, rows, cols, q, q_stride, scales,
                                                        scale_stride, (hipStream_t)stream));
}

int pagescore_last_hip_error(void) { return g_last_hip_error; }

const char *pagescore_strerror(int code)
{
    switch (code) {
    case PAGESCORE_OK:
        return "ok";
    case PAGESCORE_EINVAL:
        return "invalid argument (host-side check)";
    case PAGESCORE_ELAUNCH:
        return "kernel launch failed (see pagescore_last_hip_error)";
    case PAGESCORE_ENOSPACE:
        return "the call needs more scratch than the library's fixed array holds";
    default:
        return "unknown error code";
    }
}

}  // extern "C"
