// launch.hpp -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pagescore {

// Requests per indexer_score_decode or nvfp4_index_k_dequant call: one grid
// row per request.
constexpr int32_t kDecodeMaxReqs = 65535;
constexpr int32_t kDequantMaxReqs = 65535;

// Heads per indexer_score_prefill call: a work-group keeps one token's query
// rows (heads rounded up to 32) as f16 in LDS.
constexpr int32_t kPrefillMaxHeads = 224;
// Heads per indexer_score_prefill_ragged call (PAGESCORE_RAGGED_MAX_HEADS).
constexpr int32_t kRaggedMaxHeads = 64;

// Columns per topk16_select row: a wave reads its share of a row through a
// buffer descriptor whose byte size and offsets are 32-bit.
constexpr int32_t kTopkMaxWidth = 1 << 28;

hipError_t launch_nvfp4_dequant(const uint8_t *kv, int64_t page_stride, int64_t num_blocks,
                                const int32_t *block_table, int64_t bt_stride,
                                const int32_t *num_pages, const int32_t *page_offsets,
                                int32_t num_reqs, int32_t max_num_pages, uint8_t *out,
                                int64_t out_pages, hipStream_t stream);

hipError_t launch_score_decode(const uint8_t *kv, int64_t page_stride, int64_t num_blocks,
                               const int32_t *block_table, int64_t bt_stride,
                               const int32_t *seq_lens, const uint8_t *q, const float *q_scale,
                               int32_t num_reqs, int32_t qlen, int32_t width, float *scores,
                               int32_t *row_own, int num_cus, hipStream_t stream);

hipError_t launch_score_prefill(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                const float *k_scale, int32_t T, int32_t H, int32_t N,
                                float *scores, int64_t ld, hipStream_t stream);

hipError_t launch_score_prefill_ragged(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                       const float *k_scale, int32_t T, int32_t H, int32_t N,
                                       int32_t num_seqs, const int32_t *q_start,
                                       const int32_t *k_start, const int32_t *k_len, int32_t max_q,
                                       int32_t width, float *scores, int64_t ld, int32_t *row_len,
                                       int num_cus, hipStream_t stream);

// Block columns per token of the fused prefill top-16 (32 per 1,024 keys).
int64_t prefill_topk16_blocks(int32_t N);

hipError_t launch_prefill_topk16(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                 const float *k_scale, int32_t T, int32_t H, int32_t N, int32_t *out,
                                 int64_t out_stride, float *bmax, hipStream_t stream);

hipError_t launch_topk16(const float *scores, int64_t row_stride, int32_t num_rows, int32_t width,
                         const int32_t *valid_len, const int32_t *force_begin,
                         const int32_t *force_end, const int32_t *append_page, int32_t *out,
                         int64_t out_stride, int num_cus, hipStream_t stream);

hipError_t launch_mxfp8_quant(const uint16_t *x, int64_t ldx, int32_t rows, int32_t cols, uint8_t *q,
                              int64_t ldq, uint8_t *scales, int64_t lds, hipStream_t stream);

}  // namespace pagescore
