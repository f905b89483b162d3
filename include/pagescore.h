/*
 * pagescore.h -- C ABI of libpagescore.so, the gfx950 (MI355X) sparse-attention
 * indexer path: NVFP4 index-K dequantization, decode and prefill scores, and
 * the exact top-16 selection; and the MXFP8 quantization of the attention
 * output that follows it.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is DEVICE memory owned by the caller; the library
 *    allocates nothing and keeps no pointer after the call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued on it; no call synchronizes with the host, so every call
 *    can be captured into a HIP graph.
 *  - The return value is PAGESCORE_OK or a negative code.  Argument checks
 *    (null pointers, sizes, strides, alignment) happen on the host before
 *    anything is enqueued; on a check failure nothing is enqueued and no device
 *    memory is touched.  PAGESCORE_ELAUNCH reports a failed kernel launch; the
 *    HIP error code is then returned by pagescore_last_hip_error().
 *  - Contents of device buffers (page ids, lengths, scales) cannot be checked
 *    on the host.  Where a kernel could otherwise read out of bounds it checks
 *    on the device (page ids against num_blocks) and skips the work instead.
 *
 * Geometry: a page holds 128 tokens, the key depth is 128, decode uses 8 query
 * slots and 4 index heads, and a top-16 row holds 16 column ids.
 *
 * Source pages cited below:
 *   [GATHER] vLLM API page "vllm.models.minimax_m3.nvidia.ops.gather_nvfp4_index_k"
 *   [DECODE] vLLM API page "vllm.models.minimax_m3.nvidia.indexer_nvfp4_decode_cp"
 *   [MOJO]   Modular Mojo page "sparse_index_fp8_sm100"
 *   [MSA]    GitHub pull request wolfcomos/MSA #1 ("warp top-16")
 *   [ROCM]   vLLM pull request #65508 (ROCm MXFP8 epilogue)
 */
#ifndef PAGESCORE_H
#define PAGESCORE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAGESCORE_OK 0
#define PAGESCORE_EINVAL (-22)  /* an argument failed a host-side check      */
#define PAGESCORE_ELAUNCH (-5)  /* a kernel launch failed; see last_hip_error */
#define PAGESCORE_ENOSPACE (-28) /* more scratch needed than the fixed array holds */

#define PAGESCORE_PAGE_TOKENS 128
#define PAGESCORE_DEPTH 128
#define PAGESCORE_PAGE_BYTES 9216
#define PAGESCORE_SLOTS 8
#define PAGESCORE_DECODE_HEADS 4
#define PAGESCORE_TOPK 16

/*
 * nvfp4_index_k_dequant -- gather and dequantize packed NVFP4 index-K pages
 * into contiguous E4M3 pages ([GATHER], minimax_m3_gather_nvfp4_index_k_fp8,
 * and the module description for the page format and the rule).
 *
 * Page format (9,216 bytes, viewable as [128, 72] uint8): bytes 0..8191 hold
 * the E2M1 codes, 64 bytes per token, element 2i in the low nibble of byte i;
 * bytes 8192..9215 hold the E4M3 block scales, byte 8192 + token*8 + group for
 * the 16 elements of that group.  Element (t, e) dequantizes to
 * e4m3_rn_satfinite(e2m1(code) * e4m3(scale)): the exact product rounded once
 * to the nearest E4M3 value, ties to the even mantissa, saturating at +-448.
 * A NaN scale byte (0x7F/0xFF) gives 0x7F for every element of its group.
 *
 *   kv_cache          [num_blocks pages] at page_stride_bytes apart; 16-byte
 *                     aligned, page_stride_bytes >= 9216 and a multiple of 16.
 *   num_blocks        pages in kv_cache (>= 1 when anything is gathered).
 *   block_table       [num_reqs, bt_stride] int32: entry (r, j) is the index
 *                     in kv_cache of the page holding request r's logical
 *                     page j.
 *   num_pages         [num_reqs] int32: how many logical pages request r has.
 *   page_offsets      [num_reqs] int32: the page of out that receives request
 *                     r's logical page 0 (its later pages follow it).
 *   max_num_pages     a cap, known on the host, on the pages of one request:
 *                     request r gathers min(num_pages[r], max_num_pages)
 *                     pages, so bt_stride must be >= max_num_pages.
 *   out               [out_pages, 128, 128] E4M3 bytes, 16-byte aligned;
 *                     output page page_offsets[r] + j gets logical page j of
 *                     request r.  Nothing else is written.
 *   out_pages         pages in out.
 * Pages whose id is outside [0, num_blocks), or whose output page is outside
 * [0, out_pages), are skipped (nothing read or written for them).
 * num_reqs == 0 or max_num_pages == 0 returns PAGESCORE_OK with no launch;
 * num_reqs above 65,535 is PAGESCORE_EINVAL (one grid row per request).
 */
int nvfp4_index_k_dequant(const uint8_t *kv_cache, int64_t page_stride_bytes,
                          int64_t num_blocks, const int32_t *block_table,
                          int64_t bt_stride, const int32_t *num_pages,
                          const int32_t *page_offsets, int32_t num_reqs,
                          int32_t max_num_pages, uint8_t *out, int64_t out_pages,
                          void *stream);

/*
 * indexer_score_decode -- fused NVFP4 dequantization + decode page scores
 * ([DECODE] module description: the Q8KV4 decode scorer contract; score
 * buffer layout of Nvfp4DecodeCPPlan; own page as in _local_topk_push_kernel;
 * [MOJO] for relu and q_scale; [GATHER] for the key values).
 *
 * For request b (b < num_reqs) with context seq_lens[b] and qlen queries
 * (1 <= qlen <= 8), query i sits in slot 8 - qlen + i at position
 * seq_lens[b] - qlen + i; its own page is position / 128 (none when the
 * position is negative).  Pages 0 .. min((seq_lens[b]-1)/128, width) - 1 are
 * scored.  For score row (slot, head), row = slot*4 + head, and page j below
 * the row's own page:
 *     scores[b, row, j] = max over the page's 128 tokens t of
 *                         relu(q[b, slot, head] . k[t]) * q_scale[b, slot, head]
 * where k[t] is token t of the dequantized page and relu(x) = (x+|x|)/2.
 * The reduction over a page's tokens is the maximum (a reading: the pages do
 * not show the scorer's reduction).  NaN propagates through the maximum.
 *
 *   kv_cache, page_stride_bytes, num_blocks   as for nvfp4_index_k_dequant.
 *   block_table       [num_reqs, bt_stride] int32; bt_stride >= width.
 *   seq_lens          [num_reqs] int32 context lengths (negative counts as 0).
 *   q                 [num_reqs, 8, 4, 128] E4M3 bytes, 16-byte aligned; slots
 *                     below 8 - qlen are not read.
 *   q_scale           [num_reqs, 8, 4] float32; each value must be >= 0 or NaN
 *                     (the page maximum is taken before the multiply, which
 *                     equals the maximum of the products only for such values).
 *   width             score columns per row (>= 1).
 *   scores            [num_reqs, 32, width] float32.  Written only at
 *                     (b, row, j) with j below the row's own page and below
 *                     min((seq_lens[b]-1)/128, width); everything else keeps
 *                     its contents.
 *   row_own           nullable [num_reqs, 32] int32; receives every row's own
 *                     page, or -1 for rows without a query.
 * A page whose block-table id lies outside [0, num_blocks) is not read, and
 * its column of every row keeps its contents.
 * num_reqs == 0 returns PAGESCORE_OK with no launch; at most 65535 requests
 * per call (one grid row per request).
 */
int indexer_score_decode(const uint8_t *kv_cache, int64_t page_stride_bytes,
                         int64_t num_blocks, const int32_t *block_table,
                         int64_t bt_stride, const int32_t *seq_lens,
                         const uint8_t *q, const float *q_scale, int32_t num_reqs,
                         int32_t qlen, int32_t width, float *scores,
                         int32_t *row_own, void *stream);

/*
 * indexer_score_prefill -- lightning-indexer scores ([MOJO] module
 * description):
 *     scores[t, n] = k_scale[n] * sum over h < H of relu(q[t, h] . k[n]) * q_scale[t, h]
 * for every t < T and n < N, with relu(x) = (x+|x|)/2 and no causal mask.
 *
 *   q        [T, H, 128] E4M3 bytes, 16-byte aligned.
 *   q_scale  [T, H] float32.
 *   k        [N, 128] E4M3 bytes, 16-byte aligned.
 *   k_scale  [N] float32.
 *   scores   [T, ld] float32 with ld >= N; columns >= N are not written.
 * T == 0 or N == 0 returns PAGESCORE_OK with no launch; 1 <= H <= 224 (a
 * work-group holds one token's query rows as f16 in 64 KiB of LDS).
 *
 * NVFP4 prefill ([GATHER] module description, the Q8KV8 prefill indexer):
 * nvfp4_index_k_dequant gathers a request's pages into contiguous E4M3 pages,
 * whose first `context` rows are k here with k_scale all ones (the page
 * format has no global scale); topk16_select then keeps each query row's 16
 * best keys.
 */
int indexer_score_prefill(const uint8_t *q, const float *q_scale, const uint8_t *k,
                          const float *k_scale, int32_t T, int32_t H, int32_t N,
                          float *scores, int64_t ld, void *stream);

/*
 * indexer_score_prefill_ragged -- the lightning-indexer scores of a ragged
 * batch of sequences with causal masking and the -inf tail fill ([MOJO]
 * module description: Q over all tokens of a batch, paged K, the mask and
 * the fill as its follow-up steps).
 *
 * Sequence s owns query rows [q_start[s], q_start[s+1]) of q and keys
 * k[k_start[s] .. k_start[s] + k_len[s]).  Its q_len queries are the last
 * q_len tokens of its k_len-token context, so query i (row t = q_start[s]+i)
 * sees count = clamp(k_len - q_len + i + 1, 0, min(k_len, width)) keys, and
 *     scores[t, j] = score(q[t], k[k_start[s] + j])   for j < count
 *     scores[t, j] = -inf                              for count <= j < width
 * with the same score and relu as indexer_score_prefill; columns >= width
 * are not written, and row_len[t] = count when row_len is given (the
 * valid_len of topk16_select for the row).
 *
 *   q, q_scale, k, k_scale  as for indexer_score_prefill (T rows, N keys).
 *   q_start   [num_seqs + 1] int32, non-decreasing row offsets.
 *   k_start, k_len  [num_seqs] int32.
 *   max_q     at least every sequence's q_len (rows past it are not
 *             written).
 *   scores    [T, ld] float32, ld >= width.
 *   row_len   nullable [T] int32.
 * 1 <= H <= PAGESCORE_RAGGED_MAX_HEADS and num_seqs <=
 * PAGESCORE_RAGGED_MAX_SEQS, else PAGESCORE_EINVAL.  T, num_seqs or max_q
 * == 0 returns PAGESCORE_OK with no launch.  Device-side, row offsets are
 * clamped to [0, T] and a key slice leaving k[0, N) is cut to the part
 * inside it.
 */
#define PAGESCORE_RAGGED_MAX_HEADS 64
#define PAGESCORE_RAGGED_MAX_SEQS 65535
int indexer_score_prefill_ragged(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                 const float *k_scale, int32_t T, int32_t H, int32_t N,
                                 int32_t num_seqs, const int32_t *q_start,
                                 const int32_t *k_start, const int32_t *k_len, int32_t max_q,
                                 int32_t width, float *scores, int64_t ld, int32_t *row_len,
                                 void *stream);

/*
 * topk16_select -- exact top-16 column ids of each score row ([MSA] "Changes"
 * and "Behaviour changes vs f380d0e" for the order; [DECODE] module
 * description and _merge_kernel for the 15 + own-page row).
 *
 * Candidates of row r are the columns c < clamp(valid_len[r], 0, width).  They
 * are ranked by score descending where a column with
 * force_begin[r] <= c < force_end[r] counts as +inf, NaN as -inf and -0 as +0;
 * equal values go to the lower column.  The output row holds the first
 * min(k, #candidates) columns in that order, then append_page[r] when
 * append_page is given and append_page[r] >= 0, then -1 up to 16 entries;
 * k = 15 when append_page is given, else 16.
 *
 *   scores         [num_rows, row_stride] float32, row_stride >= width >= 1;
 *                  width above 268,435,456 is PAGESCORE_EINVAL.
 *   valid_len      nullable [num_rows] int32 (NULL: every row has width).
 *   force_begin/force_end  nullable [num_rows] int32 (both or neither).
 *   append_page    nullable [num_rows] int32 (decode: the rows' own pages).
 *   out            [num_rows, out_stride] int32, out_stride >= 16; only the
 *                  first 16 entries of rows < num_rows are written.
 * num_rows == 0 returns PAGESCORE_OK with no launch.
 */
int topk16_select(const float *scores, int64_t row_stride, int32_t num_rows,
                  int32_t width, const int32_t *valid_len,
                  const int32_t *force_begin, const int32_t *force_end,
                  const int32_t *append_page, int32_t *out, int64_t out_stride,
                  void *stream);

/*
 * indexer_prefill_topk16 -- the top-16 key ids of every prefill query row
 * without the score matrix: out[t] is exactly what topk16_select (valid_len,
 * force and append ranges NULL, width N) writes for row t of the scores
 * indexer_score_prefill computes from the same arguments ([MOJO] module
 * description for the scores, which feed a top-k; [MSA] for the order).
 *
 * The scores are never stored: a first pass keeps, per token and block (a
 * block is 32 keys: 1024 j + c + 32 i, i < 32, for block 32 j + c), the
 * largest score, where it occurs and the second largest, in the workspace;
 * a second pass sets a bar that 16 distinct keys of the row reach (so every
 * key of the best 16 does), takes the keys at or above it from the records,
 * recomputing with the identical arithmetic the keys of the rare blocks that
 * hold two such keys, and selects the exact top-16.  Ties in the score make
 * more blocks qualify and cost time, not exactness.
 *
 *   q, q_scale, k, k_scale, T, H, N  as for indexer_score_prefill, with
 *             1 <= H <= PAGESCORE_PREFILL_TOPK_MAX_HEADS and N >= 1.
 *   out       [T, out_stride] int32, out_stride >= 16; the first 16 entries
 *             of every row are written (-1 past the N-th when N < 16).
 *   workspace device memory of at least
 *             indexer_prefill_topk16_workspace(T, N) bytes, 256-byte
 *             aligned, owned by the caller; its contents on entry do not
 *             matter and on return are unspecified.  Calls sharing a
 *             workspace must be ordered (the same stream).
 * T == 0 returns PAGESCORE_OK with no launch.  PAGESCORE_EINVAL for H or N
 * out of range, a null or misaligned pointer, a short out_stride, or a
 * workspace smaller than required.
 */
#define PAGESCORE_PREFILL_TOPK_MAX_HEADS 64
int64_t indexer_prefill_topk16_workspace(int32_t T, int32_t N);
int indexer_prefill_topk16(const uint8_t *q, const float *q_scale, const uint8_t *k,
                           const float *k_scale, int32_t T, int32_t H, int32_t N, int32_t *out,
                           int64_t out_stride, void *workspace, int64_t workspace_bytes,
                           void *stream);

/*
 * indexer_prefill_topk16_noalloc -- indexer_prefill_topk16 for callers that
 * cannot allocate device memory: code under HIP graph capture, allocation-free
 * serving loops, harnesses that forbid allocation.  Same arguments (without
 * the workspace) and the same results; the workspace is instead an array of
 * PAGESCORE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from
 * the library's first use on that GPU until the process ends.
 * PAGESCORE_ENOSPACE when indexer_prefill_topk16_workspace(T, N) exceeds it
 * (nothing is enqueued).  Every call on one GPU uses the same array: calls
 * that can overlap in time on one GPU (different streams or threads) race,
 * so order them, e.g. on one stream.  The array needs no clearing between
 * calls (each call writes what it reads).
 */
#define PAGESCORE_NOALLOC_SCRATCH_BYTES (64u << 20)
int indexer_prefill_topk16_noalloc(const uint8_t *q, const float *q_scale, const uint8_t *k,
                                   const float *k_scale, int32_t T, int32_t H, int32_t N,
                                   int32_t *out, int64_t out_stride, void *stream);

/*
 * mxfp8_e4m3_quantize -- MXFP8 quantization of bf16 rows, the step after the
 * sparse attention ([ROCM] "How it works": output layout and arithmetic).
 * Each block of 32 consecutive elements of a row gets one E8M0 scale byte
 *     sb = clamp(exponent_field(amax) - 8 + (fraction(amax) > 0.75), 0, 254)
 * where amax is the block's largest magnitude compared on the bf16 bit
 * patterns (sb = ceil(log2(amax / 448)) + 127), and each element becomes
 * the E4M3 byte of x * 2^(127 - sb) rounded to nearest even.  Elements that
 * are +-inf or NaN become 0x7F (canonical NaN).
 *
 *   x       [rows, x_stride] bf16 bit patterns, 16-byte aligned, x_stride a
 *           multiple of 8 elements and >= cols.
 *   cols    a multiple of 32.
 *   q       [rows, q_stride] E4M3 bytes, 16-byte aligned, q_stride a multiple
 *           of 16 and >= cols; only the first cols bytes of a row are written.
 *   scales  [rows, scale_stride] E8M0 bytes, scale_stride >= cols / 32;
 *           only the first cols / 32 bytes of a row are written.
 * rows == 0 or cols == 0 returns PAGESCORE_OK with no launch.
 */
int mxfp8_e4m3_quantize(const uint16_t *x, int64_t x_stride, int32_t rows, int32_t cols,
                        uint8_t *q, int64_t q_stride, uint8_t *scales, int64_t scale_stride,
                        void *stream);

/* HIP error code of the most recent PAGESCORE_ELAUNCH on this thread. */
int pagescore_last_hip_error(void);

/* Static description of an error code (never NULL). */
const char *pagescore_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* PAGESCORE_H */
