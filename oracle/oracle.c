/*
 * oracle.c -- plain CPU reference of the page-scoring indexer path.
 *
 * TEST INFRASTRUCTURE ONLY.  Built into liboracle.so and loaded by the test
 * suite, by the smoke check and by the benchmark's CPU-baseline leg.  The
 * product library neither links nor calls anything here, and this file
 * shares no code, header or table with the GPU kernels.
 *
 * Scalar, single-threaded C in double precision.  Every function follows a
 * definition on the source pages:
 *
 *   [GATHER] vLLM API page "vllm.models.minimax_m3.nvidia.ops.gather_nvfp4_index_k":
 *            module description (page layout, dequantization rule) and the
 *            function minimax_m3_gather_nvfp4_index_k_fp8 (gather semantics).
 *   [DECODE] vLLM API page "vllm.models.minimax_m3.nvidia.indexer_nvfp4_decode_cp":
 *            module description (Q8KV4 scorer contract, 15 ranked pages plus
 *            the own page), _local_topk_push_kernel (own page of a query),
 *            _merge_kernel (output row), Nvfp4DecodeCPPlan (score layout).
 *   [MOJO]   Modular page "sparse_index_fp8_sm100": module description
 *            (lightning-indexer score and its branchless relu).
 *   [MSA]    GitHub pull request wolfcomos/MSA #1: "Changes" and "Behaviour
 *            changes" sections (candidate order).
 *   [ROCM]   vLLM pull request #65508 (ROCm MXFP8 epilogue): "How it works",
 *            arithmetic item (E8M0 block scale and E4M3 rounding).
 *
 * Readings taken where the pages leave a step open are marked READING.
 * Parity pins for every function are in the test suite.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PAGE_TOKENS 128
#define DEPTH 128
#define CODE_REGION 8192          /* 128 tokens x 64 code bytes            */
#define PAGE_BYTES 9216           /* codes followed by 128 x 8 scale bytes */
#define SLOTS 8
#define DECODE_HEADS 4
#define DECODE_ROWS (SLOTS * DECODE_HEADS)
#define TOPK 16

/* ------------------------------------------------------------------------
 * Element formats.  The pages name the formats (E2M1 codes, E4M3 scales and
 * outputs) without spelling them out; these are the OCP definitions.
 * ---------------------------------------------------------------------- */

/* OCP MX FP4 E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no
 * inf/NaN.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double ora_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return s ? -mag : mag;
}

/* OCP FP8 E4M3 ("fn" flavour): sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no inf. */
double ora_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7)
        return NAN;
    double mag = (e == 0) ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -mag : mag;
}

/* Encode an exactly representable non-negative E4M3 magnitude. */
static int e4m3_encode_magnitude(double v)
{
    if (v == 0.0)
        return 0;
    if (v < ldexp(1.0, -6))                     /* subnormal: v = m * 2^-9 */
        return (int)(v / ldexp(1.0, -9));
    int ex;
    double f = frexp(v, &ex);                   /* v = f * 2^ex, f in [0.5,1) */
    int unb = ex - 1;                           /* v = (1 + m/8) * 2^unb     */
    int m = (int)((2.0 * f - 1.0) * 8.0);
    return ((unb + 7) << 3) | m;
}

/* e4m3_rn_satfinite(x): round x to the nearest E4M3 value, ties to the
 * even mantissa, finite results beyond +-448 saturate to +-448, NaN gives
 * NaN.  [GATHER] names the rounding and saturation; the rest is the
 * IEEE-style rounding the name states.  READING: the NaN result is the
 * canonical byte 0x7F whatever the sign of x. */
int ora_e4m3_rn_satfinite(double x)
{
    if (isnan(x))
        return 0x7F;
    int sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0)
        return sign | 0x7E;
    double quantum;
    if (a < ldexp(1.0, -6)) {
        quantum = ldexp(1.0, -9);
    } else {
        int ex;
        frexp(a, &ex);                          /* a in [2^(ex-1), 2^ex)     */
        quantum = ldexp(1.0, ex - 1 - 3);
    }
    double n = a / quantum;                     /* exact: power-of-two divide */
    double lo = floor(n);
    double frac = n - lo;
    double r;
    if (frac > 0.5)
        r = lo + 1.0;
    else if (frac < 0.5)
        r = lo;
    else
        r = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;
    double v = r * quantum;                     /* <= 448 because a < 448    */
    return sign | e4m3_encode_magnitude(v);
}

/* ------------------------------------------------------------------------
 * [GATHER] Packed NVFP4 index-K page, 9,216 bytes.  The E2M1 codes of all
 * 128 tokens come first, 64 bytes per token, the lower nibble of a byte
 * holding the earlier element; then the E4M3 block scales, one per 16
 * elements, at index token*8 + group.  There is no global scale.
 * READING: the scale bytes start right after the 8,192 code bytes (the
 * [128, 72] shape is a byte view of the page, not 72-byte token rows).
 * ---------------------------------------------------------------------- */

int ora_page_code(const uint8_t *page, int t, int e)
{
    uint8_t b = page[t * 64 + e / 2];
    return (e & 1) ? (b >> 4) : (b & 15);
}

int ora_page_scale(const uint8_t *page, int t, int e)
{
    return page[CODE_REGION + t * 8 + e / 16];
}

/* Dequantized E4M3 byte of element e of token t: the product of the code
 * and the scale, formed exactly, rounded once ([GATHER]). */
int ora_page_element(const uint8_t *page, int t, int e)
{
    double x = ora_e2m1_value(ora_page_code(page, t, e)) *
               ora_e4m3_value(ora_page_scale(page, t, e));
    return ora_e4m3_rn_satfinite(x);
}

/* The whole page as [128 tokens][128 elements] E4M3 bytes. */
void ora_dequant_page(const uint8_t *page, uint8_t *out)
{
    for (int t = 0; t < PAGE_TOKENS; ++t)
        for (int e = 0; e < DEPTH; ++e)
            out[t * DEPTH + e] = (uint8_t)ora_page_element(page, t, e);
}

/* [GATHER] minimax_m3_gather_nvfp4_index_k_fp8: for every request r and
 * every j below both num_pages[r] and the host bound max_num_pages, the
 * physical page block_table[r][j] is dequantized into output page
 * page_offsets[r] + j.  Output pages are [128, 128] E4M3, contiguous. */
void ora_gather(const uint8_t *kv_cache, int64_t page_stride,
                const int32_t *block_table, int64_t bt_stride,
                const int32_t *num_pages, const int32_t *page_offsets,
                int32_t num_reqs, int32_t max_num_pages, uint8_t *out)
{
    for (int r = 0; r < num_reqs; ++r) {
        int n = num_pages[r] < max_num_pages ? num_pages[r] : max_num_pages;
        for (int j = 0; j < n; ++j) {
            const uint8_t *page = kv_cache + (int64_t)block_table[r * bt_stride + j] * page_stride;
            ora_dequant_page(page, out + ((int64_t)page_offsets[r] + j) * PAGE_TOKENS * DEPTH);
        }
    }
}

/* ------------------------------------------------------------------------
 * Scores.
 * ---------------------------------------------------------------------- */

/* [MOJO] branchless relu, written as the page gives it: (x + |x|) * 0.5.
 * It maps every negative value and -0 to +0 and keeps NaN. */
double ora_relu(double x)
{
    return (x + fabs(x)) * 0.5;
}

/* Exact dot product of two depth-128 E4M3 vectors.  Every E4M3 value is an
 * integer multiple of 2^-9 below 2^9, so every product is a multiple of
 * 2^-18 below 2^18 and every partial sum of 128 of them is below 2^25: 43
 * significant bits, which double holds exactly in any summation order. */
double ora_dot_e4m3(const uint8_t *a, const uint8_t *b)
{
    double acc = 0.0;
    for (int d = 0; d < DEPTH; ++d)
        acc += ora_e4m3_value(a[d]) * ora_e4m3_value(b[d]);
    return acc;
}

/* [DECODE] geometry of query i of a request with qlen queries:
 * position seq_len - qlen + i, query slot 8 - qlen + i, own page
 * position / 128.  READING: a negative position (seq_len < qlen) has no
 * query; its rows keep own page -1 and are never scored. */
int ora_decode_own(int32_t seq_len, int32_t qlen, int slot)
{
    int i = slot - (SLOTS - qlen);
    if (i < 0)
        return -1;
    int64_t pos = (int64_t)seq_len - qlen + i;
    if (pos < 0)
        return -1;
    return (int)(pos / PAGE_TOKENS);
}

/* [DECODE] the scorer covers (seq_len - 1) / 128 pages of a request (all
 * pages below the newest query's own page); none for an empty context. */
int ora_decode_pages(int32_t seq_len)
{
    return seq_len >= 1 ? (seq_len - 1) / PAGE_TOKENS : 0;
}

/* Score of one (request, page j) column for all 32 rows (row = slot*4 +
 * head).  Per row with a query whose own page is above j:
 *     S = max over the page's 128 tokens of relu(q . k_t) * q_scale
 * with NaN propagating through the max.  k_scale is 1: the NVFP4 page has no
 * global or per-token scale ([GATHER]).  READING: the reduction over a
 * page's tokens is the maximum.  Rows that are not stored get NaN in
 * col_out and 0 in stored[]. */
void ora_score_decode_column(const uint8_t *kv_cache, int64_t page_stride,
                             const int32_t *block_table, int64_t bt_stride,
                             const int32_t *seq_lens, const uint8_t *q,
                             const float *q_scale, int32_t qlen, int32_t width,
                             int b, int j, float *col_out, int32_t *stored)
{
    uint8_t k[PAGE_TOKENS * DEPTH];
    int32_t seq = seq_lens[b];
    int n_pages = ora_decode_pages(seq);
    if (n_pages > width)
        n_pages = width;
    int have_page = j < n_pages;
    if (have_page) {
        const uint8_t *page = kv_cache + (int64_t)block_table[(int64_t)b * bt_stride + j] * page_stride;
        ora_dequant_page(page, k);
    }
    for (int slot = 0; slot < SLOTS; ++slot) {
        int own = ora_decode_own(seq, qlen, slot);
        for (int h = 0; h < DECODE_HEADS; ++h) {
            int row = slot * DECODE_HEADS + h;
            col_out[row] = NAN;
            stored[row] = 0;
            if (!have_page || own < 0 || j >= own || j >= width)
                continue;
            const uint8_t *qv = q + (((int64_t)b * SLOTS + slot) * DECODE_HEADS + h) * DEPTH;
            double qs = q_scale[((int64_t)b * SLOTS + slot) * DECODE_HEADS + h];
            double best = 0.0;
            int any = 0, nan = 0;
            for (int t = 0; t < PAGE_TOKENS; ++t) {
                double v = ora_relu(ora_dot_e4m3(qv, k + t * DEPTH)) * qs;
                if (isnan(v))
                    nan = 1;
                else if (!any || v > best) {
                    best = v;
                    any = 1;
                }
            }
            col_out[row] = (float)(nan ? NAN : best);
            stored[row] = 1;
        }
    }
}

/* [DECODE] full decode scorer.  scores is [num_reqs, 32, width]; only the
 * stored entries are written.  row_own (nullable) is [num_reqs, 32] and gets
 * every row's own page or -1. */
void ora_score_decode(const uint8_t *kv_cache, int64_t page_stride,
                      const int32_t *block_table, int64_t bt_stride,
                      const int32_t *seq_lens, const uint8_t *q, const float *q_scale,
                      int32_t num_reqs, int32_t qlen, int32_t width,
                      float *scores, int32_t *row_own)
{
    float col[DECODE_ROWS];
    int32_t st[DECODE_ROWS];
    for (int b = 0; b < num_reqs; ++b) {
        if (row_own)
            for (int slot = 0; slot < SLOTS; ++slot)
                for (int h = 0; h < DECODE_HEADS; ++h)
                    row_own[(int64_t)b * DECODE_ROWS + slot * DECODE_HEADS + h] =
                        ora_decode_own(seq_lens[b], qlen, slot);
        int n_pages = ora_decode_pages(seq_lens[b]);
        if (n_pages > width)
            n_pages = width;
        for (int j = 0; j < n_pages; ++j) {
            ora_score_decode_column(kv_cache, page_stride, block_table, bt_stride, seq_lens,
                                    q, q_scale, qlen, width, b, j, col, st);
            for (int r = 0; r < DECODE_ROWS; ++r)
                if (st[r])
                    scores[((int64_t)b * DECODE_ROWS + r) * width + j] = col[r];
        }
    }
}

/* [MOJO] lightning-indexer score of query token t against key n:
 *     S[t, n] = k_scale[n] * sum over heads h of relu(q[t,h] . k[n]) * q_scale[t,h]
 * Dots exact, the head sum in double, one final rounding to float. */
float ora_score_prefill_one(const uint8_t *q, const float *q_scale,
                            const uint8_t *k, const float *k_scale,
                            int32_t H, int64_t t, int64_t n)
{
    double sum = 0.0;
    for (int h = 0; h < H; ++h) {
        double d = ora_dot_e4m3(q + (t * H + h) * DEPTH, k + n * DEPTH);
        sum += ora_relu(d) * (double)q_scale[t * H + h];
    }
    return (float)((double)k_scale[n] * sum);
}

/* All T x N scores into scores[t * ld + n]. */
void ora_score_prefill(const uint8_t *q, const float *q_scale,
                       const uint8_t *k, const float *k_scale,
                       int32_t T, int32_t H, int32_t N, float *scores, int64_t ld)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n)
            scores[t * ld + n] = ora_score_prefill_one(q, q_scale, k, k_scale, H, t, n);
}

/* Selected rows only: scores[i * N + n] for token rows[i]. */
void ora_score_prefill_rows(const uint8_t *q, const float *q_scale,
                            const uint8_t *k, const float *k_scale,
                            int32_t H, int32_t N, const int64_t *rows, int32_t num,
                            float *scores)
{
    for (int i = 0; i < num; ++i)
        for (int64_t n = 0; n < N; ++n)
            scores[(int64_t)i * N + n] = ora_score_prefill_one(q, q_scale, k, k_scale, H, rows[i], n);
}

/* [MOJO] a ragged batch with causal masking and the -inf tail fill (the
 * module description names both as the follow-up slices of its prefill
 * scorer; its Q is [total tokens, heads, depth] over a batch of sequences
 * with paged K).
 * READING: sequence s owns query rows [q_start[s], q_start[s+1]) and keys
 * k[k_start[s] .. k_start[s] + k_len[s]); its queries are the last
 * q_len = q_start[s+1] - q_start[s] tokens of its k_len-token context, so
 * query i sits at position k_len - q_len + i and sees the keys at positions
 * 0 .. k_len - q_len + i.  Row t = q_start[s] + i holds, for j < width,
 * the score of key k_start[s] + j when j < count, else -inf, where
 * count = clamp(k_len - q_len + i + 1, 0, min(k_len, width)); row_len[t] =
 * count.  Columns >= width are not written. */
int32_t ora_causal_count(int32_t q_len, int32_t k_len, int32_t i, int32_t width)
{
    int64_t c = (int64_t)k_len - q_len + i + 1;
    int64_t hi = k_len < width ? k_len : width;
    if (c > hi)
        c = hi;
    if (c < 0)
        c = 0;
    return (int32_t)c;
}

void ora_score_prefill_ragged(const uint8_t *q, const float *q_scale,
                              const uint8_t *k, const float *k_scale, int32_t H,
                              int32_t num_seqs, const int32_t *q_start,
                              const int32_t *k_start, const int32_t *k_len,
                              int32_t width, float *scores, int64_t ld, int32_t *row_len)
{
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t q_len = q_start[s + 1] - q_start[s];
        for (int32_t i = 0; i < q_len; ++i) {
            int64_t t = (int64_t)q_start[s] + i;
            int32_t count = ora_causal_count(q_len, k_len[s], i, width);
            for (int32_t j = 0; j < width; ++j)
                scores[t * ld + j] =
                    j < count ? ora_score_prefill_one(q, q_scale, k, k_scale, H, t,
                                                      (int64_t)k_start[s] + j)
                              : -INFINITY;
            row_len[t] = count;
        }
    }
}

/* ------------------------------------------------------------------------
 * Top-16.
 * ---------------------------------------------------------------------- */

/* [MSA] the rank value of a candidate column: forced columns count as +inf,
 * NaN as -inf, -0 as +0; everything else is its score. */
double ora_rank_value(float s, int forced)
{
    if (forced)
        return INFINITY;
    if (isnan(s))
        return -INFINITY;
    if (s == 0.0f)
        return 0.0;
    return (double)s;
}

typedef struct {
    double v;
    int32_t col;
} cand_t;

/* Higher rank value first; equal values go to the lower column ([MSA],
 * [DECODE] merge order "score desc, page asc"). */
static int cand_cmp(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->v > b->v)
        return -1;
    if (a->v < b->v)
        return 1;
    return (a->col > b->col) - (a->col < b->col);
}

/* Exact top-k of each row by a full sort.
 *   candidates : columns c < clamp(valid_len[r], 0, width) (valid_len NULL =
 *                width; a length past the buffer ranks what the buffer holds,
 *                [DECODE] _local_topk_push_kernel).
 *   forced     : candidates with force_begin[r] <= c < force_end[r].
 *   k          : 16, or 15 when append_page is given ([DECODE] module
 *                description: 15 ranked pages, then the own page).
 * Output row: the first min(k, #candidates) columns in rank order, then
 * append_page[r] when it is >= 0, then -1 up to 16 entries.
 * READING: a row with fewer than k candidates uses the same rule, so the
 * appended page directly follows the ranked ones. */
void ora_topk16(const float *scores, int64_t row_stride, int32_t num_rows, int32_t width,
                const int32_t *valid_len, const int32_t *force_begin, const int32_t *force_end,
                const int32_t *append_page, int32_t *out, int64_t out_stride)
{
    cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (width > 0 ? (size_t)width : 1));
    for (int64_t r = 0; r < num_rows; ++r) {
        int n = valid_len ? valid_len[r] : width;
        if (n < 0)
            n = 0;
        if (n > width)
            n = width;
        int fb = force_begin ? force_begin[r] : 0;
        int fe = force_end ? force_end[r] : 0;
        for (int i = 0; i < n; ++i) {
            c[i].v = ora_rank_value(scores[r * row_stride + i], i >= fb && i < fe);
            c[i].col = i;
        }
        qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
        int k = append_page ? TOPK - 1 : TOPK;
        int m = n < k ? n : k;
        int32_t *o = out + r * out_stride;
        int pos = 0;
        for (; pos < m; ++pos)
            o[pos] = c[pos].col;
        if (append_page && append_page[r] >= 0)
            o[pos++] = append_page[r];
        for (; pos < TOPK; ++pos)
            o[pos] = -1;
    }
    free(c);
}

/* ------------------------------------------------------------------------
 * [ROCM] MXFP8 E4M3 quantization of bf16 activations ("How it works",
 * arithmetic item): blocks of 32 consecutive elements of a row share one
 * E8M0 scale byte sb, taken from the block's largest magnitude (compared on
 * the bf16 bit patterns with the sign cleared):
 *     sb = clamp(exponent_field(amax) - 8 + (fraction(amax) > 0.75), 0, 254)
 * which is ceil(log2(amax / 448)) + 127 because 448 = 1.75 * 2^8.  Each
 * element is multiplied by 2^(127 - sb) (exact) and rounded to E4M3, nearest
 * with ties to even.
 * READING: an element that is +-inf or NaN quantizes to the canonical NaN
 * byte 0x7F; its bit pattern still takes part in the block maximum.
 * ---------------------------------------------------------------------- */

/* The value of a bf16 bit pattern: sign, 8 exponent bits (bias 127), 7
 * fraction bits; exponent 0 is subnormal (f * 2^-133). */
double ora_bf16_value(int bits)
{
    int s = (bits >> 15) & 1, e = (bits >> 7) & 0xFF, f = bits & 0x7F;
    double mag;
    if (e == 0xFF)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = f * ldexp(1.0, -133);
    else
        mag = (1.0 + f / 128.0) * ldexp(1.0, e - 127);
    return s ? -mag : mag;
}

/* E8M0 byte of one 32-element block. */
int ora_mx_block_scale(const uint16_t *x)
{
    int amax = 0;
    for (int i = 0; i < 32; ++i) {
        int a = x[i] & 0x7FFF;
        if (a > amax)
            amax = a;
    }
    int exponent_field = amax >> 7;
    int fraction_bits = amax & 0x7F;
    int sb = exponent_field - 8 + (fraction_bits / 128.0 > 0.75 ? 1 : 0);
    if (sb < 0)
        sb = 0;
    if (sb > 254)
        sb = 254;
    return sb;
}

/* Quantize rows x [rows, ld_x] bf16 (cols a multiple of 32) into
 * q [rows, ld_q] E4M3 bytes and scales [rows, ld_s] E8M0 bytes. */
void ora_mxfp8_quantize(const uint16_t *x, int64_t ld_x, int32_t rows, int32_t cols,
                        uint8_t *q, int64_t ld_q, uint8_t *scales, int64_t ld_s)
{
    for (int32_t r = 0; r < rows; ++r) {
        for (int32_t b = 0; b < cols / 32; ++b) {
            const uint16_t *blk = x + r * ld_x + 32 * b;
            int sb = ora_mx_block_scale(blk);
            scales[r * ld_s + b] = (uint8_t)sb;
            for (int i = 0; i < 32; ++i) {
                double v = ora_bf16_value(blk[i]);
                uint8_t out;
                if (isnan(v) || isinf(v))
                    out = 0x7F;
                else
                    out = (uint8_t)ora_e4m3_rn_satfinite(v * ldexp(1.0, 127 - sb));
                q[r * ld_q + 32 * b + i] = out;
            }
        }
    }
}
