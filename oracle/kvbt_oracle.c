/*
 * kvbt_oracle.c -- CPU oracle for the top-k KV-block selector and the page-16
 * sparse block table.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's
 * CPU-baseline leg call this code; the product path (the HIP library) never does,
 * and this file shares no source with it.
 *
 * It is plain and slow on purpose:
 *   - every (row, head) is fully sorted with qsort, under a comparator written
 *     from the clauses of IEEE 754 totalOrder (not from a bit trick);
 *   - the table is built by appending pages block by block in ascending block id.
 *
 * Sources (page titles as printed on prhub.com.cn, sections translated):
 *   [U] "[Minimax-M3] Using tok_sparse_select from MSA instead of triton kernels"
 *       (vLLM PR #47502 report): Implementation breakdown items 2-5, and the
 *       indexer_msa.py module docstring and metadata field comments in Key source
 *       snippets.
 *   [S] "[ROCm][Perf] Tune MiniMax-M3 decode top-k for short contexts"
 *       (vLLM PR #55235 report): Summary and Review highlights (a CPU total-order
 *       reference covering NaN, +-Inf, signed zero and ties).
 *   [D] "[ROCm][MiniMax-M3][Spec Decode] Support speculative decode with AITER
 *       sparse PA" (vLLM PR #47984 report): Implementation breakdown items 1 and 3,
 *       and both Key source snippets (the spec-decode table builder and its test).
 *
 * Readings where the pages are silent are stated next to the code that takes them.
 * Status of pins: every exported function is pinned by the CPU tests (brute force,
 * closed forms, the worked example of [D], a library special case, invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* One 128-token KV block per score tile; one physical block holds eight 16-token
 * pages ([U] indexer_msa.py: page size == sparse block size == index-K block;
 * [D] builds a page-16 table from the 128-token block table). */
#define TOKENS_PER_BLOCK 128
#define TOKENS_PER_PAGE 16
#define PAGES_PER_BLOCK (TOKENS_PER_BLOCK / TOKENS_PER_PAGE)

/* -------------------------------------------------------------------------- */
/* IEEE 754 totalOrder on binary32 data                                        */
/* -------------------------------------------------------------------------- */

/*
 * Three-way totalOrder comparison of two binary32 data given by their bits:
 * returns -1 if x is ordered below y, +1 if above, 0 if they are the same datum.
 * Written from the clauses of IEEE 754 (2008/2019) section 5.10:
 *   (a) numerically smaller orders below numerically larger;
 *   (b) -0 orders below +0;
 *   (c) a negative-signed NaN orders below every non-NaN, a positive-signed NaN
 *       above every non-NaN;
 *   (d) between NaNs: negative sign below positive; for positive NaNs signalling
 *       below quiet and smaller payload below larger; for negative NaNs reversed.
 * Binary formats have no cohorts, so two non-NaN data that are numerically equal
 * and have the same sign are the same datum.
 * The bf16 scores are widened to binary32 by appending 16 zero bits, which is
 * exact and keeps this order (the extra bits are zero for every operand).
 */
int kvbt_oracle_total_order_cmp(uint32_t xb, uint32_t yb)
{
    float xf, yf;
    memcpy(&xf, &xb, sizeof xf);
    memcpy(&yf, &yb, sizeof yf);
    const int x_nan = isnan(xf), y_nan = isnan(yf);
    const int x_neg = (int)(xb >> 31), y_neg = (int)(yb >> 31);

    if (!x_nan && !y_nan) {
        const double x = (double)xf, y = (double)yf;   /* exact widening */
        if (x < y) return -1;                           /* clause (a) */
        if (x > y) return 1;
        if (x_neg != y_neg) return x_neg ? -1 : 1;      /* clause (b): -0 < +0 */
        return 0;
    }
    if (x_nan && !y_nan) return x_neg ? -1 : 1;         /* clause (c) */
    if (!x_nan && y_nan) return y_neg ? 1 : -1;
    /* both NaN: clause (d) */
    if (x_neg != y_neg) return x_neg ? -1 : 1;
    /* The 23-bit fraction field holds the quiet bit on top of the payload, so
     * comparing it as an integer orders signalling below quiet, then by payload. */
    const uint32_t xf_field = xb & 0x007FFFFFu, yf_field = yb & 0x007FFFFFu;
    if (xf_field == yf_field) return 0;
    const int c = xf_field < yf_field ? -1 : 1;
    return x_neg ? -c : c;
}

/* -------------------------------------------------------------------------- */
/* Selector: one (row, head)                                                   */
/* -------------------------------------------------------------------------- */

typedef struct {
    int32_t block;   /* KV block id = tile index within the row */
    int forced;      /* init or local block */
    uint32_t bits;   /* score widened to binary32 */
} cand_t;

/*
 * Rank order of two candidates, for qsort (negative = a comes first):
 *   1. forced blocks before every scored block ([U] docstring: the init and local
 *      blocks are force-included). Reading: they rank above any score, +NaN
 *      included, and among themselves by ascending block id;
 *   2. scored blocks by totalOrder of their score, descending ([S]);
 *   3. equal scores (the same datum) by ascending block id ([S]: ties go to the
 *      lower block).
 */
static int cand_rank_cmp(const void* pa, const void* pb)
{
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (a->forced != b->forced) return a->forced ? -1 : 1;
    if (!a->forced) {
        const int c = kvbt_oracle_total_order_cmp(a->bits, b->bits);
        if (c != 0) return -c;
    }
    return (a->block > b->block) - (a->block < b->block);
}

static uint32_t score_bits(const void* scores, int dtype, int64_t offset)
{
    if (dtype == ORACLE_F32) {
        uint32_t u;
        memcpy(&u, (const char*)scores + offset * 4, 4);
        return u;
    }
    uint16_t h;
    memcpy(&h, (const char*)scores + offset * 2, 2);
    return (uint32_t)h << 16;
}

/*
 * Top-k of one (row, head) given its causal block count nvp (already bounded to
 * [0, max_k_tiles]). Candidates are the blocks 0..nvp-1 only: tiles at or past
 * nvp are never read ([U] docstring: each row is bounded by its causal page count).
 * Forced set F = {b < min(num_init, nvp)} U {max(0, nvp - num_local) <= b < nvp}.
 * The whole candidate list is sorted; the first min(topk, nvp) block ids are the
 * output, then -1 up to topk ([U] breakdown item 5: the valid count is
 * min(topk, cdiv(kv_len, 128)), with -1 only in the tail).
 */
static void select_one(const void* scores, int dtype, int64_t row_head, int max_k_tiles,
                       int64_t nvp, int topk, int num_init, int num_local,
                       int32_t* out, cand_t* buf)
{
    const int64_t base = row_head * (int64_t)max_k_tiles;
    for (int64_t b = 0; b < nvp; ++b) {
        buf[b].block = (int32_t)b;
        buf[b].forced = (b < num_init) || (b >= nvp - num_local);
        buf[b].bits = score_bits(scores, dtype, base + b);
    }
    qsort(buf, (size_t)nvp, sizeof(cand_t), cand_rank_cmp);
    for (int r = 0; r < topk; ++r) out[r] = (r < nvp) ? buf[r].block : -1;
}

static int64_t clamp64(int64_t v, int64_t lo, int64_t hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

static int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

/*
 * Standalone selector over rows [t_begin, t_end).
 * scores: [T, H, max_k_tiles] fp32 (dtype 0) or bf16 bits (dtype 1), token-major.
 * num_valid_pages: [T] causal page counts; each is bounded to [0, max_k_tiles].
 * out_idx: [T, H, topk] int32, token-major ([U] breakdown item 4).
 * Returns 0, or -1 if the scratch allocation fails.
 */
int kvbt_oracle_select_topk_blocks(const void* scores, int dtype, int64_t T, int H,
                                   int max_k_tiles, const int32_t* num_valid_pages,
                                   int topk, int num_init, int num_local,
                                   int32_t* out_idx, int64_t t_begin, int64_t t_end)
{
    (void)T;
    cand_t* buf = (cand_t*)malloc(sizeof(cand_t) * (size_t)(max_k_tiles > 0 ? max_k_tiles : 1));
    if (!buf) return -1;
    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t nvp = clamp64(num_valid_pages[t], 0, max_k_tiles);
        for (int h = 0; h < H; ++h) {
            const int64_t rh = t * H + h;
            select_one(scores, dtype, rh, max_k_tiles, nvp, topk, num_init, num_local,
                       out_idx + rh * topk, buf);
        }
    }
    free(buf);
    return 0;
}

/* -------------------------------------------------------------------------- */
/* Row description: request and causal length of each query row                */
/* -------------------------------------------------------------------------- */

/*
 * Request id and causal length c of row t.
 * Decode form (row_req == NULL), from [D]'s spec-decode builder: rows are laid out
 * request-major, req = t / q, local_q = t - req * q, the query sits at absolute
 * position seq_lens[req] - q + local_q, and c = max(position + 1, 0).
 * Explicit form (row_req != NULL), from [D]'s generic builder: the caller gives
 * (req, position) per row. Reading: a request id outside [0, B) describes no
 * request, and the row is treated as padded (c = 0).
 */
static void row_meta(int64_t t, int B, const int32_t* seq_lens, int q,
                     const int32_t* row_req, const int32_t* row_pos,
                     int64_t* req_out, int64_t* c_out)
{
    int64_t req, pos;
    if (row_req == NULL) {
        req = t / q;
        const int64_t local_q = t - req * q;
        pos = (int64_t)seq_lens[req] - q + local_q;
    } else {
        req = row_req[t];
        pos = row_pos[t];
        if (req < 0 || req >= B) {
            *req_out = -1;
            *c_out = 0;
            return;
        }
    }
    *req_out = req;
    *c_out = pos + 1 > 0 ? pos + 1 : 0;
}

/* -------------------------------------------------------------------------- */
/* Page-16 sparse block table: one (row, head)                                 */
/* -------------------------------------------------------------------------- */

static int cmp_i32(const void* a, const void* b)
{
    const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/*
 * Table row and context length of one (row, head), from [D] (breakdown items 1
 * and 3, and the test snippet):
 *   - the kept set S holds each distinct b of idx_row with 0 <= b < min(nvp, max_blocks),
 *     nvp = cdiv(c, 128); -1 entries, blocks past the causal count and repeats are
 *     dropped (reading: the printed test rows hold -1 in the middle and block ids
 *     past the causal count);
 *   - S is walked in ascending block id (reading: positional order, so the only
 *     partly filled block -- the last causal one -- ends the row);
 *   - block b holds t_b = min(128, c - 128 b) visible tokens and contributes the
 *     cdiv(t_b, 16) page-16 ids block_table[req][b] * 8 + j, j = 0.. (reading: a
 *     128-token physical block p holds pages 8p..8p+7; the id is formed in 32-bit
 *     two's complement);
 *   - ctx is the sum of t_b; the row is padded with 0 to topk * 8 entries, and a
 *     row with c == 0 is all zeros with ctx 0 (pinned by [D]'s test: the expected
 *     table starts as zeros and a padded row expects ctx 0).
 */
static void build_one(const int32_t* idx_row, int topk, const int32_t* bt_row,
                      int max_blocks, int64_t c, int32_t* table_row, int32_t* ctx_out)
{
    const int width = topk * PAGES_PER_BLOCK;
    int32_t kept[64];   /* callers reject topk > 64 */
    int n = 0;
    const int64_t nvp = cdiv64(c, TOKENS_PER_BLOCK);
    const int64_t limit = nvp < max_blocks ? nvp : max_blocks;
    for (int k = 0; k < topk; ++k) {
        const int32_t b = idx_row[k];
        if (b < 0 || b >= limit) continue;
        int seen = 0;
        for (int i = 0; i < n; ++i) seen |= (kept[i] == b);
        if (!seen) kept[n++] = b;
    }
    qsort(kept, (size_t)n, sizeof(int32_t), cmp_i32);

    int pos = 0;
    int64_t ctx = 0;
    for (int i = 0; i < n; ++i) {
        const int64_t b = kept[i];
        const int64_t rest = c - (int64_t)TOKENS_PER_BLOCK * b;
        const int64_t t_b = rest < TOKENS_PER_BLOCK ? rest : TOKENS_PER_BLOCK;
        const int64_t pages = cdiv64(t_b, TOKENS_PER_PAGE);
        const uint32_t phys = (uint32_t)bt_row[b];
        for (int64_t j = 0; j < pages; ++j)
            table_row[pos++] = (int32_t)(phys * (uint32_t)PAGES_PER_BLOCK + (uint32_t)j);
        ctx += t_b;
    }
    while (pos < width) table_row[pos++] = 0;
    *ctx_out = (int32_t)ctx;
}

/*
 * Standalone table builder over rows [t_begin, t_end).
 * idx: [T, H, topk] block ids (any values; see build_one for which are kept).
 * block_table: [B, max_blocks] 128-token physical block ids.
 * Row description: decode form (seq_lens [B], q = decode_query_len, row_req NULL)
 * or explicit form (row_req, row_pos [T] each).
 * out_table: [T, H, topk * 8]; out_ctx: [T, H].
 */
int kvbt_oracle_build_sparse_block_table(const int32_t* idx, int64_t T, int H, int topk,
                                         const int32_t* block_table, int B, int max_blocks,
                                         const int32_t* seq_lens, int decode_query_len,
                                         const int32_t* row_req, const int32_t* row_pos,
                                         int32_t* out_table, int32_t* out_ctx,
                                         int64_t t_begin, int64_t t_end)
{
    (void)T;
    if (topk > 64) return -1;
    for (int64_t t = t_begin; t < t_end; ++t) {
        int64_t req, c;
        row_meta(t, B, seq_lens, decode_query_len, row_req, row_pos, &req, &c);
        for (int h = 0; h < H; ++h) {
            const int64_t rh = t * H + h;
            build_one(idx + rh * topk, topk,
                      req >= 0 ? block_table + req * (int64_t)max_blocks : NULL,
                      req >= 0 ? max_blocks : 0, c,
                      out_table + rh * (int64_t)topk * PAGES_PER_BLOCK, out_ctx + rh);
        }
    }
    return 0;
}

/*
 * Selector followed by the table build, over rows [t_begin, t_end). The causal
 * block count of each row comes from its row description: nvp = cdiv(c, 128)
 * ([U] metadata comment: cdiv(seq_pos + 1, PAGE_SIZE)), bounded to max_k_tiles.
 * out_idx: [T, H, topk]; out_table: [T, H, topk * 8]; out_ctx: [T, H].
 */
int kvbt_oracle_select_topk_and_build_table(
    const void* scores, int dtype, int64_t T, int H, int max_k_tiles,
    const int32_t* block_table, int B, int max_blocks,
    const int32_t* seq_lens, int decode_query_len,
    const int32_t* row_req, const int32_t* row_pos,
    int topk, int num_init, int num_local,
    int32_t* out_idx, int32_t* out_table, int32_t* out_ctx,
    int64_t t_begin, int64_t t_end)
{
    (void)T;
    if (topk > 64) return -1;
    cand_t* buf = (cand_t*)malloc(sizeof(cand_t) * (size_t)(max_k_tiles > 0 ? max_k_tiles : 1));
    if (!buf) return -1;
    for (int64_t t = t_begin; t < t_end; ++t) {
        int64_t req, c;
        row_meta(t, B, seq_lens, decode_query_len, row_req, row_pos, &req, &c);
        const int64_t nvp = clamp64(cdiv64(c, TOKENS_PER_BLOCK), 0, max_k_tiles);
        for (int h = 0; h < H; ++h) {
            const int64_t rh = t * H + h;
            int32_t* idx_row = out_idx + rh * topk;
            select_one(scores, dtype, rh, max_k_tiles, nvp, topk, num_init, num_local,
                       idx_row, buf);
            build_one(idx_row, topk,
                      req >= 0 ? block_table + req * (int64_t)max_blocks : NULL,
                      req >= 0 ? max_blocks : 0, c,
                      out_table + rh * (int64_t)topk * PAGES_PER_BLOCK, out_ctx + rh);
        }
    }
    free(buf);
    return 0;
}
