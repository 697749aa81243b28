/*
 * kvbt_attn.h -- C ABI of libkvbt.so, part 2: sparse paged-attention decode over the
 * page-16 sparse block table, on AMD Instinct MI355X (gfx950).
 *
 * The operation: vLLM PR #47984 report on prhub.com.cn, "[ROCm][MiniMax-M3][Spec
 * Decode] Support speculative decode with AITER sparse PA", Summary and Implementation
 * breakdown items 1-3: the sparse paged attention consumes, per (row, index head), the
 * page-16 sparse block table and the sparse context length that
 * kvbt_build_sparse_block_table writes (decode and speculative-decode rows alike; an
 * empty row attends to nothing). The pages do not print the attention, so what it
 * computes is a set of readings, pinned against plain mathematics and torch rather
 * than against any value the pages print: scaled dot-product attention over exactly
 * the listed tokens (reading A19), KV head h serving index head h and its G query
 * heads (A20), the cache layouts below (A21), empty rows giving zeros and ctx clamped
 * (A22), pages outside the cache reading as zeros (A23), the arithmetic stated below
 * (A24) and a caller-given scale (A25):
 *
 *   for row t, index head h, query head j in [h*G, (h+1)*G):
 *     c = min(max(ctx[t][h], 0), 16 * width)
 *     token i < c is slot i % 16 of page table[t][h][i / 16]
 *     out[t][j] = sum_i softmax_i(scale * <q[t][j], K_i>) V_i      (zeros when c == 0)
 *
 * KV head h of the cache serves index head h and its group of G query heads.
 *
 * Conventions: as in kvbt.h (device pointers, caller-owned buffers, no allocation or
 * synchronization, asynchronous on `stream`, KVBT_* status codes, validation before
 * any HIP call).
 */
#ifndef KVBT_ATTN_H
#define KVBT_ATTN_H

#include <stdint.h>

#include "kvbt.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KVBT_ATTN_HEAD_DIM = 128,      /* the only head dimension */
    KVBT_ATTN_MAX_GROUP = 16,      /* largest number of query heads per KV head */
    KVBT_ATTN_MAX_WIDTH = 128,     /* largest table width (topk 16 x 8 pages) */
    KVBT_ATTN_MAX_SPLITS = 8       /* most workgroups per group (kvbt_sparse_attn_decode_ws) */
};

/*
 * Sparse paged-attention decode.
 *   q           [T, H*G, 128] bf16: query heads of each row, index head h owning heads
 *               h*G .. h*G + G - 1.
 *   k_cache     [num_pages, H, 16, 16, 8] bf16: keys; element (p, h, d / 8, slot, d % 8)
 *               is dimension d of token `slot` of page p for KV head h (each token's 8
 *               consecutive dimensions are 16 contiguous bytes).
 *   v_cache     [num_pages, H, 128, 16] bf16: values; element (p, h, d, slot).
 *               A page of one KV head is 4 KB of K and 4 KB of V.
 *   table       [T, H, width] int32 page ids (kvbt_build_sparse_block_table's out_table,
 *               width = topk * 8). Only entries below cdiv(c, 16) are used; a page id
 *               outside [0, num_pages) reads as zero keys and zero values.
 *   ctx         [T, H] int32 sparse context length (out_ctx); clamped to
 *               [0, 16 * width] on the device.
 *   decode_query_len  rows per request (>= 1; the spec-decode page passes it to its
 *               sparse PA): consecutive groups of that many rows (the last group may be
 *               cut short by T) are one request's speculative rows, which list mostly
 *               the same pages. With 1, every row is attended alone and its pages
 *               stream past the caches. With more, when the batch is large enough
 *               (kvbt_sparse_attn_grouped), the rows of a request (up to 4, and up to
 *               32 query heads in all) are attended together, each distinct page their
 *               lists name read once for all of them; otherwise every row is attended
 *               alone with its pages kept cacheable, so that the rows of a request find
 *               them in L2. Any value gives results of the definition for any table,
 *               within the same error bound; the rounding order depends on the kernel.
 *   scale       softmax scale (finite), e.g. 1 / sqrt(128).
 *   out         [T, H*G, 128], fp32 (out_dtype KVBT_F32) or bf16 (KVBT_BF16, rounded
 *               to nearest even). Every element is written.
 *   waves       wavefronts sharing one (row, index head): 0 (the library's choice,
 *               kvbt_sparse_attn_waves), 1, 2, 4 or 8. It changes the rounding order
 *               only.
 * Arithmetic: q.K products exact, summed in fp32; probabilities rounded to bf16 for the
 * V product (their fp32 sum uses the same rounded values); fp32 accumulation.
 * Requires T >= 0, H >= 1, 1 <= G <= 16, head_dim == 128, num_pages >= 0,
 * 1 <= width <= 128, decode_query_len >= 1, T * H < 2^31, and a launch below 2^32
 * work-items (64 x waves threads per (row, head) or per group of a request's rows).
 * Returns KVBT_OK, KVBT_E_NULL, KVBT_E_RANGE, KVBT_E_DTYPE (out_dtype) or KVBT_E_LAUNCH.
 */
int kvbt_sparse_attn_decode(const void* q, int64_t T, int H, int G, int head_dim,
                            const void* k_cache, const void* v_cache, int64_t num_pages,
                            const int32_t* table, int width, const int32_t* ctx,
                            int decode_query_len, float scale, void* out, int out_dtype,
                            int waves, void* stream);

/*
 * The same call with a caller's workspace, which lets a batch of few (row, index head)
 * pairs, which would leave most compute units idle, split every pair over several
 * workgroups: each streams a contiguous share of the row's page list, and the last of
 * them to finish merges their partial (max, sum, O) results in a fixed order. This
 * widens the interface the pages describe (they give the sparse PA no workspace); the
 * results are those of the definition above within the same error bound, and do not
 * depend on which workgroup finishes last. A split attends every row alone (pages
 * cacheable when decode_query_len > 1, so that a request's rows meet in L2). Arguments
 * as kvbt_sparse_attn_decode, plus:
 *   splits           0: the library's choice (a split when the batch has fewer than 160
 *                    (row, index head) pairs and the workspace holds it: 4 workgroups
 *                    per pair up to 64 pairs, else 2); 1: never
 *                    (the workspace is not touched; exactly kvbt_sparse_attn_decode);
 *                    2 .. KVBT_ATTN_MAX_SPLITS: that many workgroups per pair for any
 *                    batch, KVBT_E_RANGE when the workspace is smaller than
 *                    kvbt_sparse_attn_workspace_bytes gives or the batch is too large
 *                    for the split (T * H * splits * 520 partial-result slots of 16
 *                    bytes from 2^31 on).
 *   waves            as for kvbt_sparse_attn_decode; 0 with a split means 4.
 *   workspace        device buffer of workspace_bytes bytes, 16-byte aligned, owned by
 *                    the caller; may be NULL when workspace_bytes is 0. It must be all
 *                    zeros before its first use. A completed call leaves the first 16
 *                    bytes of every 256-byte line of it zero again (its arrival counters)
 *                    and partial results in the rest, which no call reads before writing
 *                    them, so it needs no clearing between calls of any batch shape (or
 *                    between replays of a captured graph). It is not interchangeable with
 *                    the selector's workspace, which must be all zeros. Calls that may run
 *                    at the same time must not share a workspace (on one stream they never
 *                    do).
 * Returns as kvbt_sparse_attn_decode, and KVBT_E_NULL or KVBT_E_RANGE for the workspace
 * (negative size, NULL with a size, not 16-byte aligned) or splits outside [0, 8].
 */
int kvbt_sparse_attn_decode_ws(const void* q, int64_t T, int H, int G, int head_dim,
                               const void* k_cache, const void* v_cache, int64_t num_pages,
                               const int32_t* table, int width, const int32_t* ctx,
                               int decode_query_len, float scale, void* out, int out_dtype,
                               int waves, int splits, void* workspace, int64_t workspace_bytes,
                               void* stream);

/* Workgroups per (row, index head) kvbt_sparse_attn_decode_ws splits over for T rows,
 * H index heads, `splits` and a workspace of workspace_bytes (pure host): 0 when it
 * does not split (it then runs as kvbt_sparse_attn_decode). */
int kvbt_sparse_attn_splits(int64_t T, int H, int splits, int64_t workspace_bytes);

/* Workspace bytes kvbt_sparse_attn_decode_ws uses for T rows, H index heads and
 * `splits` when given enough (pure host): 0 when it does not split, KVBT_E_RANGE for
 * splits outside [0, 8] or T * H past 2^31. */
int64_t kvbt_sparse_attn_workspace_bytes(int64_t T, int H, int splits);

/* 1 when kvbt_sparse_attn_decode attends the rows of each request together for this
 * batch shape: decode_query_len > 1, 1 <= G <= 16 and at least 256 (request, KV head)
 * workgroups of up to 4 rows and 32 query heads, one per compute unit (pure host;
 * 0 otherwise). */
int kvbt_sparse_attn_grouped(int64_t T, int H, int G, int decode_query_len);

/* The wavefront count kvbt_sparse_attn_decode uses for `waves` = 0 (pure host): 8 for
 * rows attended alone with decode_query_len 1 (no page shared between rows) and for
 * fewer than 128 (row, index head) pairs, else 4. */
int kvbt_sparse_attn_waves(int64_t T, int H, int decode_query_len);

#ifdef __cplusplus
}
#endif

#endif /* KVBT_ATTN_H */
