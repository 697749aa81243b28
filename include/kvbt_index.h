/*
 * kvbt_index.h -- C ABI of libkvbt.so, part 3: the decode index-score producer, the
 * step before the selector, on AMD Instinct MI355X (gfx950).
 *
 * What the pages fix (vLLM PR #47502 report on prhub.com.cn, "[Minimax-M3] Using
 * tok_sparse_select from MSA instead of triton kernels": Implementation breakdown items
 * 1-2, the indexer_msa.py module docstring and constants): the decode score kernel
 * writes only block scores -- one per (decode row, index head, 128-token block) -- into
 * the decode rows [:nd] of the unified buffer [total_q, H, max_k_tiles], and only for
 * causally valid blocks (the rest keeps the buffer's -inf fill); the index-K cache is
 * paged in the same 128-token blocks as the sparse blocks.
 *
 * Readings where the pages are silent (pinned against plain mathematics and torch, not
 * against any value the pages print):
 *   - reading A26, token score: scale * <q_idx[t][h], k_idx[token][h]> (one index key
 *     per token and index head);
 *   - reading A27, block score: the log-sum-exp (KVBT_REDUCE_LSE, the log of the
 *     block's share of the softmax mass) or the max (KVBT_REDUCE_MAX) of its causal
 *     tokens' scores -- the pages do not say which reduction their kernel uses;
 *   - reading A28, decode rows: row t = req * q + local_q at position
 *     seq_lens[req] - q + local_q, causal length c = max(position + 1, 0); blocks
 *     b < min(cdiv(c, 128), max_blocks, max_k_tiles) are written, block b covering
 *     tokens 128 b .. min(128 (b + 1), c) - 1;
 *   - reading A29, index-K cache: bf16 [num_pages, H, 16, 16, 8] (16-token pages;
 *     element (p, h, d / 8, slot, d % 8)), physical block p of the block table in pages
 *     8p .. 8p + 7; a block id outside [0, num_pages / 8) reads as zero keys;
 *   - reading A30, arithmetic: as stated at the entry point below;
 *   - reading A31, FP8 index keys (the optional FP8 index cache the pages mention): OCP
 *     FP8 E4M3 codes [num_pages, H, 8, 16, 16] (element (p, h, d / 16, slot, d % 16))
 *     and one float32 scale per (p, h, slot) in k_scale [num_pages, H, 16]; the key is
 *     scale * code.
 *
 * Conventions: as in kvbt.h (device pointers, caller-owned buffers, no allocation or
 * synchronization, asynchronous on `stream`, KVBT_* status codes, validation before
 * any HIP call).
 */
#ifndef KVBT_INDEX_H
#define KVBT_INDEX_H

#include <stdint.h>

#include "kvbt.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { KVBT_REDUCE_LSE = 0, KVBT_REDUCE_MAX = 1 };

enum { KVBT_FP8_E4M3 = 2 };        /* index-key dtype besides KVBT_BF16 */

enum {
    KVBT_INDEX_HEAD_DIM = 128,     /* the only index head dimension */
    KVBT_INDEX_MAX_QUERY_LEN = 16  /* largest decode query length */
};

/*
 * Decode index scores.
 *   q_idx        [B * q, H, 128] bf16 index queries of the decode rows (request-major).
 *   k_cache      [num_pages, H, 16, 16, 8] bf16 index keys, 16-token pages
 *                (key_dtype KVBT_BF16), or [num_pages, H, 8, 16, 16] E4M3 codes
 *                (KVBT_FP8_E4M3) with their scales in k_scale [num_pages, H, 16]
 *                float32 (NULL for bf16 keys).
 *   block_table  [B, max_blocks] int32 128-token physical block per logical block.
 *   seq_lens     [B] int32; q = decode_query_len, 1..16.
 *   scale        finite; reduce KVBT_REDUCE_LSE or KVBT_REDUCE_MAX.
 *   scores       [B * q, H, max_k_tiles], fp32 (score_dtype KVBT_F32) or bf16 (KVBT_BF16,
 *                rounded to nearest even): the decode rows of the unified buffer. Only
 *                the causally valid entries described above are written.
 * Arithmetic: q.k products exact, summed in fp32 (E4M3 codes convert exactly to bf16;
 * the token's scale multiplies its sum); max exact on those sums; log-sum-exp with the
 * hardware exp2/log2 in fp32 around the running max.
 * Requires B >= 0, 1 <= q <= 16, H >= 1, head_dim == 128, num_pages >= 0,
 * max_blocks >= 1, 1 <= max_k_tiles <= 2^24, B * q * H < 2^31, and a launch below
 * 2^32 work-items (one 64-lane wavefront per request, head and block up to
 * min(max_blocks, max_k_tiles)). Returns KVBT_OK,
 * KVBT_E_NULL, KVBT_E_RANGE, KVBT_E_DTYPE (score or key dtype) or KVBT_E_LAUNCH.
 */
int kvbt_index_decode_scores(const void* q_idx, int B, int decode_query_len, int H,
                             int head_dim, const void* k_cache, int key_dtype,
                             const float* k_scale, int64_t num_pages,
                             const int32_t* block_table, int max_blocks,
                             const int32_t* seq_lens, float scale, int reduce, void* scores,
                             int score_dtype, int max_k_tiles, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVBT_INDEX_H */
