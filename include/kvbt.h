/*
 * kvbt.h -- C ABI of libkvbt.so: top-k KV-block selector and page-16 sparse block
 * table for block-sparse attention, on AMD Instinct MI355X (gfx950).
 *
 * The operation (sources: vLLM PR report pages on prhub.com.cn):
 *   - "[Minimax-M3] Using tok_sparse_select from MSA instead of triton kernels"
 *     (PR #47502), Implementation breakdown items 2-5 and the indexer_msa.py module
 *     docstring in Key source snippets: one selection pass over a unified token-major
 *     score buffer [total_q, H, max_k_tiles] (one score per 128-token KV block, -inf
 *     in unwritten tiles); each row is bounded by its causal page count
 *     cdiv(position + 1, 128); the init and local blocks are always included; the
 *     output is token-major [T, H, topk]; the valid count of a row is
 *     min(topk, cdiv(kv_len, 128)).
 *   - "[ROCm][Perf] Tune MiniMax-M3 decode top-k for short contexts" (PR #55235),
 *     Summary, Implementation breakdown and Review highlights: a deterministic total
 *     order (NaN, +-Inf and signed zero included; ties to the lower block) and a
 *     launch policy keyed on max_block with its boundary at 128/129 blocks, which
 *     changes only the launch geometry, never the results.
 *   - "[ROCm][MiniMax-M3][Spec Decode] Support speculative decode with AITER sparse
 *     PA" (PR #47984), Implementation breakdown items 1 and 3 and Key source
 *     snippets: the page-16 sparse block table and per-row sparse context length,
 *     for decode rows (row = req * q + local_q, query position
 *     seq_lens[req] - q + local_q, causal length max(position + 1, 0)) and for rows
 *     given explicitly as (request id, absolute position); padded rows give ctx 0.
 *
 * Total order (the fixed rule for special values): IEEE 754 totalOrder on the
 * score, descending: +NaN (larger payload first) > +Inf > positive finite > +0 >
 * -0 > negative finite > -Inf > -NaN. Equal scores (identical bits) go to the lower
 * block id. The forced blocks -- blocks 0 .. num_init-1 and the last num_local
 * causal blocks -- come first, in ascending id, ahead of every scored block.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers to contiguous, row-major arrays of
 *     the stated shape; int32 arrays are int32_t. The caller allocates and owns
 *     every buffer; the library never allocates, frees, copies to the host,
 *     synchronizes or keeps state between calls, so calls may be captured in a HIP
 *     graph.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     asynchronously on it; results are visible after the stream is synchronized.
 *   - Every output element is written on every successful call.
 *   - Return value: KVBT_OK, or a negative KVBT_E_* status. Validation errors are
 *     detected on the host before any HIP call: nothing is launched and the
 *     outputs are left untouched. KVBT_E_LAUNCH reports a failed kernel launch.
 *     Device-side faults (for example a pointer to too small a buffer) surface at
 *     the caller's next synchronization, as usual for HIP.
 *   - Device-side inputs are clamped so that reads stay inside the stated arrays:
 *     causal block counts to [0, max_k_tiles], table block ids to
 *     [0, max_blocks); an explicit row whose request id is outside [0, B) is a
 *     padded row (ctx 0, all-zero table row).
 *   - A launch counts its grid in work-items in 32 bits: a batch whose launch would
 *     need 2^32 work-items or more (workgroups x threads per workgroup, see
 *     kvbt_launch_policy) is a validation error (KVBT_E_RANGE).
 *
 * Beyond the pages' own Python signatures: the launch policy takes max_k_tiles and
 * the score dtype as well as max_block (the pages' policy is keyed on max_block
 * alone), and the select and fused calls take a second hint, num_decode_rows. Both
 * hints change only the launch geometry and visiting order, never the outputs.
 *
 * Two parts of the table are readings, not values the pages print (the PR #47984
 * page's unit test elides the expected table's fill logic; only its zero-filled
 * rows for an empty request are fixed there):
 *   reading A7  -- page order: the kept blocks are listed in ascending block id, so
 *                  the sparse row is the request's dense page-16 list restricted to
 *                  them and the only partial block (the last causal one) ends it;
 *   reading A10 -- partial last block: only its cdiv(t_b, 16) occupied pages are
 *                  listed, and ctx counts exactly its visible tokens.
 */
#ifndef KVBT_H
#define KVBT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KVBT_OK = 0,
    KVBT_E_NULL = -1,    /* a required pointer is NULL */
    KVBT_E_SHAPE = -2,   /* inconsistent sizes (e.g. T != B * q in decode form) */
    KVBT_E_RANGE = -3,   /* a size or count outside its allowed range */
    KVBT_E_DTYPE = -4,   /* unknown score dtype */
    KVBT_E_LAUNCH = -5,  /* the HIP runtime refused the launch */
    KVBT_E_SCRATCH = -6  /* the batch needs more scratch than the allocation-free call holds */
};

enum { KVBT_F32 = 0, KVBT_BF16 = 1 };   /* score dtypes: fp32, or bf16 bit patterns */

enum {
    KVBT_BLOCK_TOKENS = 128,       /* tokens per KV block = per score tile */
    KVBT_PAGE_TOKENS = 16,         /* tokens per page of the sparse table */
    KVBT_PAGES_PER_BLOCK = 8,      /* pages per block */
    KVBT_FAST_K_TILES = 8192,      /* fast-path capacity (1M tokens of context) */
    KVBT_MAX_K_TILES = 1 << 24,    /* largest max_k_tiles: every block an int32 position reaches */
    KVBT_FAST_TOPK = 16,           /* largest topk of launch paths 0-4 */
    KVBT_MAX_TOPK = 64,            /* largest topk (path 5 above 16) */
    KVBT_WAVE_PATH_MAX_BLOCKS = 128, /* max_block at or below this: wave per (row, head) */
    KVBT_NOALLOC_SCRATCH_BYTES = 1 << 20 /* scratch of the allocation-free call, per GPU */
};

/* Launch geometry chosen by kvbt_launch_policy. It never changes results. */
typedef struct kvbt_policy {
    int path;                  /* 0: short-row wavefronts; 1: with the streaming long-row path;
                                  2: split, a workgroup per (row, head); 3: beyond 8192
                                  tiles, a workgroup per (row, head), a wavefront per
                                  8192-tile segment; 4: split across workgroups (workspace
                                  entry points only); 5: topk above 16, a wavefront per
                                  (row, head) */
    int threads_per_block;     /* workgroup size */
    int row_heads_per_block;   /* (row, head) pairs per workgroup */
    int64_t grid;              /* number of workgroups */
    int vec;                   /* score elements per load (paths 1 and 2) */
    int chunks;                /* streaming chunks covering max_k_tiles (path 1; per
                                  8192-tile segment when max_k_tiles > 8192), or
                                  wavefronts per workgroup, one chunk each (path 2) */
    int slices;                /* path 4: workgroups per (row, head); else 1 */
    int64_t workspace_bytes;   /* path 4: workspace bytes the launch uses; else 0 */
} kvbt_policy;

/* Cross-workgroup split (path 4) choice for the *_ws entry points. */
enum {
    KVBT_SPLIT_AUTO = 0,    /* the library's choice: few (row, head) pairs with long rows,
                               when the workspace is large enough */
    KVBT_SPLIT_ALWAYS = 1,  /* whenever the rows can take it (see kvbt_launch_policy_ws) */
    KVBT_SPLIT_NEVER = 2    /* never (the workspace is not touched) */
};

/*
 * Launch policy (pure host, no HIP call). Keyed on max_block, the largest causal
 * block count the caller expects in this batch (0 means max_k_tiles):
 * max_block <= 128 packs up to four short-row wavefronts per workgroup (path 0);
 * 129..8192 adds the streaming path for rows longer than 128 blocks (path 1), one
 * wavefront per (row, head) in both cases (PR #55235, Implementation breakdown item 2:
 * the short-context branch ends at 128 blocks and 129 switches). When rows are 16-byte
 * multiples and the batch is small, rows over 128 blocks are split instead (path 2): a
 * workgroup per pair, one wavefront per chunk of 1024 fp32 or 2048 bf16 tiles up to
 * max_block tiles (at most 8), merged in the workgroup; taken while (row, head) pairs
 * x wavefronts per pair is at most 256. A row
 * longer than max_block is still handled exactly, only less quickly. For paths 1 and 2
 * `vec` assumes a 16-byte-aligned score buffer (otherwise the launch takes path 1 with
 * single-element loads). max_k_tiles above 8192 (the fast path's capacity) always takes
 * path 3: 24-bit block ids in the ranking keys, a workgroup per (row, head) with one
 * streaming wavefront per 8192-tile segment up to max_block tiles and at most 8 of them
 * (wavefront w also takes segments w + 8, w + 16, ... of longer rows), the segments'
 * top-16 merged (`chunks` counts chunks per segment).
 * topk above 16 (up to 64) always takes path 5, the fallback the PR #55235 page keeps for
 * a topk other than 16 (Implementation breakdown item 2): one wavefront per (row,
 * head), four per workgroup, holding the running top-64 one key per lane and merging
 * the row in, 64 elements at a time, wherever they hold a key above the running topk-th.
 * Requires 0 <= max_block <= max_k_tiles and a grid below 2^32 work-items.
 * Returns KVBT_OK, KVBT_E_NULL, KVBT_E_RANGE or KVBT_E_DTYPE.
 */
int kvbt_launch_policy(int max_block, int max_k_tiles, int score_dtype, int64_t T, int H,
                       int topk, kvbt_policy* out);

/*
 * Launch policy of the *_ws entry points (pure host), given the caller's workspace size.
 * Path 4, the cross-workgroup split (PR #55235, Implementation breakdown items 1-2 and
 * the launch-policy snippet: a long row cut into fixed chunks handled by separate
 * workgroups, whose per-chunk top-k lists are merged at the end; Summary and Risks: the
 * merge counter must come back to zero so that graph replays stay correct): one
 * workgroup of S wavefronts per slice, each wavefront taking a chunk of 1024 fp32 or
 * 2048 bf16 tiles up to max_block tiles (S a power of two up to 8, the fewest that leave
 * at most 8 slices per (row, head)), each slice writing its top-16 to the workspace; the
 * last slice of a (row, head) to finish merges them, writes the outputs and clears what
 * it used. Longer rows are finished by that last slice.
 *   split  KVBT_SPLIT_AUTO: path 4 for at most 128 (row, head) pairs whose hinted rows
 *          span at least 4 chunks, where kvbt_launch_policy would take path 1 or 3 and
 *          workspace_bytes covers it; otherwise as kvbt_launch_policy.
 *          KVBT_SPLIT_ALWAYS: path 4 whenever max_block (0 = max_k_tiles) is over 128
 *          blocks and rows are 16-byte multiples (max_k_tiles * score size); a workspace
 *          smaller than it needs is KVBT_E_RANGE.
 *          KVBT_SPLIT_NEVER: exactly kvbt_launch_policy.
 * out->workspace_bytes is what the chosen launch uses (0 when it is not path 4). Returns
 * KVBT_OK, KVBT_E_NULL, KVBT_E_RANGE or KVBT_E_DTYPE.
 */
int kvbt_launch_policy_ws(int max_block, int max_k_tiles, int score_dtype, int64_t T, int H,
                          int topk, int split, int64_t workspace_bytes, kvbt_policy* out);

/*
 * Workspace bytes a *_ws call of this batch shape uses under `split` when given enough
 * (pure host): 0 when it would not take path 4; a negative KVBT_E_* status for invalid
 * arguments. Layout (for reference; the library owns its content): a 32-bit arrival
 * counter per (row, head), each at the start of a 256-byte line of its own, then 16
 * 64-bit keys per (row, head) and slice.
 */
int64_t kvbt_select_workspace_bytes(int max_block, int max_k_tiles, int score_dtype, int64_t T,
                                    int H, int topk, int split);

/*
 * Top-k block selector (PR #47502's selection pass).
 *   scores          [T, H, max_k_tiles] fp32 or bf16 (score_dtype), token-major.
 *                   Tiles at or past a row's causal block count are never read for
 *                   the result (their content does not matter).
 *   num_valid_pages [T] int32: causal block count of each row, cdiv(position+1, 128);
 *                   clamped to [0, max_k_tiles] on the device.
 *   topk            1..64; num_init, num_local >= 0 with num_init + num_local <= topk.
 *                   Above 16 every batch takes launch path 5 (kvbt_launch_policy).
 *   max_block       launch hint (see kvbt_launch_policy), 0..max_k_tiles (0 means
 *                   max_k_tiles); a larger value is KVBT_E_RANGE.
 *   num_decode_rows scheduling hint, 0..T: how many leading rows are decode rows (the
 *                   unified buffer of the PR #47502 page holds the decode rows [:nd]
 *                   ahead of the prefill rows [nd:]: indexer_msa.py module docstring,
 *                   Key source snippets). The streaming launch (path 1) visits those
 *                   rows first, then the others from the last row to the first, so
 *                   that each prefill request's longest rows start early. It never
 *                   changes the outputs; 0 (no decode rows at the head) is always
 *                   correct.
 *   out_idx         [T, H, topk] int32: block ids in rank order, -1 after the
 *                   min(topk, count) valid ones.
 * Requires 1 <= max_k_tiles <= 2^24 (KVBT_MAX_K_TILES: 128-token blocks up to the last
 * an int32 token position reaches), H >= 1, T >= 0, T * H < 2^31,
 * 0 <= num_decode_rows <= T.
 */
int kvbt_select_topk_blocks(const void* scores, int score_dtype, int64_t T, int H,
                            int max_k_tiles, const int32_t* num_valid_pages,
                            int topk, int num_init, int num_local, int max_block,
                            int64_t num_decode_rows, int32_t* out_idx, void* stream);

/*
 * Page-16 sparse block table (PR #47984's builders).
 *   idx          [T, H, topk] int32 block ids (any values: -1, ids at or past the
 *                row's causal block count or max_blocks, and repeats are dropped).
 *   block_table  [B, max_blocks] int32: 128-token physical block ids per request.
 *   Row description, one of:
 *     decode form   (row_req == NULL): seq_lens [B] int32 and decode_query_len q >= 1,
 *                   with T == B * q; row t is request t / q at position
 *                   seq_lens[req] - q + t % q;
 *     explicit form (row_req != NULL): row_req [T] and row_pos [T] int32 (request id
 *                   and absolute position of each row); seq_lens may be NULL.
 *   out_table    [T, H, topk * 8] int32: for the kept blocks in ascending id (reading
 *                A7), block b shows t_b = min(128, c - 128 b) tokens as the
 *                cdiv(t_b, 16) page ids block_table[req][b] * 8 + j (reading A10);
 *                then zeros.
 *   out_ctx      [T, H] int32: sum of t_b over the kept blocks (0 for padded rows).
 * Requires 1 <= topk <= 64, H >= 1, T >= 0, B >= 0, max_blocks >= 1, T * H < 2^31.
 */
int kvbt_build_sparse_block_table(const int32_t* idx, int64_t T, int H, int topk,
                                  const int32_t* block_table, int B, int max_blocks,
                                  const int32_t* seq_lens, int decode_query_len,
                                  const int32_t* row_req, const int32_t* row_pos,
                                  int32_t* out_table, int32_t* out_ctx, void* stream);

/*
 * Fused selector + table in one launch (the selector's EMIT_SPARSE_TABLE mode on
 * the PR #55235 page). The causal block count of each row comes from its row
 * description: min(cdiv(c, 128), max_k_tiles), c = max(position + 1, 0). Outputs
 * are exactly those of kvbt_select_topk_blocks (with that count) followed by
 * kvbt_build_sparse_block_table. Arguments as above.
 */
int kvbt_select_topk_and_build_table(const void* scores, int score_dtype, int64_t T, int H,
                                     int max_k_tiles, const int32_t* block_table, int B,
                                     int max_blocks, const int32_t* seq_lens,
                                     int decode_query_len, const int32_t* row_req,
                                     const int32_t* row_pos, int topk, int num_init,
                                     int num_local, int max_block, int64_t num_decode_rows,
                                     int32_t* out_idx, int32_t* out_table, int32_t* out_ctx,
                                     void* stream);

/*
 * The selector and the fused call with a workspace, for the cross-workgroup split (path
 * 4, kvbt_launch_policy_ws). Arguments as kvbt_select_topk_blocks and
 * kvbt_select_topk_and_build_table, plus:
 *   split            KVBT_SPLIT_AUTO, KVBT_SPLIT_ALWAYS or KVBT_SPLIT_NEVER.
 *   workspace        device buffer of workspace_bytes bytes, 16-byte aligned, owned by
 *                    the caller; may be NULL when workspace_bytes is 0. It must be all
 *                    zeros before its first use; every completed call leaves it all zeros
 *                    again (its counters and the lists it wrote), so it needs no clearing
 *                    between calls of any batch shape (or between replays of a captured
 *                    graph). Calls that may run at the same time must not share a
 *                    workspace (on one stream they never do).
 * The outputs are exactly those of the calls without a workspace. A score buffer that is
 * not 16-byte aligned never takes path 4.
 */
int kvbt_select_topk_blocks_ws(const void* scores, int score_dtype, int64_t T, int H,
                               int max_k_tiles, const int32_t* num_valid_pages, int topk,
                               int num_init, int num_local, int max_block,
                               int64_t num_decode_rows, int32_t* out_idx, int split,
                               void* workspace, int64_t workspace_bytes, void* stream);

int kvbt_select_topk_and_build_table_ws(const void* scores, int score_dtype, int64_t T, int H,
                                        int max_k_tiles, const int32_t* block_table, int B,
                                        int max_blocks, const int32_t* seq_lens,
                                        int decode_query_len, const int32_t* row_req,
                                        const int32_t* row_pos, int topk, int num_init,
                                        int num_local, int max_block, int64_t num_decode_rows,
                                        int32_t* out_idx, int32_t* out_table, int32_t* out_ctx,
                                        int split, void* workspace, int64_t workspace_bytes,
                                        void* stream);

/*
 * The fused call without allocation and without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): kvbt_select_topk_and_build_table_ws with the
 * library's own scratch in place of the caller's workspace. The scratch is one array of
 * KVBT_NOALLOC_SCRATCH_BYTES bytes in device memory per GPU, held until the process
 * ends, zero when the library is loaded and left all zeros by every completed call.
 * Every call on one GPU shares it, so calls that may overlap in time on one GPU (on
 * different streams) race and must not be issued; on one stream they never overlap.
 * Arguments as kvbt_select_topk_and_build_table, plus split (KVBT_SPLIT_*). A batch
 * whose split would need more scratch (kvbt_select_workspace_bytes with workspace
 * unlimited, over KVBT_NOALLOC_SCRATCH_BYTES: only KVBT_SPLIT_ALWAYS on large batches)
 * is refused with KVBT_E_SCRATCH before any HIP call. The library looks up the array's
 * device address on its first call on each device (with that device current) and
 * allocates nothing, ever. Outputs are exactly those of the calls with a workspace.
 */
int kvbt_select_topk_and_build_table_noalloc(const void* scores, int score_dtype, int64_t T,
                                             int H, int max_k_tiles,
                                             const int32_t* block_table, int B, int max_blocks,
                                             const int32_t* seq_lens, int decode_query_len,
                                             const int32_t* row_req, const int32_t* row_pos,
                                             int topk, int num_init, int num_local,
                                             int max_block, int64_t num_decode_rows,
                                             int32_t* out_idx, int32_t* out_table,
                                             int32_t* out_ctx, int split, void* stream);

/* Static English text for a status code. */
const char* kvbt_status_string(int status);

/* Library version, as "major.minor.patch". */
const char* kvbt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVBT_H */
