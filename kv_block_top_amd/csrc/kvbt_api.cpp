// kvbt_api.cpp -- C-ABI host layer of libkvbt.so: argument validation (before any
// HIP call), the launch policy, and the hand-off to the kernel launchers on the
// caller's stream. No allocation, no copy, no synchronization.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <math.h>

#include "kvbt.h"
#include "kvbt_attn.h"
#include "kvbt_attn_launch.h"
#include "kvbt_index.h"
#include "kvbt_index_launch.h"
#include "kvbt_launch.h"

namespace {

constexpr int64_t kMaxRowHeads = 0x7FFFFFFF;   // grid dimension and 32-bit row ids
// A dispatch packet counts its grid in work-items in a 32-bit field, so workgroups x
// threads per workgroup must stay below 2^32.
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFLL;

bool fits_dispatch(int64_t groups, int64_t threads)
{
    return groups >= 0 && threads > 0 && groups <= kMaxWorkItems / threads;
}
// Rows over 128 blocks take the split path (a workgroup per (row, head), one wavefront
// per chunk) while the whole launch stays within this many wavefronts; beyond it, one
// wavefront per pair was measured faster.
constexpr int64_t kSplitMaxTotalWaves = 256;
constexpr int kSplitMaxWaves = 8;

int split_waves(int mb, int max_k_tiles, int score_dtype)
{
    const int chunk = score_dtype == KVBT_F32 ? 1024 : 2048;
    const int span = mb < max_k_tiles ? mb : max_k_tiles;
    const int waves = (span + chunk - 1) / chunk;
    return waves < kSplitMaxWaves ? waves : kSplitMaxWaves;
}

int pow2_at_least(int64_t x)
{
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

int check_select_common(const void* scores, int score_dtype, int64_t T, int H, int max_k_tiles,
                        int topk, int num_init, int num_local, int max_block,
                        int64_t num_decode_rows, const int32_t* out_idx)
{
    if (num_decode_rows < 0 || num_decode_rows > T) return KVBT_E_RANGE;
    if (score_dtype != KVBT_F32 && score_dtype != KVBT_BF16) return KVBT_E_DTYPE;
    if (T < 0 || H < 1) return KVBT_E_RANGE;
    if (max_k_tiles < 1 || max_k_tiles > KVBT_MAX_K_TILES) return KVBT_E_RANGE;
    if (topk < 1 || topk > KVBT_MAX_TOPK) return KVBT_E_RANGE;
    if (num_init < 0 || num_local < 0 || num_init + num_local > topk) return KVBT_E_RANGE;
    if (max_block < 0 || max_block > max_k_tiles) return KVBT_E_RANGE;
    if (T > kMaxRowHeads / H) return KVBT_E_RANGE;
    if (T > 0 && (scores == nullptr || out_idx == nullptr)) return KVBT_E_NULL;
    return KVBT_OK;
}

// A workspace is 16-byte aligned, and present when it has a size.
int check_workspace(const void* workspace, int64_t workspace_bytes)
{
    if (workspace_bytes < 0) return KVBT_E_RANGE;
    if (workspace_bytes > 0 && workspace == nullptr) return KVBT_E_NULL;
    if (((uintptr_t)workspace % 16) != 0) return KVBT_E_RANGE;
    return KVBT_OK;
}

int check_rows(int64_t T, int B, int max_blocks, const int32_t* block_table,
               const int32_t* seq_lens, int decode_query_len, const int32_t* row_req,
               const int32_t* row_pos)
{
    if (B < 0 || max_blocks < 1) return KVBT_E_RANGE;
    if (row_req == nullptr) {
        if (decode_query_len < 1) return KVBT_E_RANGE;
        if ((int64_t)B * decode_query_len != T) return KVBT_E_SHAPE;
        if (T > 0 && seq_lens == nullptr) return KVBT_E_NULL;
    } else {
        if (T > 0 && row_pos == nullptr) return KVBT_E_NULL;
    }
    if (T > 0 && B > 0 && block_table == nullptr) return KVBT_E_NULL;
    return KVBT_OK;
}

// The cross-workgroup split (path 4): a row's hinted span is cut into chunks of 64
// lanes x 4 loads of 16 bytes, one per wavefront; a slice workgroup takes S of them (a
// power of two up to 8), S chosen so that a row has at most kXSplitTargetSlices slices
// (fewer lists to merge, fewer arrivals on one counter; 8 measured a little faster than
// 4 or 16 on rows of 65536 tiles).
constexpr int kXSplitMaxSlices = 64;
constexpr int kXSplitMaxWaves = 8;
constexpr int kXSplitTargetSlices = 8;
// The library's own choice takes it for batches of at most this many (row, head) pairs
// whose hinted rows span at least kXSplitMinChunks chunks, where the launch without a
// workspace would stream each row with one wavefront (path 1) or one workgroup of
// 8192-tile segments (path 3). Measured on MI355X, graph-replayed, 4 heads, rows at full
// capacity (launch floor 1.58 us): 65536 tiles, 8 rows 7.9 against 9.3 us (fp32) and 8.3
// against 9.6 us (bf16), 1 row 7.7 against 9.2 us; 16384 tiles, 2 rows 7.3 against 7.5
// us; 8192 tiles, 32 rows 7.1 against 7.4 us. Where the workgroup split (path 2) holds a
// row in one compute unit it stays faster (8192 tiles, 1-8 rows: 5.5-5.7 against 6.6
// us: the cross-workgroup merge adds a list store, a counter increment and a list load,
// each a round trip to the point of coherence), and so does one wavefront per row from
// 256 pairs on (16384 tiles, 64 rows: 8.7 against 10.2 us).
constexpr int64_t kXSplitMaxPairs = 128;
constexpr int kXSplitMinChunks = 4;

void xsplit_shape(int mb, int max_k_tiles, int score_dtype, int* chunks, int* waves, int* slices)
{
    const int chunk = score_dtype == KVBT_F32 ? 1024 : 2048;
    const int span = mb < max_k_tiles ? mb : max_k_tiles;
    const int n = (span + chunk - 1) / chunk;
    int S = 1;
    while (S < kXSplitMaxWaves && (n + S - 1) / S > kXSplitTargetSlices) S *= 2;
    const int ns = (n + S - 1) / S;
    *chunks = n;
    *waves = S;
    *slices = ns < kXSplitMaxSlices ? ns : kXSplitMaxSlices;
}

int policy_no_split(int max_block, int max_k_tiles, int score_dtype, int64_t T, int H,
                    int topk, kvbt_policy* out);

}  // namespace

extern "C" {

int kvbt_launch_policy(int max_block, int max_k_tiles, int score_dtype, int64_t T, int H,
                       int topk, kvbt_policy* out)
{
    return kvbt_launch_policy_ws(max_block, max_k_tiles, score_dtype, T, H, topk,
                                 KVBT_SPLIT_NEVER, 0, out);
}

int kvbt_launch_policy_ws(int max_block, int max_k_tiles, int score_dtype, int64_t T, int H,
                          int topk, int split, int64_t workspace_bytes, kvbt_policy* out)
{
    if (out == nullptr) return KVBT_E_NULL;
    if (split != KVBT_SPLIT_AUTO && split != KVBT_SPLIT_ALWAYS && split != KVBT_SPLIT_NEVER)
        return KVBT_E_RANGE;
    if (workspace_bytes < 0) return KVBT_E_RANGE;
    kvbt_policy p;
    const int st = policy_no_split(max_block, max_k_tiles, score_dtype, T, H, topk, &p);
    if (st != KVBT_OK) return st;
    if (split != KVBT_SPLIT_NEVER) {
        const int mb = max_block == 0 ? max_k_tiles : max_block;
        const int elem = score_dtype == KVBT_F32 ? 4 : 2;
        const bool aligned = ((int64_t)max_k_tiles * elem) % 16 == 0;
        int chunks, waves, slices;
        xsplit_shape(mb, max_k_tiles, score_dtype, &chunks, &waves, &slices);
        const int64_t pairs = T * H;
        const int64_t need = kvbt::xsplit_workspace_bytes(pairs, slices);
        // rows past 128 blocks that 16-byte loads can stream
        const bool legal = aligned && mb > KVBT_WAVE_PATH_MAX_BLOCKS &&
                           topk <= KVBT_FAST_TOPK && fits_dispatch(pairs * slices, 64 * waves);
        // the library's choice only where the slices cover the hinted rows (past that,
        // the last slice to arrive streams the rest alone)
        const bool covered = chunks <= (int64_t)slices * waves;
        const bool take = legal && (split == KVBT_SPLIT_ALWAYS ||
                                    (pairs <= kXSplitMaxPairs && chunks >= kXSplitMinChunks &&
                                     covered && (p.path == 1 || p.path == 3) &&
                                     workspace_bytes >= need));
        if (take) {
            if (workspace_bytes < need) return KVBT_E_RANGE;
            p.path = 4;
            p.threads_per_block = 64 * waves;
            p.row_heads_per_block = 1;
            p.grid = pairs * slices;
            p.vec = 16 / elem;
            p.chunks = waves;
            p.slices = slices;
            p.workspace_bytes = need;
        }
    }
    *out = p;
    return KVBT_OK;
}

int64_t kvbt_select_workspace_bytes(int max_block, int max_k_tiles, int score_dtype, int64_t T,
                                    int H, int topk, int split)
{
    kvbt_policy p;
    const int st = kvbt_launch_policy_ws(max_block, max_k_tiles, score_dtype, T, H, topk, split,
                                         INT64_MAX, &p);
    if (st != KVBT_OK) return st;
    return p.workspace_bytes;
}

}  // extern "C"

namespace {

int policy_no_split(int max_block, int max_k_tiles, int score_dtype, int64_t T, int H,
                    int topk, kvbt_policy* out)
{
    if (score_dtype != KVBT_F32 && score_dtype != KVBT_BF16) return KVBT_E_DTYPE;
    if (max_k_tiles < 1 || max_k_tiles > KVBT_MAX_K_TILES) return KVBT_E_RANGE;
    if (max_block < 0 || max_block > max_k_tiles) return KVBT_E_RANGE;
    if (T < 0 || H < 1 || T > kMaxRowHeads / H) return KVBT_E_RANGE;
    if (topk < 1 || topk > KVBT_MAX_TOPK) return KVBT_E_RANGE;
    const int mb = max_block == 0 ? max_k_tiles : max_block;
    const int64_t row_heads = T * H;
    kvbt_policy p;
    if (max_k_tiles > KVBT_FAST_K_TILES) {
        // past the fast path's capacity (path 3): wide keys, a workgroup per (row, head)
        // with one streaming wavefront per 8192-tile segment up to max_block tiles and
        // kvbt::kSegmentMaxWaves of them (wavefront w also takes segments w + S,
        // w + 2S, ... of longer rows); chunks counts chunks per segment
        const int elem = score_dtype == KVBT_F32 ? 4 : 2;
        const bool aligned = ((int64_t)max_k_tiles * elem) % 16 == 0;
        const int span = mb < max_k_tiles ? mb : max_k_tiles;
        const int segs = (span + KVBT_FAST_K_TILES - 1) / KVBT_FAST_K_TILES;
        p.path = 3;
        p.threads_per_block = 64 * (segs < kvbt::kSegmentMaxWaves ? segs : kvbt::kSegmentMaxWaves);
        p.row_heads_per_block = 1;
        p.grid = row_heads;
        p.vec = aligned ? 16 / elem : 1;
        p.chunks = KVBT_FAST_K_TILES / (aligned ? 64 * 4 * p.vec : 64 * 16);
    } else if (mb <= KVBT_WAVE_PATH_MAX_BLOCKS) {
        // one wavefront per (row, head); pack up to four per workgroup once there are
        // enough of them to give every compute unit a workgroup
        int rhpb = 1;
        while (rhpb < 4 && row_heads >= (int64_t)256 * rhpb * 2) rhpb *= 2;
        p.path = 0;
        p.threads_per_block = 64 * rhpb;
        p.row_heads_per_block = rhpb;
        p.grid = (row_heads + rhpb - 1) / rhpb;
        p.vec = 1;
        p.chunks = 2;
    } else if (row_heads * split_waves(mb, max_k_tiles, score_dtype) <= kSplitMaxTotalWaves &&
               ((int64_t)max_k_tiles * (score_dtype == KVBT_F32 ? 4 : 2)) % 16 == 0) {
        // few (row, head) pairs with long rows: a workgroup per (row, head), one
        // wavefront per chunk of 64 lanes x 4 loads of 16 bytes up to max_block tiles
        const int waves = split_waves(mb, max_k_tiles, score_dtype);
        p.path = 2;
        p.threads_per_block = 64 * waves;
        p.row_heads_per_block = 1;
        p.grid = row_heads;
        p.vec = score_dtype == KVBT_F32 ? 4 : 8;
        p.chunks = waves;
    } else {
        // one wavefront per (row, head), four per workgroup; rows stream in chunks of
        // 64 lanes x 4 loads of 16 bytes (64 lanes x 16 single loads when rows are not
        // 16-byte multiples)
        const int elem = score_dtype == KVBT_F32 ? 4 : 2;
        const bool aligned = ((int64_t)max_k_tiles * elem) % 16 == 0;
        p.path = 1;
        p.threads_per_block = 256;
        p.row_heads_per_block = 4;
        p.grid = (row_heads + 3) / 4;
        p.vec = aligned ? 16 / elem : 1;
        const int chunk = aligned ? 64 * 4 * p.vec : 64 * 16;
        p.chunks = pow2_at_least((max_k_tiles + chunk - 1) / chunk);
    }
    if (topk > KVBT_FAST_TOPK) {
        // topk above 16 (path 5): one wavefront per (row, head), four per workgroup, a
        // running top-64 merged column by column
        const int elem = score_dtype == KVBT_F32 ? 4 : 2;
        const bool aligned = ((int64_t)max_k_tiles * elem) % 16 == 0;
        p.path = 5;
        p.threads_per_block = 256;
        p.row_heads_per_block = 4;
        p.grid = (row_heads + 3) / 4;
        p.vec = aligned ? 16 / elem : 1;
        p.chunks = 1;
    }
    if (!fits_dispatch(p.grid, p.threads_per_block)) return KVBT_E_RANGE;
    p.slices = 1;
    p.workspace_bytes = 0;
    *out = p;
    return KVBT_OK;
}

}  // namespace

extern "C" {

int kvbt_select_topk_blocks(const void* scores, int score_dtype, int64_t T, int H,
                            int max_k_tiles, const int32_t* num_valid_pages, int topk,
                            int num_init, int num_local, int max_block,
                            int64_t num_decode_rows, int32_t* out_idx, void* stream)
{
    return kvbt_select_topk_blocks_ws(scores, score_dtype, T, H, max_k_tiles, num_valid_pages,
                                      topk, num_init, num_local, max_block, num_decode_rows,
                                      out_idx, KVBT_SPLIT_NEVER, nullptr, 0, stream);
}

int kvbt_select_topk_blocks_ws(const void* scores, int score_dtype, int64_t T, int H,
                               int max_k_tiles, const int32_t* num_valid_pages, int topk,
                               int num_init, int num_local, int max_block,
                               int64_t num_decode_rows, int32_t* out_idx, int split,
                               void* workspace, int64_t workspace_bytes, void* stream)
{
    int st = check_select_common(scores, score_dtype, T, H, max_k_tiles, topk, num_init,
                                 num_local, max_block, num_decode_rows, out_idx);
    if (st != KVBT_OK) return st;
    if (T > 0 && num_valid_pages == nullptr) return KVBT_E_NULL;
    st = check_workspace(workspace, workspace_bytes);
    if (st != KVBT_OK) return st;
    kvbt::SelectLaunch l = {};
    st = kvbt_launch_policy_ws(max_block, max_k_tiles, score_dtype, T, H, topk, split,
                               workspace_bytes, &l.policy);
    if (st != KVBT_OK) return st;
    if (l.policy.path == 4 && ((uintptr_t)scores % 16) != 0)   // the split reads 16-byte vectors
        st = kvbt_launch_policy_ws(max_block, max_k_tiles, score_dtype, T, H, topk,
                                   KVBT_SPLIT_NEVER, 0, &l.policy);
    if (st != KVBT_OK) return st;
    if (T == 0) return KVBT_OK;
    l.workspace = workspace;
    l.scores = scores;
    l.dtype = score_dtype;
    l.T = T;
    l.H = H;
    l.M = max_k_tiles;
    l.num_valid_pages = num_valid_pages;
    l.q = 1;
    l.num_decode_rows = num_decode_rows;
    l.topk = topk;
    l.num_init = num_init;
    l.num_local = num_local;
    l.out_idx = out_idx;
    l.fused = false;
    return kvbt::launch_select(l, (hipStream_t)stream) == hipSuccess ? KVBT_OK : KVBT_E_LAUNCH;
}

int kvbt_build_sparse_block_table(const int32_t* idx, int64_t T, int H, int topk,
                                  const int32_t* block_table, int B, int max_blocks,
                                  const int32_t* seq_lens, int decode_query_len,
                                  const int32_t* row_req, const int32_t* row_pos,
                                  int32_t* out_table, int32_t* out_ctx, void* stream)
{
    if (T < 0 || H < 1 || T > kMaxRowHeads / H) return KVBT_E_RANGE;
    if (topk < 1 || topk > KVBT_MAX_TOPK) return KVBT_E_RANGE;
    // 16 pairs per 256-thread workgroup (4 for topk above 16)
    if (!fits_dispatch((T * H + 15) / 16 * (topk > KVBT_FAST_TOPK ? 4 : 1), 256)) return KVBT_E_RANGE;
    int st = check_rows(T, B, max_blocks, block_table, seq_lens, decode_query_len, row_req,
                        row_pos);
    if (st != KVBT_OK) return st;
    if (T > 0 && (idx == nullptr || out_table == nullptr || out_ctx == nullptr))
        return KVBT_E_NULL;
    if (T == 0) return KVBT_OK;
    kvbt::TableLaunch l = {};
    l.idx = idx;
    l.T = T;
    l.H = H;
    l.topk = topk;
    l.block_table = block_table;
    l.B = B;
    l.max_blocks = max_blocks;
    l.seq_lens = seq_lens;
    l.q = row_req == nullptr ? decode_query_len : 1;
    l.row_req = row_req;
    l.row_pos = row_pos;
    l.out_table = out_table;
    l.out_ctx = out_ctx;
    return kvbt::launch_table(l, (hipStream_t)stream) == hipSuccess ? KVBT_OK : KVBT_E_LAUNCH;
}

int kvbt_select_topk_and_build_table(const void* scores, int score_dtype, int64_t T, int H,
                                     int max_k_tiles, const int32_t* block_table, int B,
                                     int max_blocks, const int32_t* seq_lens,
                                     int decode_query_len, const int32_t* row_req,
                                     const int32_t* row_pos, int topk, int num_init,
                                     int num_local, int max_block, int64_t num_decode_rows,
                                     int32_t* out_idx, int32_t* out_table, int32_t* out_ctx,
                                     void* stream)
{
    return kvbt_select_topk_and_build_table_ws(
        scores, score_dtype, T, H, max_k_tiles, block_table, B, max_blocks, seq_lens,
        decode_query_len, row_req, row_pos, topk, num_init, num_local, max_block,
        num_decode_rows, out_idx, out_table, out_ctx, KVBT_SPLIT_NEVER, nullptr, 0, stream);
}

}  // extern "C"

namespace {

// The fused call with a caller's workspace, or (static_scratch) with the library's
// scratch array in its place.
int fused_call(const void* scores, int score_dtype, int64_t T, int H, int max_k_tiles,
               const int32_t* block_table, int B, int max_blocks, const int32_t* seq_lens,
               int decode_query_len, const int32_t* row_req, const int32_t* row_pos, int topk,
               int num_init, int num_local, int max_block, int64_t num_decode_rows,
               int32_t* out_idx, int32_t* out_table, int32_t* out_ctx, int split,
               void* workspace, int64_t workspace_bytes, bool static_scratch, void* stream)
{
    int st = check_select_common(scores, score_dtype, T, H, max_k_tiles, topk, num_init,
                                 num_local, max_block, num_decode_rows, out_idx);
    if (st != KVBT_OK) return st;
    st = check_rows(T, B, max_blocks, block_table, seq_lens, decode_query_len, row_req, row_pos);
    if (st != KVBT_OK) return st;
    if (T > 0 && (out_table == nullptr || out_ctx == nullptr)) return KVBT_E_NULL;
    st = check_workspace(workspace, workspace_bytes);
    if (st != KVBT_OK) return st;
    kvbt::SelectLaunch l = {};
    // with the library's scratch, the launch the batch takes with unlimited workspace
    st = kvbt_launch_policy_ws(max_block, max_k_tiles, score_dtype, T, H, topk, split,
                               static_scratch ? INT64_MAX : workspace_bytes, &l.policy);
    if (st != KVBT_OK) return st;
    if (l.policy.path == 4 && ((uintptr_t)scores % 16) != 0)   // the split reads 16-byte vectors
        st = kvbt_launch_policy_ws(max_block, max_k_tiles, score_dtype, T, H, topk,
                                   KVBT_SPLIT_NEVER, 0, &l.policy);
    if (st != KVBT_OK) return st;
    if (static_scratch && l.policy.path == 4 &&
        l.policy.workspace_bytes > KVBT_NOALLOC_SCRATCH_BYTES)
        return KVBT_E_SCRATCH;
    if (T == 0) return KVBT_OK;
    if (static_scratch && l.policy.path == 4) {
        if (kvbt::noalloc_scratch(&workspace) != hipSuccess) return KVBT_E_LAUNCH;
    }
    l.workspace = workspace;
    l.scores = scores;
    l.dtype = score_dtype;
    l.T = T;
    l.H = H;
    l.M = max_k_tiles;
    l.seq_lens = seq_lens;
    l.row_req = row_req;
    l.row_pos = row_pos;
    l.q = row_req == nullptr ? decode_query_len : 1;
    l.B = B;
    l.num_decode_rows = num_decode_rows;
    l.topk = topk;
    l.num_init = num_init;
    l.num_local = num_local;
    l.out_idx = out_idx;
    l.fused = true;
    l.block_table = block_table;
    l.max_blocks = max_blocks;
    l.out_table = out_table;
    l.out_ctx = out_ctx;
    return kvbt::launch_select(l, (hipStream_t)stream) == hipSuccess ? KVBT_OK : KVBT_E_LAUNCH;
}

}  // namespace

extern "C" {

int kvbt_select_topk_and_build_table_ws(const void* scores, int score_dtype, int64_t T, int H,
                                        int max_k_tiles, const int32_t* block_table, int B,
                                        int max_blocks, const int32_t* seq_lens,
                                        int decode_query_len, const int32_t* row_req,
                                        const int32_t* row_pos, int topk, int num_init,
                                        int num_local, int max_block, int64_t num_decode_rows,
                                        int32_t* out_idx, int32_t* out_table, int32_t* out_ctx,
                                        int split, void* workspace, int64_t workspace_bytes,
                                        void* stream)
{
    return fused_call(scores, score_dtype, T, H, max_k_tiles, block_table, B, max_blocks,
                      seq_lens, decode_query_len, row_req, row_pos, topk, num_init, num_local,
                      max_block, num_decode_rows, out_idx, out_table, out_ctx, split, workspace,
                      workspace_bytes, false, stream);
}

int kvbt_select_topk_and_build_table_noalloc(const void* scores, int score_dtype, int64_t T,
                                             int H, int max_k_tiles,
                                             const int32_t* block_table, int B, int max_blocks,
                                             const int32_t* seq_lens, int decode_query_len,
                                             const int32_t* row_req, const int32_t* row_pos,
                                             int topk, int num_init, int num_local,
                                             int max_block, int64_t num_decode_rows,
                                             int32_t* out_idx, int32_t* out_table,
                                             int32_t* out_ctx, int split, void* stream)
{
    return fused_call(scores, score_dtype, T, H, max_k_tiles, block_table, B, max_blocks,
                      seq_lens, decode_query_len, row_req, row_pos, topk, num_init, num_local,
                      max_block, num_decode_rows, out_idx, out_table, out_ctx, split, nullptr, 0,
                      true, stream);
}

int kvbt_sparse_attn_waves(int64_t T, int H, int decode_query_len)
{
    // Eight wavefronts per (row, head) when fewer than 128 pairs leave most compute
    // units without a workgroup, and for rows that share no page (one row per request,
    // pages streamed nontemporally): long-context single rows x 4 heads ran 41.9 against
    // 42.1-44.3 us at 256 pairs, 65.5 against 68.6 us at 384, 169 against 174 us at 1024.
    // Four otherwise: speculative rows of one request meet in L2, and there eight lose
    // 2-4 % from 128 pairs up (the spec-decode table's 512 pairs 53.2-53.5 against 54.3 us,
    // its first 128 rows 26.4 against 27.6 us).
    const int64_t pairs = T * (int64_t)(H > 0 ? H : 1);
    return decode_query_len == 1 || pairs < 128 ? 8 : 4;
}

int kvbt_sparse_attn_grouped(int64_t T, int H, int G, int decode_query_len)
{
    return kvbt::attn_group_policy(T, H, G, decode_query_len, nullptr, nullptr) ? 1 : 0;
}

namespace {

// The sparse-attention call, with a caller's workspace (splits as in
// kvbt_sparse_attn_decode_ws) or without one (splits 1, no workspace).
int attn_call(const void* q, int64_t T, int H, int G, int head_dim, const void* k_cache,
              const void* v_cache, int64_t num_pages, const int32_t* table, int width,
              const int32_t* ctx, int decode_query_len, float scale, void* out, int out_dtype,
              int waves, int splits, void* workspace, int64_t workspace_bytes, void* stream)
{
    if (decode_query_len < 1) return KVBT_E_RANGE;
    if (out_dtype != KVBT_F32 && out_dtype != KVBT_BF16) return KVBT_E_DTYPE;
    if (T < 0 || H < 1 || T > kMaxRowHeads / H) return KVBT_E_RANGE;
    if (G < 1 || G > KVBT_ATTN_MAX_GROUP || head_dim != KVBT_ATTN_HEAD_DIM) return KVBT_E_RANGE;
    if (num_pages < 0 || width < 1 || width > KVBT_ATTN_MAX_WIDTH) return KVBT_E_RANGE;
    if (!isfinite(scale)) return KVBT_E_RANGE;
    if (waves != 0 && waves != 1 && waves != 2 && waves != 4 && waves != 8) return KVBT_E_RANGE;
    if (splits < 0 || splits > kvbt::kAttnMaxSplits) return KVBT_E_RANGE;
    int st = check_workspace(workspace, workspace_bytes);
    if (st != KVBT_OK) return st;
    if (T > 0 && (q == nullptr || table == nullptr || ctx == nullptr || out == nullptr))
        return KVBT_E_NULL;
    if (T > 0 && num_pages > 0 && (k_cache == nullptr || v_cache == nullptr)) return KVBT_E_NULL;
    const int S = T > 0 ? kvbt::attn_split_policy(T, H, splits, workspace_bytes, nullptr) : 0;
    if (S < 0) return KVBT_E_RANGE;
    // four wavefronts per workgroup of a split (its shares are short)
    const int W = waves != 0 ? waves
                             : (S > 0 ? 4 : kvbt_sparse_attn_waves(T, H, decode_query_len));
    {
        // a workgroup of 64 x W threads per (row, head), per group of a request's rows,
        // or per split of a (row, head)
        int gr = 0, gpr = 0;
        const int64_t groups =
            S > 0 ? T * H * S
                  : (kvbt::attn_group_policy(T, H, G, decode_query_len, &gr, &gpr)
                         ? (T + decode_query_len - 1) / decode_query_len * gpr * H
                         : T * H);
        if (!fits_dispatch(groups, 64 * W)) return KVBT_E_RANGE;
    }
    if (T == 0) return KVBT_OK;
    kvbt::AttnArgs a = {};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.num_pages = num_pages > 0x7FFFFFFF ? 0x7FFFFFFF : num_pages;
    a.table = table;
    a.width = width;
    a.ctx = ctx;
    a.T = T;
    a.H = H;
    a.G = G;
    a.c2 = (float)((double)scale * 1.4426950408889634);   // log2(e)
    a.out = out;
    a.out_bf16 = out_dtype == KVBT_BF16;
    a.waves = W;
    a.nt = decode_query_len == 1;
    a.rows_per_req = decode_query_len;
    hipError_t e;
    if (S > 0) {
        a.splits = S;
        a.ws = workspace;
        e = kvbt::launch_sparse_attn_split(a, (hipStream_t)stream);
    } else {
        e = kvbt::launch_sparse_attn(a, (hipStream_t)stream);
    }
    return e == hipSuccess ? KVBT_OK : KVBT_E_LAUNCH;
}

}  // namespace

int kvbt_sparse_attn_decode(const void* q, int64_t T, int H, int G, int head_dim,
                            const void* k_cache, const void* v_cache, int64_t num_pages,
                            const int32_t* table, int width, const int32_t* ctx,
                            int decode_query_len, float scale, void* out, int out_dtype,
                            int waves, void* stream)
{
    return attn_call(q, T, H, G, head_dim, k_cache, v_cache, num_pages, table, width, ctx,
                     decode_query_len, scale, out, out_dtype, waves, 1, nullptr, 0, stream);
}

int kvbt_sparse_attn_decode_ws(const void* q, int64_t T, int H, int G, int head_dim,
                               const void* k_cache, const void* v_cache, int64_t num_pages,
                               const int32_t* table, int width, const int32_t* ctx,
                               int decode_query_len, float scale, void* out, int out_dtype,
                               int waves, int splits, void* workspace, int64_t workspace_bytes,
                               void* stream)
{
    return attn_call(q, T, H, G, head_dim, k_cache, v_cache, num_pages, table, width, ctx,
                     decode_query_len, scale, out, out_dtype, waves, splits, workspace,
                     workspace_bytes, stream);
}

int kvbt_sparse_attn_splits(int64_t T, int H, int splits, int64_t workspace_bytes)
{
    if (T < 1 || H < 1 || T > kMaxRowHeads / H || workspace_bytes < 0) return 0;
    if (splits < 0 || splits > kvbt::kAttnMaxSplits) return 0;
    const int S = kvbt::attn_split_policy(T, H, splits, workspace_bytes, nullptr);
    return S > 0 ? S : 0;
}

int64_t kvbt_sparse_attn_workspace_bytes(int64_t T, int H, int splits)
{
    if (splits < 0 || splits > kvbt::kAttnMaxSplits) return KVBT_E_RANGE;
    if (T < 1 || H < 1) return 0;
    if (T > kMaxRowHeads / H) return KVBT_E_RANGE;
    int64_t need = 0;
    const int S = kvbt::attn_split_policy(T, H, splits, INT64_MAX, &need);
    if (S < 0) return KVBT_E_RANGE;
    return S > 0 ? need : 0;
}

int kvbt_index_decode_scores(const void* q_idx, int B, int decode_query_len, int H,
                             int head_dim, const void* k_cache, int key_dtype,
                             const float* k_scale, int64_t num_pages,
                             const int32_t* block_table, int max_blocks,
                             const int32_t* seq_lens, float scale, int reduce, void* scores,
                             int score_dtype, int max_k_tiles, void* stream)
{
    if (score_dtype != KVBT_F32 && score_dtype != KVBT_BF16) return KVBT_E_DTYPE;
    if (key_dtype != KVBT_BF16 && key_dtype != KVBT_FP8_E4M3) return KVBT_E_DTYPE;
    if (reduce != KVBT_REDUCE_LSE && reduce != KVBT_REDUCE_MAX) return KVBT_E_RANGE;
    if (B < 0 || H < 1 || decode_query_len < 1 || decode_query_len > KVBT_INDEX_MAX_QUERY_LEN)
        return KVBT_E_RANGE;
    if (head_dim != KVBT_INDEX_HEAD_DIM || num_pages < 0 || max_blocks < 1) return KVBT_E_RANGE;
    if (max_k_tiles < 1 || max_k_tiles > KVBT_MAX_K_TILES || !isfinite(scale))
        return KVBT_E_RANGE;
    const int64_t rows = (int64_t)B * decode_query_len;
    if (rows * H > kMaxRowHeads) return KVBT_E_RANGE;
    const int mb = max_blocks < max_k_tiles ? max_blocks : max_k_tiles;
    // one wavefront per (request, head, block), four per 256-thread workgroup
    if (!fits_dispatch(((int64_t)B * H * mb + 3) / 4, 256)) return KVBT_E_RANGE;
    if (B > 0 && (q_idx == nullptr || block_table == nullptr || seq_lens == nullptr ||
                  scores == nullptr))
        return KVBT_E_NULL;
    if (B > 0 && num_pages > 0 && k_cache == nullptr) return KVBT_E_NULL;
    if (B > 0 && num_pages > 0 && key_dtype == KVBT_FP8_E4M3 && k_scale == nullptr)
        return KVBT_E_NULL;
    if (B == 0) return KVBT_OK;
    kvbt::IndexArgs a = {};
    a.q_idx = q_idx;
    a.k_cache = k_cache;
    a.fp8 = key_dtype == KVBT_FP8_E4M3;
    a.k_scale = a.fp8 ? k_scale : nullptr;
    a.num_pages = num_pages > 0x7FFFFFF8 ? 0x7FFFFFF8 : num_pages;
    a.block_table = block_table;
    a.max_blocks = max_blocks;
    a.seq_lens = seq_lens;
    a.B = B;
    a.q = decode_query_len;
    a.H = H;
    a.M = max_k_tiles;
    a.mb = mb;
    a.lse = reduce == KVBT_REDUCE_LSE;
    a.mul = a.lse ? (float)((double)scale * 1.4426950408889634) : scale;
    a.scores = scores;
    a.out_bf16 = score_dtype == KVBT_BF16;
    return kvbt::launch_index_scores(a, (hipStream_t)stream) == hipSuccess ? KVBT_OK
                                                                           : KVBT_E_LAUNCH;
}

const char* kvbt_status_string(int status)
{
    switch (status) {
        case KVBT_OK: return "ok";
        case KVBT_E_NULL: return "a required pointer is NULL";
        case KVBT_E_SHAPE: return "inconsistent sizes (decode form needs T == B * decode_query_len)";
        case KVBT_E_RANGE: return "a size or count is outside its allowed range";
        case KVBT_E_DTYPE: return "unknown score dtype (expected KVBT_F32 or KVBT_BF16)";
        case KVBT_E_LAUNCH: return "the HIP runtime refused the kernel launch";
        case KVBT_E_SCRATCH:
            return "the batch needs more scratch than the allocation-free call holds "
                   "(KVBT_NOALLOC_SCRATCH_BYTES); use the call with a workspace";
        default: return "unknown status";
    }
}

const char* kvbt_version(void) { return "0.1.0"; }

}  // extern "C"
