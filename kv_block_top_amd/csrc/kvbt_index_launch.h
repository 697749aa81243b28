// kvbt_index_launch.h -- internal interface between the C-ABI host layer and the
// index-score kernel launcher (kvbt_index.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvbt {

struct IndexArgs {
    const void* q_idx;           // [B*q, H, 128] bf16
    const void* k_cache;         // [num_pages, H, 16, 16, 8] bf16, or [num_pages, H, 8, 16, 16]
                                 // FP8 E4M3 codes
    const float* k_scale;        // FP8 only: [num_pages, H, 16]
    bool fp8;
    int64_t num_pages;
    const int32_t* block_table;  // [B, max_blocks]
    int max_blocks;
    const int32_t* seq_lens;     // [B]
    int B;
    int q;
    int H;
    int M;                       // max_k_tiles (row length of the score buffer)
    int mb;                      // min(max_blocks, M): logical blocks a request can score
    float mul;                   // scale (max) or scale * log2(e) (log-sum-exp)
    bool lse;
    void* scores;                // [B*q, H, M] fp32 or bf16
    bool out_bf16;
};

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream);

}  // namespace kvbt
