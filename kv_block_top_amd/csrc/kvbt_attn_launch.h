// kvbt_attn_launch.h -- internal interface between the C-ABI host layer and the
// sparse-attention kernel launcher (kvbt_attn.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvbt {

struct AttnArgs {
    const void* q;             // [T, H*G, 128] bf16
    const void* k_cache;       // [num_pages, H, 16, 16, 8] bf16
    const void* v_cache;       // [num_pages, H, 128, 16] bf16
    int64_t num_pages;
    const int32_t* table;      // [T, H, width]
    int width;
    const int32_t* ctx;        // [T, H]
    int64_t T;
    int H;
    int G;
    float c2;                  // softmax scale times log2(e)
    void* out;                 // [T, H*G, 128] fp32 or bf16
    bool out_bf16;
    int waves;                 // wavefronts per workgroup: 1, 2, 4 or 8
    bool nt;                   // nontemporal page loads (no page shared between rows)
    int rows_per_req;          // rows per request (decode query length)
    // filled by the launcher for the request-grouped kernel (q > 1)
    int group_rows;            // rows per workgroup
    int groups_per_req;        // workgroups per request and KV head
};

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream);

// Whether launch_sparse_attn attends the rows of a request together (and how many rows
// per workgroup, workgroups per request); pure host.
bool attn_group_policy(int64_t T, int H, int G, int q, int* group_rows, int* groups_per_req);

}  // namespace kvbt
