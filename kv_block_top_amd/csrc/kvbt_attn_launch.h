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
    // each (row, head) split across workgroups (a caller's workspace)
    int splits;                // workgroups per (row, head)
    void* ws;                  // attn_split_bytes(T * H, splits) bytes, 16-byte aligned
};

// Most workgroups one (row, head) is split over.
constexpr int kAttnMaxSplits = 8;

// Launches the per-row kernel, or the request-grouped kernel when attn_group_policy
// takes it (splits and ws are not used).
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream);

// Launches the per-row kernel with each (row, head) split over a.splits workgroups
// (2 .. kAttnMaxSplits) that merge through the workspace a.ws.
hipError_t launch_sparse_attn_split(const AttnArgs& a, hipStream_t stream);

// Workgroups per (row, head) a call with a workspace of workspace_bytes takes for
// `splits` = 0 (the library's choice), 1 (never) or 2 .. kAttnMaxSplits (that many): 0
// for no split, -1 when the requested split does not fit the batch or the workspace.
// When it splits, *bytes is the workspace the launch uses. Pure host.
int attn_split_policy(int64_t T, int H, int splits, int64_t workspace_bytes, int64_t* bytes);

// Workspace bytes of the split launch over `pairs` (row, head) pairs, `splits`
// workgroups each (-1 past the kernel's 32-bit slot index). Pure host.
int64_t attn_split_bytes(int64_t pairs, int splits);

// Whether launch_sparse_attn attends the rows of a request together (and how many rows
// per workgroup, workgroups per request); pure host.
bool attn_group_policy(int64_t T, int H, int G, int q, int* group_rows, int* groups_per_req);

}  // namespace kvbt
