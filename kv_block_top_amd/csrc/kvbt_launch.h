// kvbt_launch.h -- internal interface between the C-ABI host layer (kvbt_api.cpp)
// and the kernel launchers (kvbt_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvbt.h"

namespace kvbt {

struct SelectLaunch {
    const void* scores;
    int dtype;                 // KVBT_F32 / KVBT_BF16
    int64_t T;
    int H;
    int M;                     // max_k_tiles
    // row description
    const int32_t* num_valid_pages;   // standalone selector only
    const int32_t* seq_lens;
    const int32_t* row_req;
    const int32_t* row_pos;
    int q;
    int B;
    int64_t num_decode_rows;   // leading decode rows (visiting order only)
    // selection
    int topk, num_init, num_local;
    int32_t* out_idx;
    // table (fused call only)
    bool fused;
    const int32_t* block_table;
    int max_blocks;
    int32_t* out_table;
    int32_t* out_ctx;
    kvbt_policy policy;
    void* workspace;           // path 4 only: counters, then the slices' lists
};

// Wavefronts of a path-3 workgroup at most (one per 8192-tile segment; longer rows
// give each wavefront every kSegmentMaxWaves-th segment).
constexpr int kSegmentMaxWaves = 8;

// Workspace layout of the cross-workgroup split (path 4): one 32-bit arrival counter per
// (row, head), each in a 256-byte line of its own (atomics on one line serialize, so
// counters sharing a line would queue every slice of every row behind each other),
// then [row_heads, slices, 16] 64-bit keys (one 128-byte line per slice).
constexpr int kXSplitCounterStride = 64;   // uint32 per counter line

inline int64_t xsplit_counter_bytes(int64_t row_heads)
{
    return row_heads * kXSplitCounterStride * 4;
}

inline int64_t xsplit_workspace_bytes(int64_t row_heads, int slices)
{
    return xsplit_counter_bytes(row_heads) + row_heads * (int64_t)slices * 16 * 8;
}

struct TableLaunch {
    const int32_t* idx;
    int64_t T;
    int H;
    int topk;
    const int32_t* block_table;
    int B;
    int max_blocks;
    const int32_t* seq_lens;
    int q;
    const int32_t* row_req;
    const int32_t* row_pos;
    int32_t* out_table;
    int32_t* out_ctx;
};

hipError_t launch_select(const SelectLaunch& a, hipStream_t stream);

// Device address (on the current device) of the allocation-free call's scratch array,
// KVBT_NOALLOC_SCRATCH_BYTES bytes; looked up on the first call on each device.
hipError_t noalloc_scratch(void** out);
hipError_t launch_table(const TableLaunch& a, hipStream_t stream);

}  // namespace kvbt
