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
};

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
hipError_t launch_table(const TableLaunch& a, hipStream_t stream);

}  // namespace kvbt
