// kvbt_bench.hip -- measurement helpers: an empty kernel (launch floor) and a plain
// 16-byte grid-stride copy (achievable HBM bandwidth, and the reference reading for
// the HBM byte counters).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvbt.h"
#include "kvbt_bench.h"

namespace {

__global__ void empty_kernel() {}

__global__ __launch_bounds__(256) void copy_kernel(uint4* __restrict__ dst,
                                                   const uint4* __restrict__ src, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

}  // namespace

extern "C" int kvbt_bench_empty(int blocks, void* stream)
{
    if (blocks < 1 || blocks > (1 << 20)) return KVBT_E_RANGE;
    hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(64), 0, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? KVBT_OK : KVBT_E_LAUNCH;
}

extern "C" int kvbt_bench_copy(void* dst, const void* src, int64_t bytes, void* stream)
{
    if (dst == nullptr || src == nullptr) return KVBT_E_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)dst % 16) != 0 || ((uintptr_t)src % 16) != 0)
        return KVBT_E_RANGE;
    const int64_t n = bytes / 16;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;   // 32 workgroups per compute unit
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<uint4*>(dst), static_cast<const uint4*>(src), n);
    return hipGetLastError() == hipSuccess ? KVBT_OK : KVBT_E_LAUNCH;
}

