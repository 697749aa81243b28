// kvbt_bench.hip -- measurement helpers: an empty kernel (launch floor), a plain
// 16-byte grid-stride copy (the reference reading for the HBM byte counters) and a
// read-only stream in the selector's own access pattern (the achievable read ceiling).
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

// One wavefront per 32 KiB segment, read with 16-byte nontemporal buffer loads in
// chunks of 64 lanes x 4 loads, two chunks in flight (the long-row selector's stream),
// folded into a checksum that is stored only if it equals a value it never takes.
constexpr int kSegBytes = 32768;
constexpr int kChunkBytes = 64 * 4 * 16;

__global__ __launch_bounds__(256) void read_kernel(const char* __restrict__ src, int64_t bytes,
                                                   uint32_t* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t seg = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t base = seg * kSegBytes;
    if (base >= bytes) return;
    const int64_t left = bytes - base;
    const int nbytes = left < kSegBytes ? (int)left : kSegBytes;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + base, (short)0, nbytes, 0x00020000);
    constexpr int NC = kSegBytes / kChunkBytes;
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    v4u buf[2][4];
    auto load = [&](int c, v4u (&b)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            b[u] = __builtin_amdgcn_raw_buffer_load_b128(r, c * kChunkBytes + u * 1024 + lane * 16, 0, 2);
    };
    load(0, buf[0]);
    load(1, buf[1]);
    uint32_t acc = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const v4u v = buf[c & 1][u];
            acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
        }
        if (c + 2 < NC) load(c + 2, buf[c & 1]);
    }
    if (acc == 0x9E3779B9u && lane == 0) sink[0] = (uint32_t)seg;
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

extern "C" int kvbt_bench_read(const void* src, int64_t bytes, void* sink, void* stream)
{
    if (src == nullptr || sink == nullptr) return KVBT_E_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)src % 16) != 0) return KVBT_E_RANGE;
    const int64_t segs = (bytes + kSegBytes - 1) / kSegBytes;
    const int64_t blocks = (segs + 3) / 4;
    if (blocks > 0x7FFFFFFF) return KVBT_E_RANGE;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const char*>(src), bytes, static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? KVBT_OK : KVBT_E_LAUNCH;
}
