// kvbt_index.hip -- decode index-score producer for gfx950 (MI355X): one score per
// (decode row, index head, causal 128-token block) into the decode rows of the unified
// score buffer, the step before the selector.
//
// What the pages fix (vLLM PR #47502 report, "[Minimax-M3] Using tok_sparse_select from
// MSA instead of triton kernels", Implementation breakdown items 1-2, the
// indexer_msa.py module docstring and constants): the decode score kernel writes block
// scores only, for causally valid blocks only, into rows [:nd] of [total_q, H,
// max_k_tiles]; the index-K cache is paged in the same 128-token blocks. The token
// score (scale times the index query-key product per index head) and the block
// reduction (log-sum-exp or max, chosen by the caller) are readings.
//
// Work: one wavefront per (request, index head, logical block), four per workgroup; a
// wavefront scores its block for all the request's decode rows at once. The block's
// keys sit in 8 pages of 16 tokens in the page-16 layout [page][head][D/8][16][8]; per
// page, four v_mfma_f32_16x16x32_bf16 multiply the page's keys (A operand: lane l holds
// token l % 16's dimensions 32s + 8(l / 16) .. + 8, 1 KB contiguous per load
// instruction) by the request's rows' queries (B operand, column n = decode row n of
// the request, zero past q), giving 16 tokens x 16 rows of dot products. Each lane folds
// its 4 tokens per page into a running (max, sum of exp2) per row, masked by the row's
// causal length; lane exchanges combine the four lane groups at the end. Four pages are
// in flight while one is used; key loads are nontemporal (each key is read once). Rows
// that do not reach the block write nothing, so the caller's -inf fill stays.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvbt_device.h"
#include "kvbt_index_launch.h"

namespace kvbt {
namespace {

constexpr int kPageBytes = 16 * 128 * 2;   // one 16-token page of one head
constexpr int kBlockPages = 8;
constexpr int kRing = 4;                   // pages in flight per wavefront
constexpr int kBufferFlags = 0x00020000;
// Every key is read by exactly one wavefront, so key loads are nontemporal: random
// 4 KB pages then stream at the sequential read rate (measured: 6.0 -> 6.8 TB/s for a
// plain page gather; 81 -> 70 us on the 64k-token requests).
constexpr int kLoadNT = 2;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int P>
__device__ __forceinline__ float xor_f(float x)
{
    return __uint_as_float(xor_lane<P>(__float_as_uint(x)));
}

struct KeyPage {
    u32x4 k[4];
};

__device__ __forceinline__ void load_key_page(KeyPage& r, const unsigned char* kc,
                                              int64_t page_stride, int64_t head_off,
                                              uint32_t first_page, bool ok, int j, int lane)
{
    const int64_t off = (int64_t)(first_page + (uint32_t)j) * page_stride + head_off;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(kc + off),
                                                      (short)0, ok ? kPageBytes : 0,
                                                      kBufferFlags);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        r.k[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rk, lane * 16, s * 1024, kLoadNT));
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool LSE, bool OUT_BF16>
__global__ __launch_bounds__(256) void index_scores_kernel(IndexArgs a)
{
    const int lane = lane_id();
    const int64_t wid = (int64_t)blockIdx.x * 4 + uniform((int)(threadIdx.x >> 6));
    const int64_t per_req = (int64_t)a.H * a.mb;
    const int r = uniform((int)(wid / per_req));
    if (r >= a.B) return;
    const int64_t rem = wid - (int64_t)r * per_req;
    const int h = uniform((int)(rem / a.mb));
    const int b = uniform((int)(rem - (int64_t)h * a.mb));
    const int seq = uniform(a.seq_lens[r]);
    // the request's last row sees the most: c = seq_len tokens
    if ((int64_t)b * 128 >= (int64_t)seq) return;

    const int n = lane & 15;
    const int g = lane >> 4;
    // causal tokens of this block for decode row n of the request (0 if none)
    const int64_t cn = (int64_t)seq - a.q + n + 1 - (int64_t)b * 128;
    const int ntok = n < a.q ? (cn < 0 ? 0 : (cn > 128 ? 128 : (int)cn)) : 0;

    const int phys = uniform(a.block_table[(int64_t)r * a.max_blocks + b]);
    const bool ok = phys >= 0 && ((int64_t)phys + 1) * kBlockPages <= a.num_pages;
    const uint32_t first_page = ok ? (uint32_t)phys * kBlockPages : 0u;
    const int64_t page_stride = (int64_t)a.H * kPageBytes;
    const int64_t head_off = (int64_t)h * kPageBytes;
    const unsigned char* kc = (const unsigned char*)a.k_cache;

    // queries of the request's rows for head h as the B operand (zero past row q - 1)
    bf16x8 qb[4];
    {
        const int64_t q0 = ((int64_t)r * a.q * a.H + h) * 256;
        const auto rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void*>((const void*)((const unsigned char*)a.q_idx + q0)), (short)0,
            ((a.q - 1) * a.H + 1) * 256, kBufferFlags);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            qb[k] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rq, n * a.H * 256 + (32 * k + 8 * g) * 2,
                                                   0, 0));
    }

    KeyPage ring[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j)
        load_key_page(ring[j], kc, page_stride, head_off, first_page, ok, j, lane);

    float m = -__builtin_inff();   // running max of this lane's masked scores (log2 units
    float sum = 0.f;               // for LSE), and the sum of exp2(x - m)
#pragma unroll
    for (int j = 0; j < kBlockPages; ++j) {
        floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, ring[j % kRing].k[k]), qb[k], s, 0, 0, 0);
        if (j + kRing < kBlockPages)
            load_key_page(ring[j % kRing], kc, page_stride, head_off, first_page, ok,
                          j + kRing, lane);
        // s[i]: token 16j + 4g + i of the block, decode row n
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[i] = 16 * j + 4 * g + i < ntok ? s[i] * a.mul : -__builtin_inff();
        const float pm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        if constexpr (LSE) {
            const float mn = fmaxf(m, pm);
            if (mn != -__builtin_inff()) {
                float add = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) add += __builtin_amdgcn_exp2f(x[i] - mn);
                sum = sum * __builtin_amdgcn_exp2f(m - mn) + add;
                m = mn;
            }
        } else {
            m = fmaxf(m, pm);
        }
    }
    // combine the four lane groups of each row
    float mall = fmaxf(m, xor_f<16>(m));
    mall = fmaxf(mall, xor_f<32>(mall));
    float result = mall;
    if constexpr (LSE) {
        float part = m == -__builtin_inff() ? 0.f : sum * __builtin_amdgcn_exp2f(m - mall);
        part += xor_f<16>(part);
        part += xor_f<32>(part);
        // log2-sum-exp2 back to natural units
        result = (mall + __builtin_amdgcn_logf(part)) * 0.69314718055994531f;
    }
    if (g != 0 || ntok == 0) return;
    const int64_t e = (((int64_t)r * a.q + n) * a.H + h) * a.M + b;
    if constexpr (OUT_BF16) {
        const __bf16 v = (__bf16)result;
        ((unsigned short*)a.scores)[e] = __builtin_bit_cast(unsigned short, v);
    } else {
        ((float*)a.scores)[e] = result;
    }
}

}  // namespace

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream)
{
    const int64_t waves = (int64_t)a.B * a.H * a.mb;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (a.lse) {
        if (a.out_bf16)
            hipLaunchKernelGGL((index_scores_kernel<true, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((index_scores_kernel<true, false>), grid, block, 0, stream, a);
    } else {
        if (a.out_bf16)
            hipLaunchKernelGGL((index_scores_kernel<false, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((index_scores_kernel<false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kvbt
