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
// keys sit in 8 pages of 16 tokens in the page-16 layout [page][head][D/8][16][8] (bf16;
// FP8 E4M3 keys: [page][head][D/16][16][16] codes and one float32 scale per token, the
// codes converted exactly to bf16 in registers and the scale applied to each token's
// dot product); per
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

// One 16-token page of one head as this lane holds it. bf16 keys: step s of the score
// MFMA takes dimensions 32s + 8g .. + 8 of token (lane & 15), g = lane >> 4 (four 16-byte
// loads). FP8 keys ([D/16][16][16] codes): load u holds dimensions 64u + 16g .. + 16 of
// the token (two 16-byte loads), which feed steps 2u and 2u + 1; plus the scales of the
// lane's four score tokens 4g .. 4g + 3.
template <bool FP8>
struct KeyPage {
    u32x4 k[FP8 ? 2 : 4];
    u32x4 sc;                    // FP8 only
};

struct KeySrc {
    const unsigned char* kc;     // keys
    const unsigned char* sc;     // FP8 scales [page][head][16] float32
    int64_t page_stride, head_off;          // key bytes
    int64_t scale_stride, scale_head_off;   // scale bytes
    uint32_t first_page;
    bool ok;
};

template <bool FP8>
__device__ __forceinline__ void load_key_page(KeyPage<FP8>& r, const KeySrc& src, int j,
                                              int lane)
{
    constexpr int bytes = FP8 ? kPageBytes / 2 : kPageBytes;
    const int64_t page = (int64_t)(src.first_page + (uint32_t)j);
    const int64_t off = page * src.page_stride + src.head_off;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(src.kc + off),
                                                      (short)0, src.ok ? bytes : 0,
                                                      kBufferFlags);
#pragma unroll
    for (int s = 0; s < (FP8 ? 2 : 4); ++s) {
        r.k[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rk, lane * 16, s * 1024, kLoadNT));
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (FP8) {
        const int64_t so = page * src.scale_stride + src.scale_head_off;
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(src.sc + so), (short)0, src.ok ? 64 : 0, kBufferFlags);
        r.sc = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rs, (lane >> 4) * 16, 0, kLoadNT));
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Eight FP8 E4M3 codes (two dwords) to the bf16x8 MFMA operand; exact (every E4M3 value
// is a bf16 value). The hardware conversion decodes the OCP E4M3 format on gfx950.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi)
{
    bf16x8 r;
    const uint32_t w[2] = {lo, hi};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
        const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
        r[4 * i + 0] = (__bf16)a[0];
        r[4 * i + 1] = (__bf16)a[1];
        r[4 * i + 2] = (__bf16)b[0];
        r[4 * i + 3] = (__bf16)b[1];
    }
    return r;
}

template <bool LSE, bool OUT_BF16, bool FP8>
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
    KeySrc src;
    src.ok = phys >= 0 && ((int64_t)phys + 1) * kBlockPages <= a.num_pages;
    src.first_page = src.ok ? (uint32_t)phys * kBlockPages : 0u;
    src.kc = (const unsigned char*)a.k_cache;
    src.sc = (const unsigned char*)a.k_scale;
    src.page_stride = (int64_t)a.H * (FP8 ? kPageBytes / 2 : kPageBytes);
    src.head_off = (int64_t)h * (FP8 ? kPageBytes / 2 : kPageBytes);
    src.scale_stride = (int64_t)a.H * 64;
    src.scale_head_off = (int64_t)h * 64;

    // queries of the request's rows for head h as the B operand (zero past row q - 1)
    bf16x8 qb[4];
    {
        const int64_t q0 = ((int64_t)r * a.q * a.H + h) * 256;
        const auto rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void*>((const void*)((const unsigned char*)a.q_idx + q0)), (short)0,
            ((a.q - 1) * a.H + 1) * 256, kBufferFlags);
        // step k's dimensions, matching the keys' operand layout above
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int d0 = FP8 ? 64 * (k >> 1) + 16 * g + 8 * (k & 1) : 32 * k + 8 * g;
            qb[k] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rq, n * a.H * 256 + d0 * 2, 0, 0));
        }
    }

    KeyPage<FP8> ring[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) load_key_page<FP8>(ring[j], src, j, lane);

    float m = -__builtin_inff();   // running max of this lane's masked scores (log2 units
    float sum = 0.f;               // for LSE), and the sum of exp2(x - m)
#pragma unroll
    for (int j = 0; j < kBlockPages; ++j) {
        floatx4 s = {0.f, 0.f, 0.f, 0.f};
        float ksc[4] = {1.f, 1.f, 1.f, 1.f};
        const KeyPage<FP8>& kp = ring[j % kRing];
        if constexpr (FP8) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const u32x4& raw = kp.k[k >> 1];
                const bf16x8 kb = (k & 1) ? e4m3x8_to_bf16(raw[2], raw[3])
                                          : e4m3x8_to_bf16(raw[0], raw[1]);
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb[k], s, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) ksc[i] = __uint_as_float(kp.sc[i]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kp.k[k]),
                                                           qb[k], s, 0, 0, 0);
        }
        if (j + kRing < kBlockPages) load_key_page<FP8>(ring[j % kRing], src, j + kRing, lane);
        // s[i]: token 16j + 4g + i of the block, decode row n (times its key scale)
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[i] = 16 * j + 4 * g + i < ntok ? s[i] * ksc[i] * a.mul : -__builtin_inff();
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

template <bool LSE, bool OUT_BF16>
void launch_k(const IndexArgs& a, dim3 grid, hipStream_t stream)
{
    if (a.fp8)
        hipLaunchKernelGGL((index_scores_kernel<LSE, OUT_BF16, true>), grid, dim3(256), 0, stream,
                           a);
    else
        hipLaunchKernelGGL((index_scores_kernel<LSE, OUT_BF16, false>), grid, dim3(256), 0,
                           stream, a);
}

}  // namespace

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream)
{
    const int64_t waves = (int64_t)a.B * a.H * a.mb;
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (a.lse) {
        if (a.out_bf16) launch_k<true, true>(a, grid, stream);
        else launch_k<true, false>(a, grid, stream);
    } else {
        if (a.out_bf16) launch_k<false, true>(a, grid, stream);
        else launch_k<false, false>(a, grid, stream);
    }
    return hipGetLastError();
}

}  // namespace kvbt
