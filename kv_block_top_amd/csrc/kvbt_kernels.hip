// kvbt_kernels.hip -- HIP kernels for gfx950 (CDNA4, wave64) of the top-k KV-block
// selector and the page-16 sparse block table, and their launchers.
//
// Two selector kernels, chosen by the launch policy from max_block:
//   * wave path (max_block <= 128): one wavefront per (row, head), several per
//     workgroup. Each lane holds two tiles of a 128-tile chunk; an exact bit-serial
//     top-k over the 128 keys (one ballot per key bit) merges them into the running
//     result. A row longer than 128 tiles loops over chunks, so results never
//     depend on the policy.
//   * workgroup path (129..8192): one 256-thread workgroup per (row, head). The row
//     is streamed once from HBM with 16-byte loads into registers. A cheap filter
//     finds, per wavefront, a threshold that the row's top-k must reach (the k-th
//     largest per-lane maximum); the few elements above it are compacted into LDS
//     and wavefront 0 selects the exact top-k among them plus the forced blocks.
//     Degenerate rows (mostly negative scores or mass ties) fall back, inside the
//     same launch, to a filter on exact unique keys that always fits in LDS.
// Both can emit the page-16 table in the same launch (the fused call).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "kvbt_device.h"
#include "kvbt_launch.h"

namespace kvbt {

struct SelArgs {
    const void* scores;
    int64_t T;
    int H;
    int M;
    Rows rows;
    int topk;
    int num_init;
    int num_local;
    int32_t* out_idx;
    const int32_t* block_table;
    int max_blocks;
    int32_t* out_table;
    int32_t* out_ctx;
    int rhpb;        // wave path: (row, head) pairs per workgroup
    int reverse;     // workgroup path: visit (row, head) pairs last to first
    int table_vec;   // out_table is 16-byte aligned
};

struct TabArgs {
    const int32_t* idx;
    int64_t T;
    int H;
    int topk;
    Rows rows;
    const int32_t* block_table;
    int max_blocks;
    int32_t* out_table;
    int32_t* out_ctx;
    int table_vec;
};

// Score element as a binary32 bit pattern (bf16 widened by 16 zero bits).
template <bool BF16>
__device__ inline uint32_t load_bits(const void* p, int64_t off)
{
    if constexpr (BF16)
        return (uint32_t)(static_cast<const uint16_t*>(p)[off]) << 16;
    else
        return static_cast<const uint32_t*>(p)[off];
}

template <bool BF16>
using KeyOf = typename std::conditional<BF16, KeyBF16, KeyF32>::type;

// Exact top-k of one (row, head) by one wavefront, over tiles [0, nvp) in chunks
// of 128. r0/r1 are the row's tiles lane and lane+64 (loaded by the caller, any
// value past nvp). Forced blocks get the forced key. Returns lane r = rank-r key.
template <bool BF16>
__device__ inline typename KeyOf<BF16>::T wave_select_row(const void* scores, int64_t row_off,
                                                          int nvp, int topk, int ni, int nl,
                                                          uint32_t r0, uint32_t r1)
{
    using KT = KeyOf<BF16>;
    using T = typename KT::T;
    const int lane = lane_id();
    const int lo_local = nvp - nl;
    T carry = 0;
    for (int base = 0; base < nvp; base += 2 * kWave) {
        uint32_t raw[2] = {r0, r1};
        if (base > 0) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int e = base + s * kWave + lane;
                raw[s] = e < nvp ? load_bits<BF16>(scores, row_off + e) : 0u;
            }
        }
        T k[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int e = base + s * kWave + lane;
            const bool forced = e < ni || e >= lo_local;
            k[s] = e < nvp ? (forced ? KT::forced(e) : KT::scored(raw[s], e)) : T(0);
        }
        carry = wave_topk_merge<T, KT::kBits, 2>(k, carry, topk);
    }
    return carry;
}

// ---------------------------------------------------------------------------
// Wave path
// ---------------------------------------------------------------------------
template <bool BF16, bool FUSED>
__global__ __launch_bounds__(256) void select_wave_kernel(SelArgs a)
{
    using T = typename KeyOf<BF16>::T;
    const int wave = (int)(threadIdx.x >> 6);
    const int lane = lane_id();
    const int64_t total = a.T * a.H;
    const int64_t rh = (int64_t)blockIdx.x * a.rhpb + wave;
    if (rh >= total) return;
    const int64_t t = rh / a.H;
    const int64_t row_off = rh * (int64_t)a.M;

    // The first chunk's tiles are fetched before the row metadata is known, so the
    // two memory round trips overlap; tiles past the causal count are masked below.
    const uint32_t r0 = lane < a.M ? load_bits<BF16>(a.scores, row_off + lane) : 0u;
    const uint32_t r1 = lane + kWave < a.M ? load_bits<BF16>(a.scores, row_off + lane + kWave) : 0u;

    int nvp;
    int64_t c = 0;
    int req = -1;
    if constexpr (FUSED) {
        const RowInfo ri = row_info(a.rows, t);
        c = ri.c;
        req = ri.req;
        nvp = (int)clamp_count((c + kBlockTokens - 1) / kBlockTokens, a.M);
    } else {
        nvp = (int)clamp_count(a.rows.num_valid_pages[t], a.M);
    }

    const T top = wave_select_row<BF16>(a.scores, row_off, nvp, a.topk, a.num_init,
                                        a.num_local, r0, r1);
    const int id = key_block(top);
    if (lane < a.topk) a.out_idx[rh * a.topk + lane] = id;
    if constexpr (FUSED) {
        const int32_t* bt_row = req >= 0 ? a.block_table + (int64_t)req * a.max_blocks : nullptr;
        emit_table_group(id, lane < 16, c, bt_row, a.max_blocks, a.topk,
                         a.out_table + rh * (int64_t)a.topk * kPagesPerBlock, a.out_ctx + rh,
                         a.table_vec != 0);
    }
}

// ---------------------------------------------------------------------------
// Workgroup path
// ---------------------------------------------------------------------------
template <bool BF16, int VEC>
__device__ inline void load_vec(const void* scores, int64_t row_off, int e0, uint32_t (&out)[VEC])
{
    if constexpr (VEC == 1) {
        out[0] = load_bits<BF16>(scores, row_off + e0);
    } else if constexpr (!BF16 && VEC == 4) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(scores) +
                                                        row_off + e0);
        out[0] = w.x; out[1] = w.y; out[2] = w.z; out[3] = w.w;
    } else {
        static_assert(BF16 && VEC == 8, "vector widths: fp32 x4, bf16 x8");
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(scores) +
                                                        row_off + e0);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = ws[i] << 16;
            out[2 * i + 1] = ws[i] & 0xFFFF0000u;
        }
    }
}

template <bool BF16, int VEC, int NCH, bool FUSED>
__global__ __launch_bounds__(256) void select_wg_kernel(SelArgs a)
{
    using KT = KeyOf<BF16>;
    using T = typename KT::T;
    constexpr int EPT = VEC * NCH;              // score elements per thread
    constexpr int CH = 256 * VEC;               // elements per chunk of the workgroup
    constexpr int CAP = 4 * kMaxTopk * EPT;     // candidate capacity, never exceeded
    __shared__ T s_cand[CAP];
    __shared__ int s_count;
    __shared__ int s_overflow;

    const int tid = (int)threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int64_t total = a.T * a.H;
    const int64_t rh = a.reverse ? total - 1 - (int64_t)blockIdx.x : (int64_t)blockIdx.x;
    const int64_t t = rh / a.H;
    const int64_t row_off = rh * (int64_t)a.M;
    const int topk = a.topk, ni = a.num_init, nl = a.num_local;

    int nvp;
    int64_t c = 0;
    int req = -1;
    if constexpr (FUSED) {
        const RowInfo ri = row_info(a.rows, t);
        c = ri.c;
        req = ri.req;
        nvp = (int)clamp_count((c + kBlockTokens - 1) / kBlockTokens, a.M);
    } else {
        nvp = (int)clamp_count(a.rows.num_valid_pages[t], a.M);
    }
    const int lo_local = nvp - nl;

    T top;
    if (nvp <= 2 * kWave) {
        // short row: one wavefront does it exactly
        if (wave != 0) return;
        const uint32_t r0 = lane < nvp ? load_bits<BF16>(a.scores, row_off + lane) : 0u;
        const uint32_t r1 = lane + kWave < nvp ? load_bits<BF16>(a.scores, row_off + lane + kWave) : 0u;
        top = wave_select_row<BF16>(a.scores, row_off, nvp, topk, ni, nl, r0, r1);
    } else {
        if (tid == 0) {
            s_count = 0;
            s_overflow = 0;
        }
        // stream the row into registers; elements past nvp read as the -0 pattern
        uint32_t raw[NCH][VEC];
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int e0 = (j * 256 + tid) * VEC;
#pragma unroll
            for (int v = 0; v < VEC; ++v) raw[j][v] = 0x80000000u;
            if (j * CH < nvp && e0 < nvp) load_vec<BF16, VEC>(a.scores, row_off, e0, raw[j]);
        }

        // Filter key: the score bits as a signed integer, clamped below at -1. It is
        // non-decreasing in the rank order (positive patterns keep their order, every
        // negative pattern maps to -1), so the k-th largest per-lane maximum of a
        // wavefront is a value the row's top-k all reach.
        int lmax = INT32_MIN;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            if ((j + 1) * CH <= nvp) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) lmax = max(lmax, (int)raw[j][v]);
            } else if (j * CH < nvp) {
                const int e0 = (j * 256 + tid) * VEC;
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    lmax = max(lmax, e0 + v < nvp ? (int)raw[j][v] : INT32_MIN);
            }
        }
        const bool lane_valid = tid * VEC < nvp;
        const int lkey = lane_valid ? max(lmax, -1) : INT32_MIN;
        const uint32_t tau_u = wave_kth<uint32_t, 32>((uint32_t)lkey ^ 0x80000000u, topk);
        __syncthreads();

        // tau_u == 0: fewer than topk lanes of this wavefront hold elements, so all of
        // them are candidates (at most (topk-1) * EPT). tau == -1: fewer than topk
        // lanes reach a non-negative score; the clamped key cannot separate them, so
        // take the exact-key path.
        const int tau = tau_u == 0 ? -1 : (int)(tau_u ^ 0x80000000u);
        if (tau_u != 0 && tau == -1) {
            if (lane == 0) s_overflow = 1;
        } else if (lkey >= tau) {
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int e0 = (j * 256 + tid) * VEC;
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const int e = e0 + v;
                    const bool forced = e < ni || e >= lo_local;
                    if (j * CH < nvp && e < nvp && !forced && max((int)raw[j][v], -1) >= tau) {
                        const int pos = atomicAdd(&s_count, 1);
                        if (pos < CAP)
                            s_cand[pos] = KT::scored(raw[j][v], e);
                        else
                            s_overflow = 1;
                    }
                }
            }
        }
        __syncthreads();

        if (s_overflow) {
            // Exact unique keys: the k-th largest per-lane maximum is met by exactly
            // topk lanes, so at most topk * EPT candidates per wavefront (= CAP in all).
            if (tid == 0) s_count = 0;
            __syncthreads();
            T lk = 0;
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const int e0 = (j * 256 + tid) * VEC;
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const int e = e0 + v;
                    if (j * CH < nvp && e < nvp) {
                        const T k = KT::scored(raw[j][v], e);
                        lk = k > lk ? k : lk;
                    }
                }
            }
            T tk = wave_kth<T, KT::kBits>(lk, topk);
            if (tk == 0) tk = 1;
            if (lk >= tk) {
#pragma unroll
                for (int j = 0; j < NCH; ++j) {
                    const int e0 = (j * 256 + tid) * VEC;
#pragma unroll
                    for (int v = 0; v < VEC; ++v) {
                        const int e = e0 + v;
                        const bool forced = e < ni || e >= lo_local;
                        if (j * CH < nvp && e < nvp && !forced) {
                            const T k = KT::scored(raw[j][v], e);
                            if (k >= tk) {
                                const int pos = atomicAdd(&s_count, 1);
                                if (pos < CAP) s_cand[pos] = k;
                            }
                        }
                    }
                }
            }
            __syncthreads();
        }
        if (wave != 0) return;

        // exact top-k of the forced blocks plus the candidates, by wavefront 0
        const int n = min(s_count, CAP);
        int f = -1;
        if (lane < ni) f = lane;
        else if (lane < ni + nl) f = lo_local + (lane - ni);
        top = f >= 0 ? KT::forced(f) : T(0);
        int base = 0;
        do {
            T k[2];
            k[0] = base + lane < n ? s_cand[base + lane] : T(0);
            k[1] = base + kWave + lane < n ? s_cand[base + kWave + lane] : T(0);
            top = wave_topk_merge<T, KT::kBits, 2>(k, top, topk);
            base += 2 * kWave;
        } while (base < n);
    }

    const int id = key_block(top);
    if (lane < topk) a.out_idx[rh * topk + lane] = id;
    if constexpr (FUSED) {
        const int32_t* bt_row = req >= 0 ? a.block_table + (int64_t)req * a.max_blocks : nullptr;
        emit_table_group(id, lane < 16, c, bt_row, a.max_blocks, topk,
                         a.out_table + rh * (int64_t)topk * kPagesPerBlock, a.out_ctx + rh,
                         a.table_vec != 0);
    }
}

// ---------------------------------------------------------------------------
// Standalone table builder: 16 lanes per (row, head), 16 (row, head) per workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void table_kernel(TabArgs a)
{
    const int wave = (int)(threadIdx.x >> 6);
    const int lane = lane_id();
    const int g = lane >> 4, gl = lane & 15;
    const int64_t total = a.T * a.H;
    const int64_t first = ((int64_t)blockIdx.x * 4 + wave) * 4;
    if (first >= total) return;
    const int64_t rh = first + g;
    const bool active = rh < total;
    int id = -1;
    int64_t c = 0;
    const int32_t* bt_row = nullptr;
    if (active) {
        const RowInfo ri = row_info(a.rows, rh / a.H);
        c = ri.c;
        if (ri.req >= 0) bt_row = a.block_table + (int64_t)ri.req * a.max_blocks;
        if (gl < a.topk) id = a.idx[rh * a.topk + gl];
    }
    const int64_t rh_out = active ? rh : 0;
    emit_table_group(id, active, c, bt_row, a.max_blocks, a.topk,
                     a.out_table + rh_out * (int64_t)a.topk * kPagesPerBlock, a.out_ctx + rh_out,
                     a.table_vec != 0);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {

template <bool BF16, bool FUSED>
hipError_t launch_wave(const SelArgs& s, int rhpb, hipStream_t stream)
{
    const int64_t total = s.T * s.H;
    const int64_t blocks = (total + rhpb - 1) / rhpb;
    hipLaunchKernelGGL((select_wave_kernel<BF16, FUSED>), dim3((unsigned)blocks),
                       dim3(kWave * rhpb), 0, stream, s);
    return hipGetLastError();
}

template <bool BF16, int VEC, int NCH, bool FUSED>
hipError_t launch_wg_one(const SelArgs& s, hipStream_t stream)
{
    hipLaunchKernelGGL((select_wg_kernel<BF16, VEC, NCH, FUSED>), dim3((unsigned)(s.T * s.H)),
                       dim3(256), 0, stream, s);
    return hipGetLastError();
}

template <bool BF16, int VEC, bool FUSED>
hipError_t launch_wg_vec(const SelArgs& s, int chunks, hipStream_t stream)
{
    switch (chunks) {
        case 1: return launch_wg_one<BF16, VEC, 1, FUSED>(s, stream);
        case 2: return launch_wg_one<BF16, VEC, 2, FUSED>(s, stream);
        case 4: return launch_wg_one<BF16, VEC, 4, FUSED>(s, stream);
        case 8: if constexpr (VEC * 8 <= 32) return launch_wg_one<BF16, VEC, 8, FUSED>(s, stream);
                break;
        case 16: if constexpr (VEC * 16 <= 32) return launch_wg_one<BF16, VEC, 16, FUSED>(s, stream);
                 break;
        case 32: if constexpr (VEC * 32 <= 32) return launch_wg_one<BF16, VEC, 32, FUSED>(s, stream);
                 break;
        default: break;
    }
    return hipErrorInvalidValue;
}

template <bool BF16, bool FUSED>
hipError_t launch_wg(const SelArgs& s, int vec, int chunks, hipStream_t stream)
{
    if (vec == 1) return launch_wg_vec<BF16, 1, FUSED>(s, chunks, stream);
    if constexpr (BF16) {
        if (vec == 8) return launch_wg_vec<true, 8, FUSED>(s, chunks, stream);
    } else {
        if (vec == 4) return launch_wg_vec<false, 4, FUSED>(s, chunks, stream);
    }
    return hipErrorInvalidValue;
}

int pow2_at_least(int64_t x)
{
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

}  // namespace

hipError_t launch_select(const SelectLaunch& l, hipStream_t stream)
{
    const int64_t total = l.T * l.H;
    if (total == 0) return hipSuccess;
    SelArgs s;
    s.scores = l.scores;
    s.T = l.T;
    s.H = l.H;
    s.M = l.M;
    s.rows.num_valid_pages = l.num_valid_pages;
    s.rows.seq_lens = l.seq_lens;
    s.rows.row_req = l.row_req;
    s.rows.row_pos = l.row_pos;
    s.rows.q = l.q > 0 ? l.q : 1;
    s.rows.B = l.B;
    s.topk = l.topk;
    s.num_init = l.num_init;
    s.num_local = l.num_local;
    s.out_idx = l.out_idx;
    s.block_table = l.block_table;
    s.max_blocks = l.max_blocks;
    s.out_table = l.out_table;
    s.out_ctx = l.out_ctx;
    s.rhpb = l.policy.row_heads_per_block;
    s.reverse = 1;
    s.table_vec = ((uintptr_t)l.out_table % 16) == 0;
    const bool bf16 = l.dtype == KVBT_BF16;

    if (l.policy.path == 0) {
        if (bf16) return l.fused ? launch_wave<true, true>(s, s.rhpb, stream)
                                 : launch_wave<true, false>(s, s.rhpb, stream);
        return l.fused ? launch_wave<false, true>(s, s.rhpb, stream)
                       : launch_wave<false, false>(s, s.rhpb, stream);
    }
    int vec = l.policy.vec;
    int chunks = l.policy.chunks;
    if (vec > 1 && ((uintptr_t)l.scores % 16) != 0) {
        vec = 1;
        chunks = pow2_at_least((l.M + 255) / 256);
    }
    if (bf16) return l.fused ? launch_wg<true, true>(s, vec, chunks, stream)
                             : launch_wg<true, false>(s, vec, chunks, stream);
    return l.fused ? launch_wg<false, true>(s, vec, chunks, stream)
                   : launch_wg<false, false>(s, vec, chunks, stream);
}

hipError_t launch_table(const TableLaunch& l, hipStream_t stream)
{
    const int64_t total = l.T * l.H;
    if (total == 0) return hipSuccess;
    TabArgs s;
    s.idx = l.idx;
    s.T = l.T;
    s.H = l.H;
    s.topk = l.topk;
    s.rows.num_valid_pages = nullptr;
    s.rows.seq_lens = l.seq_lens;
    s.rows.row_req = l.row_req;
    s.rows.row_pos = l.row_pos;
    s.rows.q = l.q > 0 ? l.q : 1;
    s.rows.B = l.B;
    s.block_table = l.block_table;
    s.max_blocks = l.max_blocks;
    s.out_table = l.out_table;
    s.out_ctx = l.out_ctx;
    s.table_vec = ((uintptr_t)l.out_table % 16) == 0;
    const int64_t blocks = (total + 15) / 16;
    hipLaunchKernelGGL(table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, s);
    return hipGetLastError();
}

}  // namespace kvbt
