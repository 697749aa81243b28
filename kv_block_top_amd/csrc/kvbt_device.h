// kvbt_device.h -- device-side building blocks of the selector and table kernels
// (gfx950, wave64). Everything here works on integer images of the scores: the
// selector does no floating-point arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvbt_divide.h"

namespace kvbt {

constexpr int kWave = 64;
constexpr int kBlockTokens = 128;      // tokens per KV block (= per score tile)
constexpr int kPagesPerBlock = 8;      // 16-token pages per block
constexpr int kMaxTopk = 16;
constexpr int kRidBits = 13;           // block ids are < 8192
constexpr uint32_t kRidMask = (1u << kRidBits) - 1u;

// ---------------------------------------------------------------------------
// Row description: where a row's causal length and request come from.
// ---------------------------------------------------------------------------
struct Rows {
    const int32_t* num_valid_pages;  // standalone selector: causal block counts [T]
    const int32_t* seq_lens;         // decode form: [B]
    const int32_t* row_req;          // explicit form: [T] (nullptr selects decode form)
    const int32_t* row_pos;          // explicit form: [T]
    int q;                           // decode query length
    int B;                           // requests
    uint32_t q_mul, q_shift;         // make_divisor(q)
};

struct RowInfo {
    int64_t c;   // causal length in tokens, >= 0
    int req;     // request id, -1 when the row names no request
};

// Decode form (row_req == nullptr): row t is request t / q at position
// seq_lens[req] - q + t % q (spec-decode row layout). Explicit form: (row_req[t],
// row_pos[t]); a request id outside [0, B) makes the row a padded row. t < 2^31.
__device__ __forceinline__ RowInfo row_info_of(const int32_t* seq_lens, const int32_t* row_req,
                                               const int32_t* row_pos, int q, uint32_t q_mul,
                                               uint32_t q_shift, int B, int64_t t)
{
    RowInfo o;
    int64_t pos;
    if (row_req == nullptr) {
        const int64_t req = divide_by((uint32_t)t, q_mul, q_shift);
        pos = (int64_t)seq_lens[req] - q + (t - req * q);
        o.req = (int)req;
    } else {
        const int req = row_req[t];
        if (req < 0 || req >= B) {
            o.req = -1;
            o.c = 0;
            return o;
        }
        pos = row_pos[t];
        o.req = req;
    }
    o.c = pos + 1 > 0 ? pos + 1 : 0;
    return o;
}

__device__ __forceinline__ RowInfo row_info(const Rows& r, int64_t t)
{
    return row_info_of(r.seq_lens, r.row_req, r.row_pos, r.q, r.q_mul, r.q_shift, r.B, t);
}

// Workspace shared between workgroups (cross-workgroup splits). The XCDs' L2 caches
// are not coherent with each other for ordinary stores, and an agent-scope release
// fence writes back a whole L2 (microseconds each). A workspace is therefore only ever
// written and read with agent-scope atomic stores and loads, which go through to the
// point of coherence; a wavefront orders its workspace stores before an arrival counter
// increment by waiting for them to complete, with a workgroup-scope fence to keep the
// compiler from reordering them.
__device__ __forceinline__ void ws_store(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t ws_load(const uint64_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt with vmcnt 0 and the other counters left alone (expcnt 7, lgkmcnt 15)
constexpr int kWaitVmem = (0x7 << 4) | (0xF << 8);

// This wavefront's earlier workspace stores complete before anything after this.
__device__ __forceinline__ void ws_order_release()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
}

// Nothing after this is issued before the counter's returned value arrived.
__device__ __forceinline__ void ws_order_acquire()
{
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// A value the whole wavefront holds (for example loaded from one address by every
// lane), moved to a scalar register so that the compiler treats it as uniform.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int64_t uniform(int64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t clamp_count(int64_t v, int64_t hi)
{
    return v < 0 ? 0 : (v > hi ? hi : v);
}

// ---------------------------------------------------------------------------
// Rank keys. A candidate's key packs [class:2][order image of the score][13-bit
// reversed block id]; a larger key ranks first and distinct blocks have distinct
// keys, so every comparison is one unsigned integer compare.
//   class 2 = forced block (score ignored), 1 = scored block, key 0 = no candidate.
// The order image maps a binary32 pattern to an unsigned integer whose order is
// IEEE 754 totalOrder: flip every bit of a negative pattern, set the sign bit of
// a positive one. bf16 scores are held as binary32 patterns (bf16 << 16); their
// image keeps only the top 16 bits, which carry all of the order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_image(uint32_t bits)
{
    return bits ^ ((uint32_t)((int32_t)bits >> 31) | 0x80000000u);
}

// 64-bit rank key of binary32 patterns (bf16 widened by 16 zero bits orders the same):
// [class:2][totalOrder image:32][(2^RID - 1) - id:RID]. RID = 13 covers block ids below
// 8192, the fast path's capacity; RID = 24 covers every block id below 2^24, which is as
// many 128-token blocks as an int32 token position can reach. Either way the key fits
// in 58 bits, so a 6-bit lane index can ride below it in one 64-bit sort.
template <int RID>
struct KeyU64 {
    using T = uint64_t;
    static constexpr int kRid = RID;
    static constexpr uint32_t kMask = (1u << RID) - 1u;
    static constexpr int kBits = 2 + 32 + RID;
    __device__ __forceinline__ static T scored(uint32_t bits, int id)
    {
        return (T(1) << (32 + RID)) | (T(order_image(bits)) << RID) | T(kMask - (uint32_t)id);
    }
    __device__ __forceinline__ static T forced(int id) { return (T(2) << (32 + RID)) | T(kMask - (uint32_t)id); }
    __device__ __forceinline__ static int block(T key)
    {
        return key ? (int)(kMask - (uint32_t)(key & kMask)) : -1;
    }
};

using KeyF32 = KeyU64<kRidBits>;    // 47 bits
using KeyWide = KeyU64<24>;         // 58 bits

// 32-bit rank key of bf16 patterns: [class:2][image:16][8191 - id:13].
struct KeyBF16 {
    using T = uint32_t;
    static constexpr int kBits = 2 + 16 + kRidBits;   // 31
    __device__ __forceinline__ static T scored(uint32_t bits, int id)
    {
        return (1u << 29) | ((order_image(bits) >> 16) << kRidBits) | (kRidMask - (uint32_t)id);
    }
    __device__ __forceinline__ static T forced(int id) { return (2u << 29) | (kRidMask - (uint32_t)id); }
    __device__ __forceinline__ static int block(T key)
    {
        return key ? (int)(kRidMask - (key & kRidMask)) : -1;
    }
};

// ---------------------------------------------------------------------------
// Wave primitives (all 64 lanes must be active).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }


__device__ __forceinline__ uint32_t readlane(uint32_t v, int l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

__device__ __forceinline__ uint64_t readlane(uint64_t v, int l)
{
    const uint32_t lo = readlane((uint32_t)v, l);
    const uint32_t hi = readlane((uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int shfl(int v, int src_lane)
{
    return __builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}

// ---------------------------------------------------------------------------
// Cross-lane exchange with lane ^ P, and bitonic sorting networks on it.
// P = 1, 2, 3: DPP quad permutes; 4: half-row mirror then quad reverse; 7, 15: DPP
// half-row / row mirrors; 8: DPP row rotate; 16, 31: gfx950 permlane16 swap (after a
// row mirror for 31); 32, 63: permlane32 swap (after the 31 exchange for 63). All of
// them are vector-ALU operations with no LDS round trip, which matters when a
// wavefront sorts alone on its SIMD; the networks below issue no scalar-ALU work per
// comparison beyond combining lane masks.
// ---------------------------------------------------------------------------
template <int P>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x)
{
    // Every exchange stays in the vector ALU (no LDS round trip): DPP within 16-lane
    // rows, and gfx950's permlane swaps across rows (a swap of x with itself returns the
    // even and the odd row (or half) of each pair duplicated; the lane takes the other).
    if constexpr (P == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
    } else if constexpr (P == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
    } else if constexpr (P == 3) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x1B, 0xF, 0xF, false);   // quad [3,2,1,0]
    } else if constexpr (P == 4) {
        // half-row mirror (i -> 7 - i) then quad reverse (j -> 3 - j): i -> i ^ 4
        const int m = __builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);
        return (uint32_t)__builtin_amdgcn_update_dpp(0, m, 0x1B, 0xF, 0xF, false);
    } else if constexpr (P == 7) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);  // half-row mirror
    } else if constexpr (P == 8) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);  // row rotate by 8
    } else if constexpr (P == 15) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false);  // row mirror
    } else if constexpr (P == 16 || P == 31) {
        const uint32_t y = P == 31 ? xor_lane<15>(x) : x;
        const auto p = __builtin_amdgcn_permlane16_swap(y, y, false, false);
        return (lane_id() & 16) ? p[0] : p[1];
    } else {
        static_assert(P == 32 || P == 63, "unsupported lane pattern");
        const uint32_t y = P == 63 ? xor_lane<31>(x) : x;
        const auto p = __builtin_amdgcn_permlane32_swap(y, y, false, false);
        return (lane_id() & 32) ? p[0] : p[1];
    }
}

template <int P>
__device__ __forceinline__ uint64_t xor_lane(uint64_t x)
{
    const uint32_t lo = xor_lane<P>((uint32_t)x);
    const uint32_t hi = xor_lane<P>((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// One compare-exchange step between lane and lane ^ P: the lane keeps the larger value
// when `keep_max`, else the smaller. For 32-bit keys as max / min / select; for 64-bit
// keys the lane takes its partner's key when "partner is larger" equals keep_max (two
// lane masks combined by one scalar XNOR): for distinct keys the same, for equal keys
// no change.
template <int P>
__device__ __forceinline__ uint32_t cx_step(uint32_t x, bool keep_max)
{
    const uint32_t p = xor_lane<P>(x);
    const uint32_t hi = x > p ? x : p;
    const uint32_t lo = x > p ? p : x;
    return keep_max ? hi : lo;
}

template <int P>
__device__ __forceinline__ uint64_t cx_step(uint64_t x, bool keep_max)
{
    const uint64_t p = xor_lane<P>(x);
    return keep_max == (p > x) ? p : x;
}

// Bitonic sort in the "flip" form: merging two sorted blocks of K/2 lanes starts by
// comparing lane i with its mirror i ^ (K-1), then lanes i and i ^ J for J = K/4 .. 1.
// The lower lane of every pair keeps the larger key (DESC) or the smaller (!DESC), so
// the only lane masks are "bit J of the lane is clear", J = 1 .. 32.
template <bool DESC, int K, int J, typename T>
__device__ __forceinline__ T flip_stages(T x, int lane)
{
    if constexpr (J == K / 2)
        x = cx_step<K - 1>(x, ((lane & J) == 0) == DESC);
    else
        x = cx_step<J>(x, ((lane & J) == 0) == DESC);
    if constexpr (J > 1) return flip_stages<DESC, K, J / 2>(x, lane);
    else return x;
}

template <bool DESC, int K, int KMAX, typename T>
__device__ __forceinline__ T flip_sort(T x, int lane)
{
    x = flip_stages<DESC, K, K / 2>(x, lane);
    if constexpr (K < KMAX) return flip_sort<DESC, K * 2, KMAX>(x, lane);
    else return x;
}

// One key per lane, descending: lane 0 ends with the largest.
template <typename T>
__device__ __forceinline__ T sort64_desc(T x)
{
    return flip_sort<true, 2, 64>(x, lane_id());
}

// Descending xor stages J .. 1 (the tail of a merge).
template <int J, typename T>
__device__ __forceinline__ T desc_xor_stages(T x, int lane)
{
    x = cx_step<J>(x, (lane & J) == 0);
    if constexpr (J > 1) return desc_xor_stages<J / 2>(x, lane);
    else return x;
}

// Top 16 of 128 unique keys, two per lane (element i = 64 * slot + lane), in rank order
// in lanes 0..15 (other lanes: unspecified) -- top16_of_128 below. Only the best 16 are
// ever needed, so the network does not sort all 128: the 16-lane rows of both registers
// are sorted (10 stages each, the two registers stage by stage together), each row of
// one register is folded with the same row of the other (the element-wise maximum of
// one sorted list and the other mirrored holds the top 16 of their union as a bitonic
// sequence, which xor stages 8..1 sort), then rows 0 and 1 with rows 2 and 3 through the
// mirror across lane 31 (row r + 1 against row r), and the result across lane 63: 35
// register-stages against 55 for a full 128-key sort.
// top16_of_sorted_rows: the same when the 16-lane rows of both registers are already
// sorted descending (only the three folds).
template <typename T>
__device__ __forceinline__ T top16_of_sorted_rows(T a, T b)
{
    const int lane = lane_id();
    T r = xor_lane<15>(b);
    T x = desc_xor_stages<8>(r > a ? r : a, lane);
    r = xor_lane<31>(x);
    x = desc_xor_stages<8>(r > x ? r : x, lane);
    r = xor_lane<63>(x);
    return desc_xor_stages<8>(r > x ? r : x, lane);
}

// The networks above on N registers at once, stage by stage: the N chains are
// independent, so each one's exchanges fill the others' waits (written one network
// after the other, the compiler kept them apart and every stage waited on its own
// previous one).
template <bool DESC, int K, int J, int N, typename T>
__device__ __forceinline__ void flip_stages_n(T (&x)[N], int lane)
{
    const bool keep = ((lane & J) == 0) == DESC;
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = cx_step<J == K / 2 ? K - 1 : J>(x[i], keep);
    if constexpr (J > 1) flip_stages_n<DESC, K, J / 2>(x, lane);
}

template <bool DESC, int K, int KMAX, int N, typename T>
__device__ __forceinline__ void flip_sort_n(T (&x)[N], int lane)
{
    flip_stages_n<DESC, K, K / 2>(x, lane);
    if constexpr (K < KMAX) flip_sort_n<DESC, K * 2, KMAX>(x, lane);
}

template <int J, int N, typename T>
__device__ __forceinline__ void desc_xor_stages_n(T (&x)[N], int lane)
{
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = cx_step<J>(x[i], (lane & J) == 0);
    if constexpr (J > 1) desc_xor_stages_n<J / 2>(x, lane);
}

// top16_of_128 of N pairs (a[i], b[i]) at once; a[i] ends with pair i's result.
template <int N, typename T>
__device__ __forceinline__ void top16_of_128_n(T (&a)[N], T (&b)[N])
{
    const int lane = lane_id();
    flip_sort_n<true, 2, 16>(a, lane);
    flip_sort_n<true, 2, 16>(b, lane);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const T r = xor_lane<15>(b[i]);
        a[i] = r > a[i] ? r : a[i];
    }
    desc_xor_stages_n<8>(a, lane);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const T r = xor_lane<31>(a[i]);
        a[i] = r > a[i] ? r : a[i];
    }
    desc_xor_stages_n<8>(a, lane);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const T r = xor_lane<63>(a[i]);
        a[i] = r > a[i] ? r : a[i];
    }
    desc_xor_stages_n<8>(a, lane);
}

// The network on one pair: interleaving its two row sorts took the 74-block batch from
// 2.73 to 2.71 us, and all chunks of a row together the 512-tile decode batch from 4.42
// to 4.10 us (wave_select_chunks).
template <typename T>
__device__ __forceinline__ T top16_of_128(T a, T b)
{
    T x[1] = {a}, y[1] = {b};
    top16_of_128_n<1>(x, y);
    return x[0];
}

// Top 16 of two descending 16-lists held in lanes 0..15 (`top` and `add`), in rank
// order in lanes 0..15; other lanes return 0. The element-wise maximum of one list and
// the other mirrored holds the top 16 of the union as a bitonic sequence, which xor
// stages 8 .. 1 sort.
template <typename T>
__device__ __forceinline__ T merge_top16(T top, T add)
{
    const int lane = lane_id();
    const T r = xor_lane<15>(add);
    const T x = desc_xor_stages<8>(r > top ? r : top, lane);
    return lane < 16 ? x : T(0);
}

// Best 16 of the first n keys of k0 (elements 0..63, element = lane) and k1 (elements
// 64..127), the rest zero, in rank order in lanes 0..15 (other lanes: unspecified). With
// 64-bit keys, whose exchanges cost twice as much, the network is no wider than the keys
// present (a 16- or 32-lane sort leaves every key in the first lanes, as n <= 16 or 32
// puts all of them there: workload 1, at most 16 fp32 tiles, 2.26 against 2.62 us per
// call); with 32-bit keys the two extra networks' code cost the 74-block batch more
// (2.79 against 2.71 us) than their shorter chains saved.
template <typename T>
__device__ __forceinline__ T top16_of_short(T k0, T k1, int n)
{
    const int lane = lane_id();
    if constexpr (sizeof(T) == 8) {
        if (n <= 16) return flip_sort<true, 2, 16>(k0, lane);
        if (n <= 32) return flip_sort<true, 2, 32>(k0, lane);
    }
    if (n <= kWave) return flip_sort<true, 2, 64>(k0, lane);
    return top16_of_128(k0, k1);
}

// Top 16 of N descending 16-lists held in lanes 0..15 of x[0..N-1] (zero elsewhere; N a
// power of two), in rank order in lanes 0..15: merged pairwise as merge_top16, the
// merges of one level stage by stage together.
template <int N, typename T>
__device__ __forceinline__ T fold_top16_n(T (&x)[N])
{
    if constexpr (N == 1) {
        return x[0];
    } else {
        const int lane = lane_id();
        T y[N / 2];
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const T r = xor_lane<15>(x[2 * i + 1]);
            y[i] = r > x[2 * i] ? r : x[2 * i];
        }
        desc_xor_stages_n<8>(y, lane);
#pragma unroll
        for (int i = 0; i < N / 2; ++i) y[i] = lane < 16 ? y[i] : T(0);
        return fold_top16_n<N / 2>(y);
    }
}

// Ascending sort of the 16 lanes of each row (one key per lane).
__device__ __forceinline__ uint32_t sort16_asc(uint32_t x)
{
    return flip_sort<false, 2, 16>(x, lane_id());
}

// Exact top-16 (rank order in lanes 0..15, 0 beyond the valid count) of a list of
// n unique keys, where key_at(i) gives the i-th key (0 = no candidate). The list is
// taken 128 keys at a time: the top 16 of each chunk come from the bitonic networks
// above and are merged into the running top-16.
template <typename T, typename F>
__device__ __forceinline__ T topk16_of_list(int n, F key_at)
{
    const int lane = lane_id();
    T carry = 0;
    for (int base = 0; base < n; base += 2 * kWave) {
        T a = base + lane < n ? key_at(base + lane) : T(0);
        T top;
        if (n - base <= kWave) {
            top = sort64_desc(a);
        } else {
            T b = base + kWave + lane < n ? key_at(base + kWave + lane) : T(0);
            top = top16_of_128(a, b);
        }
        carry = base == 0 ? (lane < 16 ? top : T(0)) : merge_top16(carry, top);
    }
    return carry;
}

// Table row of one (row, head) from its selected blocks with their physical ids already
// fetched: lane r < topk holds the rank-r block id (-1 if none) and its physical block.
// Kept ids (below the causal block count and max_blocks) are sorted ascending with a
// 16-lane network that carries the source lane; kept block r then owns entries
// 8r..8r+7 (only the last causal block can be partly filled, and it is the largest id).
// With one_store (and a 16-byte-aligned row), the row is written by one store instruction
// of 2 topk lanes, 16 contiguous bytes each (whole lines instead of two instructions of
// alternate 16-byte pieces): faster where the stores share HBM with a read stream (the
// mixed unified batch 110.3-112.2 against 112.0-112.8 us, the 512-tile decode batch 4.61
// against 4.85 us), slower by the two lane permutes on a call that is only its
// latency chain (the 74-block batch 2.97-3.02 against 2.94-2.96 us).
__device__ __forceinline__ void emit_table_phys(int id, int phys, int64_t c, int max_blocks,
                                                int topk, int32_t* table_row, int32_t* ctx_out,
                                                bool vec_store, bool one_store = true)
{
    const int lane = lane_id();
    const int64_t nvp_c = (c + kBlockTokens - 1) / kBlockTokens;
    const int64_t lim = nvp_c < max_blocks ? nvp_c : (int64_t)max_blocks;
    const bool ok = lane < topk && id >= 0 && id < lim;
    const uint32_t sk = sort16_asc(ok ? ((uint32_t)id << 6) | (uint32_t)lane : 0xFFFFFFFFu);
    const bool kept = lane < 16 && sk != 0xFFFFFFFFu;
    const int src = (int)(sk & 63u);
    const int ph = __builtin_amdgcn_ds_bpermute(src << 2, phys);
    int tb = 0;
    if (kept) {
        const int64_t rest = c - (int64_t)kBlockTokens * (sk >> 6);
        tb = rest < kBlockTokens ? (int)rest : kBlockTokens;
    }
    const int np = (tb + 15) >> 4;
    uint32_t sum = (uint32_t)tb;
    sum += xor_lane<8>(sum);
    sum += xor_lane<4>(sum);
    sum += xor_lane<2>(sum);
    sum += xor_lane<1>(sum);
    if (vec_store && one_store) {
        // one store instruction writes the whole row contiguously: lane l < 2 topk takes
        // the 16 bytes of entries 4l .. 4l + 3, half (l & 1) of kept block l >> 1
        const int r = lane >> 1, half = lane & 1;
        const uint32_t base = (uint32_t)__builtin_amdgcn_ds_bpermute(r << 2, ph) *
                              (uint32_t)kPagesPerBlock;
        const int npr = __builtin_amdgcn_ds_bpermute(r << 2, np);
        if (lane < 2 * topk) {
            int v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = 4 * half + j;
                v[j] = e < npr ? (int)(base + (uint32_t)e) : 0;
            }
            reinterpret_cast<int4*>(table_row)[lane] = make_int4(v[0], v[1], v[2], v[3]);
        }
    } else if (lane < topk) {
        const uint32_t base = (uint32_t)ph * (uint32_t)kPagesPerBlock;
        int v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = j < np ? (int)(base + (uint32_t)j) : 0;
        int32_t* p = table_row + lane * kPagesPerBlock;
        if (vec_store) {
            reinterpret_cast<int4*>(p)[0] = make_int4(v[0], v[1], v[2], v[3]);
            reinterpret_cast<int4*>(p)[1] = make_int4(v[4], v[5], v[6], v[7]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = v[j];
        }
    }
    if (lane == 0) *ctx_out = (int32_t)sum;
}

// Page-16 table row of one (row, head) from its selected blocks: lane r < topk holds
// the rank-r block id (-1 if none); ids are unique. Each lane gathers the physical block
// of its id first, so that the gather is in flight while the kept ids are sorted; then
// as emit_table_phys. A row without a request (bt_row null) keeps nothing. Every lane
// of the wave must call this.
__device__ __forceinline__ void emit_table_sorted(int id, int64_t c, const int32_t* bt_row, int max_blocks,
                                         int topk, int32_t* table_row, int32_t* ctx_out,
                                         bool vec_store, bool one_store = true)
{
    int phys = 0;
    if (lane_id() < topk && bt_row != nullptr && id >= 0 && id < max_blocks) phys = bt_row[id];
    emit_table_phys(id, phys, bt_row != nullptr ? c : 0, max_blocks, topk, table_row, ctx_out,
                    vec_store, one_store);
}

// ---------------------------------------------------------------------------
// Page-16 table emission. Lanes 16g .. 16g+15 of a wave cooperate on one
// (row, head): lane 16g + j holds the j-th block id of that row's index list
// (-1 or anything when j >= topk). Every lane of the wave must call this.
//   - kept blocks: ids in [0, min(cdiv(c, 128), max_blocks)), first occurrence only;
//   - they are listed in ascending id; block b shows t_b = min(128, c - 128 b)
//     tokens as cdiv(t_b, 16) pages block_table[req][b] * 8 + j. Only the last
//     causal block can be partly filled and it is the largest kept id, so the
//     r-th kept block starts at entry 8 r;
//   - the rest of the row (topk * 8 entries) is 0; ctx = sum of t_b.
// `active` is false for groups with no row (their lanes write nothing).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void emit_table_group(int id, bool active, int64_t c, const int32_t* bt_row,
                                        int max_blocks, int topk, int32_t* table_row,
                                        int32_t* ctx_out, bool vec_store)
{
    const int lane = lane_id();
    const int gl = lane & 15;
    const int gb = lane & ~15;
    const int64_t nvp_c = (c + kBlockTokens - 1) / kBlockTokens;
    const int64_t lim = nvp_c < max_blocks ? nvp_c : (int64_t)max_blocks;
    bool ok = active && bt_row != nullptr && gl < topk && id >= 0 && id < lim;

    // drop repeats: a lane is a repeat if an earlier lane of its group holds its id
    const int k0 = ok ? id : -1 - gl;
    bool dup = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int o = shfl(k0, gb + j);
        dup |= (j < gl) && (o == k0);
    }
    ok = ok && !dup;

    // ascending rank; lanes without a block sort after all kept ones
    const int sk = ok ? id : 0x7FFFFFF0 + gl;
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) rank += (shfl(sk, gb + j) < sk) ? 1 : 0;

    int phys = 0, tb = 0;
    if (ok) {
        phys = bt_row[id];
        const int64_t rest = c - (int64_t)kBlockTokens * id;
        tb = rest < kBlockTokens ? (int)rest : kBlockTokens;
    }
    const int np = (tb + 15) >> 4;
    const int dst = (gb + rank) << 2;
    const int phys_r = __builtin_amdgcn_ds_permute(dst, phys);
    const int np_r = __builtin_amdgcn_ds_permute(dst, np);

    int sum = tb;
    sum += __shfl_xor(sum, 8);
    sum += __shfl_xor(sum, 4);
    sum += __shfl_xor(sum, 2);
    sum += __shfl_xor(sum, 1);

    if (active && gl < topk) {
        const uint32_t base = (uint32_t)phys_r * (uint32_t)kPagesPerBlock;
        int v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = j < np_r ? (int)(base + (uint32_t)j) : 0;
        int32_t* p = table_row + gl * kPagesPerBlock;
        if (vec_store) {
            reinterpret_cast<int4*>(p)[0] = make_int4(v[0], v[1], v[2], v[3]);
            reinterpret_cast<int4*>(p)[1] = make_int4(v[4], v[5], v[6], v[7]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = v[j];
        }
    }
    if (active && gl == 0) *ctx_out = sum;
}

}  // namespace kvbt
