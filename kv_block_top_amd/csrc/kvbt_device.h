// kvbt_device.h -- device-side building blocks of the selector and table kernels
// (gfx950, wave64). Everything here works on integer images of the scores: the
// selector does no floating-point arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
};

struct RowInfo {
    int64_t c;   // causal length in tokens, >= 0
    int req;     // request id, -1 when the row names no request
};

// Decode form: row t is request t / q at position seq_lens[req] - q + t % q
// (spec-decode row layout). Explicit form: (row_req[t], row_pos[t]); a request id
// outside [0, B) makes the row a padded row.
__device__ inline RowInfo row_info(const Rows& r, int64_t t)
{
    RowInfo o;
    int64_t pos;
    if (r.row_req == nullptr) {
        const int64_t req = t / r.q;
        pos = (int64_t)r.seq_lens[req] - r.q + (t - req * r.q);
        o.req = (int)req;
    } else {
        const int req = r.row_req[t];
        if (req < 0 || req >= r.B) {
            o.req = -1;
            o.c = 0;
            return o;
        }
        pos = r.row_pos[t];
        o.req = req;
    }
    o.c = pos + 1 > 0 ? pos + 1 : 0;
    return o;
}

__device__ inline int64_t clamp_count(int64_t v, int64_t hi)
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
__device__ inline uint32_t order_image(uint32_t bits)
{
    return bits ^ ((uint32_t)((int32_t)bits >> 31) | 0x80000000u);
}

struct KeyF32 {
    using T = uint64_t;
    static constexpr int kBits = 2 + 32 + kRidBits;   // 47
    __device__ static T scored(uint32_t bits, int id)
    {
        return (T(1) << 45) | (T(order_image(bits)) << kRidBits) | T(kRidMask - (uint32_t)id);
    }
    __device__ static T forced(int id) { return (T(2) << 45) | T(kRidMask - (uint32_t)id); }
};

struct KeyBF16 {
    using T = uint32_t;
    static constexpr int kBits = 2 + 16 + kRidBits;   // 31
    __device__ static T scored(uint32_t bits, int id)
    {
        return (1u << 29) | ((order_image(bits) >> 16) << kRidBits) | (kRidMask - (uint32_t)id);
    }
    __device__ static T forced(int id) { return (2u << 29) | (kRidMask - (uint32_t)id); }
};

template <typename T>
__device__ inline int key_block(T key)
{
    return key ? (int)(kRidMask - (uint32_t)(key & kRidMask)) : -1;
}

// ---------------------------------------------------------------------------
// Wave primitives (all 64 lanes must be active).
// ---------------------------------------------------------------------------
__device__ inline int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ inline uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ inline int count(bool p) { return __builtin_popcountll(ballot(p)); }

__device__ inline uint32_t readlane(uint32_t v, int l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

__device__ inline uint64_t readlane(uint64_t v, int l)
{
    const uint32_t lo = readlane((uint32_t)v, l);
    const uint32_t hi = readlane((uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

__device__ inline int shfl(int v, int src_lane)
{
    return __builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}

// Largest x such that at least k lanes hold a key >= x: the k-th largest key of
// the wave when at least k keys are nonzero, else 0. Bit-serial over the key
// width, one ballot per bit; the prefix stays wave-uniform (scalar registers).
template <typename T, int NB>
__device__ inline T wave_kth(T key, int k)
{
    T prefix = 0;
#pragma unroll
    for (int bit = NB - 1; bit >= 0; --bit) {
        const T cand = prefix | (T(1) << bit);
        if (count(key >= cand) >= k) prefix = cand;
    }
    return prefix;
}

// One merge step of the exact wave top-k. Candidates are S keys per lane plus the
// running result `carry` (lanes 0..k-1 hold the current top-k in rank order, the
// other lanes 0). Keys are unique unless 0. Returns the new top-k of all of them in
// rank order: lane r holds the rank-r key, lanes past the valid count hold 0.
template <typename T, int NB, int S>
__device__ inline T wave_topk_merge(const T (&key)[S], T carry, int k)
{
    T prefix = 0;
#pragma unroll
    for (int bit = NB - 1; bit >= 0; --bit) {
        const T cand = prefix | (T(1) << bit);
        int n = count(carry >= cand);
#pragma unroll
        for (int s = 0; s < S; ++s) n += count(key[s] >= cand);
        if (n >= k) prefix = cand;
    }
    // prefix is the k-th largest key, or 0 with fewer than k candidates.
    const T th = prefix ? prefix : T(1);
    const int lane = lane_id();
    T out = 0;
    // Each selected key's rank is the number of keys above it; every key above a
    // selected key is itself selected, so ranks are 0 .. selected-1.
    auto place = [&](T v) {
        uint64_t m = ballot(v >= th);
        while (m) {
            const int l = __builtin_ctzll(m);
            m &= m - 1;
            const T x = readlane(v, l);
            int r = count(carry > x);
#pragma unroll
            for (int s = 0; s < S; ++s) r += count(key[s] > x);
            if (lane == r) out = x;
        }
    };
    place(carry);
#pragma unroll
    for (int s = 0; s < S; ++s) place(key[s]);
    return out;
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
__device__ inline void emit_table_group(int id, bool active, int64_t c, const int32_t* bt_row,
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
