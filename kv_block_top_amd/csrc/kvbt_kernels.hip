// kvbt_kernels.hip -- HIP kernels for gfx950 (CDNA4, wave64) of the top-k KV-block
// selector and the page-16 sparse block table, and their launchers.
//
// Two selector kernels:
//   * wave kernel: one wavefront per (row, head), several per workgroup. A 128-tile
//     chunk sits two tiles per lane; a bitonic network sorts the 128 rank keys and
//     the first 16 are merged into the running result. A row longer than 128 tiles
//     loops over chunks. With max_block <= 128 it handles every row; otherwise it
//     handles only the rows of at most 128 causal blocks and leaves the rest to:
//   * stream kernel: persistent 256-thread workgroups that walk the rows of more than
//     128 causal blocks. A row is streamed once from HBM with 16-byte loads into
//     registers. Each lane takes the exact maximum (in rank order) of its elements;
//     the k-th largest maximum over groups of lanes is a threshold the row's top-k
//     must reach. Only the lanes whose maximum reaches it (about k of them) copy their
//     elements to LDS, where wavefront 0 picks the candidates and sorts them with the
//     forced blocks. As soon as a row is staged, every wavefront issues the loads of
//     the workgroup's next row, so they are in flight while wavefront 0 finishes the
//     current row. Row metadata is read 64 rows ahead, one row per lane.
//     Rows with mass ties, which could overflow the staging, fall back inside the same
//     launch to a filter on exact unique keys that always fits in LDS.
// Results never depend on which kernel handles a row. Both can emit the page-16 table
// in the same pass (the fused call).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

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
    int rhpb;        // wave kernel: (row, head) pairs per workgroup
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
__device__ __forceinline__ uint32_t load_bits(const void* p, int64_t off)
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
// value past nvp). Forced blocks get the forced key. Returns lane r = rank-r key
// for r < 16, 0 past the valid count.
template <bool BF16>
__device__ __forceinline__ typename KeyOf<BF16>::T wave_select_row(const void* scores, int64_t row_off,
                                                          int nvp, int ni, int nl,
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
        T top;
        if (nvp - base <= kWave) {
            top = sort64_desc(k[0]);
        } else {
            sort128_desc(k[0], k[1]);
            top = k[0];
        }
        carry = base == 0 ? (lane < 16 ? top : T(0)) : merge_top16(carry, top);
    }
    return carry;
}

// ---------------------------------------------------------------------------
// Wave kernel
// ---------------------------------------------------------------------------
template <bool FUSED>
__device__ __forceinline__ int row_count(const SelArgs& a, int64_t t, int64_t& c, int& req)
{
    if constexpr (FUSED) {
        const RowInfo ri = row_info(a.rows, t);
        c = ri.c;
        req = ri.req;
        return (int)clamp_count((c + kBlockTokens - 1) / kBlockTokens, a.M);
    } else {
        c = 0;
        req = -1;
        return (int)clamp_count(a.rows.num_valid_pages[t], a.M);
    }
}

// SHORT_ONLY: handle only rows of at most 128 causal blocks (the stream kernel takes
// the others); the row metadata is then read before any score.
template <bool BF16, bool FUSED, bool SHORT_ONLY>
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

    uint32_t r0 = 0, r1 = 0;
    if constexpr (!SHORT_ONLY) {
        // The first chunk's tiles are fetched before the row metadata is known, so the
        // two memory round trips overlap; tiles past the causal count are masked below.
        r0 = lane < a.M ? load_bits<BF16>(a.scores, row_off + lane) : 0u;
        r1 = lane + kWave < a.M ? load_bits<BF16>(a.scores, row_off + lane + kWave) : 0u;
    }
    int64_t c;
    int req;
    const int nvp = row_count<FUSED>(a, t, c, req);
    if constexpr (SHORT_ONLY) {
        if (nvp > 2 * kWave) return;
        r0 = lane < nvp ? load_bits<BF16>(a.scores, row_off + lane) : 0u;
        r1 = lane + kWave < nvp ? load_bits<BF16>(a.scores, row_off + lane + kWave) : 0u;
    }

    const T top = wave_select_row<BF16>(a.scores, row_off, nvp, a.num_init, a.num_local, r0, r1);
    const int id = key_block(top);
    if (lane < a.topk) a.out_idx[rh * a.topk + lane] = id;
    if constexpr (FUSED) {
        const int32_t* bt_row = req >= 0 ? a.block_table + (int64_t)req * a.max_blocks : nullptr;
        emit_table_sorted(id, c, bt_row, a.max_blocks, a.topk,
                          a.out_table + rh * (int64_t)a.topk * kPagesPerBlock, a.out_ctx + rh,
                          a.table_vec != 0);
    }
}

// ---------------------------------------------------------------------------
// Workgroup path
// ---------------------------------------------------------------------------
template <bool BF16, int VEC>
__device__ __forceinline__ void load_vec(const void* scores, int64_t row_off, int e0, uint32_t (&out)[VEC])
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

// Row visited by a stream workgroup.
struct StreamRow {
    int64_t rh;    // (row, head) index
    int nvp;       // causal blocks (bounded to max_k_tiles)
    int64_t c;     // causal length in tokens (fused call)
    int req;       // request (fused call)
};

// The rows of more than 128 causal blocks that stream workgroup g visits:
// it = g, g + G, g + 2G, ... (G = grid size) with (row, head) index total - 1 - it, so
// the last rows of a unified buffer (prefill rows with the longest contexts) come first.
// The metadata of 64 rows of the sequence is read at once, one row per lane; every
// wavefront keeps its own copy so that loop control stays uniform without LDS.
template <bool FUSED>
struct RowWalker {
    const SelArgs& a;
    int64_t total, G, wb;
    int w_nvp = 0;
    int64_t w_c = 0;
    int w_req = -1;
    uint64_t w_mask = 0;

    __device__ __forceinline__ RowWalker(const SelArgs& args)
        : a(args), total(args.T * args.H), G(gridDim.x), wb(blockIdx.x)
    {
        load();
    }
    __device__ __forceinline__ void load()
    {
        const int64_t it = wb + (int64_t)lane_id() * G;
        w_nvp = 0;
        w_c = 0;
        w_req = -1;
        if (it < total) w_nvp = row_count<FUSED>(a, (total - 1 - it) / a.H, w_c, w_req);
        w_mask = ballot(it < total && w_nvp > 2 * kWave);
    }
    __device__ __forceinline__ bool next(StreamRow& r)
    {
        while (w_mask == 0) {
            wb += (int64_t)kWave * G;
            if (wb >= total) return false;
            load();
        }
        const int l = __builtin_ctzll(w_mask);
        w_mask &= w_mask - 1;
        r.rh = total - 1 - (wb + (int64_t)l * G);
        r.nvp = (int)readlane((uint32_t)w_nvp, l);
        r.c = (int64_t)readlane((uint64_t)w_c, l);
        r.req = (int)readlane((uint32_t)w_req, l);
        return true;
    }
};

// LDS of a stream workgroup.
template <typename T, int EPT>
struct StreamShared {
    static constexpr int STAGE = 64;                     // staged lanes (fast path)
    static constexpr int MCAP = 128;                     // candidate keys (fast path)
    static constexpr int CAP = 4 * kMaxTopk * EPT;       // exact-key fallback candidates
    static constexpr int FAST_BYTES = STAGE * EPT * 4 + MCAP * (int)sizeof(T);
    static constexpr int SLOW_BYTES = CAP * (int)sizeof(T);
    static constexpr int BUF_BYTES = FAST_BYTES > SLOW_BYTES ? FAST_BYTES : SLOW_BYTES;
    alignas(16) unsigned char buf[BUF_BYTES];   // staged rows [STAGE][EPT] + candidates [MCAP],
                                                // or exact-key candidates [CAP]
    uint32_t gmax[64];
    int stage_tid[STAGE];
    int nstage;      // staged lanes
    int ncand;       // candidates found in the staged lanes
    int count;       // exact-key candidates
    int overflow;    // staging overflowed: exact-key path
    int mover;       // more than MCAP candidates: the selector sorts every staged element
    uint32_t tau;
    __device__ __forceinline__ uint32_t* stage() { return reinterpret_cast<uint32_t*>(buf); }
    __device__ __forceinline__ T* mcand() { return reinterpret_cast<T*>(buf + STAGE * EPT * 4); }
    __device__ __forceinline__ T* cand() { return reinterpret_cast<T*>(buf); }
};

// Key of staged element i (row slot i / EPT, element slot i % EPT), or 0 unless it is a
// non-forced causal element whose rank image reaches tau.
template <typename KT, int VEC, int EPT>
__device__ __forceinline__ typename KT::T staged_key(const uint32_t* stage, const int* stage_tid,
                                                     int i, int nvp, int ni, int lo_local,
                                                     uint32_t tau)
{
    const int sl = i / EPT, p = i - sl * EPT;
    const uint32_t bits = stage[i];
    const int e = ((p / VEC) * 256 + stage_tid[sl]) * VEC + (p % VEC);
    const bool forced = e < ni || e >= lo_local;
    const bool cand = e < nvp && !forced && max(order_image(bits), 1u) >= tau;
    return cand ? KT::scored(bits, e) : typename KT::T(0);
}

// Streaming wavefronts 0-3 (256 lanes). Element e of a row sits in chunk
// j = e / (256 VEC), lane tid = (e / VEC) % 256, slot v = e % VEC. Per row: load,
// per-lane maximum, group maxima (barrier A), threshold from wavefront 4 (barrier B),
// staging of the lanes that reach it (barrier C); then the next row's loads are
// issued and, while they are in flight, the staged elements are scanned for the
// candidates (barrier D).
template <bool BF16, int VEC, int NCH, bool FUSED>
__device__ __forceinline__ void stream_role(const SelArgs& a,
                                            StreamShared<typename KeyOf<BF16>::T, VEC * NCH>& sh)
{
    using KT = KeyOf<BF16>;
    using T = typename KT::T;
    using SH = StreamShared<T, VEC * NCH>;
    constexpr int EPT = VEC * NCH;
    constexpr int CH = 256 * VEC;
    const int tid = (int)threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int topk = a.topk, ni = a.num_init, nl = a.num_local;

    RowWalker<FUSED> walk(a);
    StreamRow cur;
    if (!walk.next(cur)) return;
    uint32_t raw[NCH][VEC];
    auto issue_loads = [&](const StreamRow& r) {
        const int64_t row_off = r.rh * (int64_t)a.M;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int e0 = (j * 256 + tid) * VEC;
#pragma unroll
            for (int v = 0; v < VEC; ++v) raw[j][v] = 0x80000000u;
            if (j * CH < r.nvp && e0 < r.nvp) load_vec<BF16, VEC>(a.scores, row_off, e0, raw[j]);
        }
    };
    issue_loads(cur);

    for (;;) {
        const int nvp = cur.nvp;
        const int lo_local = nvp - nl;
        // Exact per-lane maximum in rank order: as signed integers, non-negative score
        // patterns keep their order and negative ones reverse it, so the maximum is the
        // largest pattern if it is non-negative, else the smallest.
        int mx = INT32_MIN, mn = INT32_MAX;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            if ((j + 1) * CH <= nvp) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    mx = max(mx, (int)raw[j][v]);
                    mn = min(mn, (int)raw[j][v]);
                }
            } else if (j * CH < nvp) {
                const int e0 = (j * 256 + tid) * VEC;
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const bool ok = e0 + v < nvp;
                    mx = max(mx, ok ? (int)raw[j][v] : INT32_MIN);
                    mn = min(mn, ok ? (int)raw[j][v] : INT32_MAX);
                }
            }
        }
        // rank image of the lane maximum, at least 1 so that 0 means "no element"
        const uint32_t lkey =
            tid * VEC < nvp ? max(order_image(mx >= 0 ? (uint32_t)mx : (uint32_t)mn), 1u) : 0u;
        // Group maxima over gs adjacent lanes (1, 2 or 4: the lanes holding elements fit
        // 64 groups). The k-th largest group maximum is reached by at least k elements,
        // so every element of the top-k reaches it.
        const int L = min(256, (nvp + VEC - 1) / VEC);
        const int gs = L <= 64 ? 1 : (L <= 128 ? 2 : 4);
        uint32_t gm = lkey;
        if (gs >= 2) gm = max(gm, xor_lane<1>(gm));
        if (gs == 4) gm = max(gm, xor_lane<2>(gm));
        if ((tid & (gs - 1)) == 0 && tid / gs < 64) sh.gmax[tid / gs] = gm;
        __syncthreads();                                           // A
        __syncthreads();                                           // B
        const uint32_t tau = sh.tau;
        // stage the lanes whose maximum reaches tau (about topk of them)
        {
            const bool cand_lane = lkey >= tau;
            const uint64_t m = ballot(cand_lane);
            int wbase = 0;
            if (lane == 0 && m != 0) wbase = atomicAdd(&sh.nstage, __builtin_popcountll(m));
            wbase = __builtin_amdgcn_readfirstlane(wbase);
            const int slot = wbase + (int)__builtin_amdgcn_mbcnt_hi(
                                         (uint32_t)(m >> 32),
                                         __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (cand_lane) {
                if (slot < SH::STAGE) {
                    sh.stage_tid[slot] = tid;
                    uint32_t* dst = sh.stage() + slot * EPT;
#pragma unroll
                    for (int j = 0; j < NCH; ++j)
#pragma unroll
                        for (int v = 0; v < VEC; ++v) dst[j * VEC + v] = raw[j][v];
                } else {
                    sh.overflow = 1;
                }
            }
        }
        __syncthreads();                                           // C
        const bool overflow = sh.overflow != 0;
        StreamRow nxt;
        const bool more = walk.next(nxt);
        if (more) issue_loads(nxt);    // in flight during the rest of this row

        if (overflow) {
            // Mass ties: exact unique keys. The k-th largest per-lane maximum is met by
            // exactly topk lanes of a wavefront, so at most topk * EPT candidates each.
            // This rare path re-reads the row (just streamed, so cache-resident) in
            // rolled loops instead of holding a key per element in registers.
            __syncthreads();                                       // S1: count reset
            const int64_t row_off = cur.rh * (int64_t)a.M;
            T lk = 0;
#pragma unroll 1
            for (int j = 0; j < NCH && j * CH < nvp; ++j) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const int e = (j * 256 + tid) * VEC + v;
                    if (e < nvp) {
                        const T k = KT::scored(load_bits<BF16>(a.scores, row_off + e), e);
                        lk = k > lk ? k : lk;
                    }
                }
            }
            T tk = wave_kth<T, KT::kBits>(lk, topk);
            if (tk == 0) tk = 1;
            if (lk >= tk) {
#pragma unroll 1
                for (int j = 0; j < NCH && j * CH < nvp; ++j) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) {
                        const int e = (j * 256 + tid) * VEC + v;
                        const bool forced = e < ni || e >= lo_local;
                        if (e < nvp && !forced) {
                            const T k = KT::scored(load_bits<BF16>(a.scores, row_off + e), e);
                            if (k >= tk) {
                                const int pos = atomicAdd(&sh.count, 1);
                                if (pos < SH::CAP) sh.cand()[pos] = k;
                            }
                        }
                    }
                }
            }
        } else {
            // the staged elements that reach tau are the candidates
            const int n = min(sh.nstage, SH::STAGE) * EPT;
            for (int i0 = wave * kWave; i0 < n; i0 += 4 * kWave) {
                const int i = i0 + lane;
                const T k = i < n ? staged_key<KT, VEC, EPT>(sh.stage(), sh.stage_tid, i, nvp, ni,
                                                            lo_local, tau)
                                  : T(0);
                const uint64_t cm = ballot(k != 0);
                if (cm != 0) {
                    int base = 0;
                    if (lane == 0) base = atomicAdd(&sh.ncand, __builtin_popcountll(cm));
                    base = __builtin_amdgcn_readfirstlane(base);
                    const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                               (uint32_t)(cm >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)cm, 0u));
                    if (k != 0) {
                        if (pos < SH::MCAP) sh.mcand()[pos] = k;
                        else sh.mover = 1;
                    }
                }
            }
        }
        __syncthreads();                                           // D
        if (!more) return;
        cur = nxt;
    }
}

// Table row of one (row, head) from its selected blocks with their physical ids already
// fetched: lane r < topk holds the rank-r block id (-1 if none) and its physical block.
// Kept ids (below the causal block count and max_blocks) are sorted ascending with a
// 16-lane network that carries the source lane; kept block r then owns entries
// 8r..8r+7 (only the last causal block can be partly filled, and it is the largest id).
__device__ __forceinline__ void emit_table_phys(int id, int phys, int64_t c, int max_blocks,
                                                int topk, int32_t* table_row, int32_t* ctx_out,
                                                bool vec_store)
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
    if (lane < topk) {
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

// Selecting wavefront 4: threshold (between barriers A and B); after the candidates are
// found (barrier D), the exact top-k of the forced blocks and the candidates, the
// outputs and the table row -- while wavefronts 0-3 already load the next row. With at
// most 64 keys in all, each lane fetches the physical block of its key before a single
// 64-lane sort; the key carries its lane, so the fetch is off the critical path.
template <bool BF16, int VEC, int NCH, bool FUSED>
__device__ __forceinline__ void select_role(const SelArgs& a,
                                            StreamShared<typename KeyOf<BF16>::T, VEC * NCH>& sh)
{
    using KT = KeyOf<BF16>;
    using T = typename KT::T;
    using SH = StreamShared<T, VEC * NCH>;
    constexpr int EPT = VEC * NCH;
    const int lane = lane_id();
    const int topk = a.topk, ni = a.num_init, nl = a.num_local;

    RowWalker<FUSED> walk(a);
    StreamRow cur;
    if (!walk.next(cur)) return;
    for (;;) {
        const int nvp = cur.nvp;
        const int lo_local = nvp - nl;
        __syncthreads();                                           // A
        {
            const uint32_t sorted = sort64_desc(sh.gmax[lane]);
            const uint32_t t = readlane(sorted, topk - 1);
            if (lane == 0) {
                sh.tau = t ? t : 1u;
                sh.nstage = 0;
                sh.ncand = 0;
                sh.overflow = 0;
                sh.mover = 0;
            }
        }
        __syncthreads();                                           // B
        __syncthreads();                                           // C
        const uint32_t tau = sh.tau;
        const bool overflow = sh.overflow != 0;
        if (overflow) {
            if (lane == 0) sh.count = 0;
            __syncthreads();                                       // S1
        }
        __syncthreads();                                           // D
        const int nf = ni + nl;      // disjoint: nvp > 128 >= ni + nl
        auto forced_key = [&](int i) { return KT::forced(i < ni ? i : lo_local + (i - ni)); };
        const int32_t* bt_row = FUSED && cur.req >= 0
                                    ? a.block_table + (int64_t)cur.req * a.max_blocks
                                    : nullptr;
        const int nc = overflow ? 0 : sh.ncand;
        if (!overflow && sh.mover == 0 && nf + nc <= kWave) {
            // one key per lane, with its lane below the key bits
            const T key = lane < nf ? forced_key(lane)
                                    : (lane < nf + nc ? sh.mcand()[lane - nf] : T(0));
            const int kid = key_block(key);
            int phys = 0;
            if constexpr (FUSED)
                if (bt_row != nullptr && kid >= 0 && kid < a.max_blocks) phys = bt_row[kid];
            const uint64_t sorted = sort64_desc(((uint64_t)key << 6) | (uint64_t)lane);
            const int id = key_block((T)(sorted >> 6));
            if (lane < topk) a.out_idx[cur.rh * topk + lane] = id;
            if constexpr (FUSED) {
                const int ph = __builtin_amdgcn_ds_bpermute((int)(sorted & 63u) << 2, phys);
                emit_table_phys(id, ph, cur.c, a.max_blocks, topk,
                                a.out_table + cur.rh * (int64_t)topk * kPagesPerBlock,
                                a.out_ctx + cur.rh, a.table_vec != 0);
            }
        } else {
            T top;
            if (overflow) {
                const int n = min(sh.count, SH::CAP);
                T* cand = sh.cand();
                top = topk16_of_list<T>(nf + n, [&](int i) {
                    return i < nf ? forced_key(i) : cand[i - nf];
                });
            } else if (sh.mover == 0) {
                T* mcand = sh.mcand();
                top = topk16_of_list<T>(nf + nc, [&](int i) {
                    return i < nf ? forced_key(i) : mcand[i - nf];
                });
            } else {
                // many equal scores at the threshold: sort every staged element
                const int n = min(sh.nstage, SH::STAGE) * EPT;
                const uint32_t* stage = sh.stage();
                top = topk16_of_list<T>(nf + n, [&](int i) {
                    return i < nf ? forced_key(i)
                                  : staged_key<KT, VEC, EPT>(stage, sh.stage_tid, i - nf, nvp, ni,
                                                             lo_local, tau);
                });
            }
            const int id = key_block(top);
            if (lane < topk) a.out_idx[cur.rh * topk + lane] = id;
            if constexpr (FUSED) {
                emit_table_sorted(id, cur.c, bt_row, a.max_blocks, topk,
                                  a.out_table + cur.rh * (int64_t)topk * kPagesPerBlock,
                                  a.out_ctx + cur.rh, a.table_vec != 0);
            }
        }
        StreamRow nxt;
        if (!walk.next(nxt)) return;
        cur = nxt;
    }
}

// Wavefronts per SIMD the register budget is tuned for (8 allows 64 VGPRs, 6 allows
// 80, 5 allows 96, 2 allows 256): the most each instance reaches without spilling.
template <bool BF16, int VEC, int NCH>
constexpr int stream_waves_per_simd()
{
    if (VEC == 1) return NCH <= 8 ? 8 : (NCH <= 16 ? 5 : 2);
    if (BF16) return NCH <= 2 ? 8 : 6;
    return NCH <= 4 ? 8 : 5;
}

template <bool BF16, int VEC, int NCH, bool FUSED>
__global__ __launch_bounds__(320, (stream_waves_per_simd<BF16, VEC, NCH>()))
void select_stream_kernel(SelArgs a)
{
    __shared__ StreamShared<typename KeyOf<BF16>::T, VEC * NCH> sh;
    if (threadIdx.x >= 256)
        select_role<BF16, VEC, NCH, FUSED>(a, sh);
    else
        stream_role<BF16, VEC, NCH, FUSED>(a, sh);
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

template <bool BF16, bool FUSED, bool SHORT_ONLY>
hipError_t launch_wave(const SelArgs& args, int rhpb, hipStream_t stream)
{
    SelArgs s = args;
    s.rhpb = rhpb;
    const int64_t total = s.T * s.H;
    const int64_t blocks = (total + rhpb - 1) / rhpb;
    hipLaunchKernelGGL((select_wave_kernel<BF16, FUSED, SHORT_ONLY>), dim3((unsigned)blocks),
                       dim3(kWave * rhpb), 0, stream, s);
    return hipGetLastError();
}

// Workgroups of the stream kernel that fit the device at once (cached per device and
// kernel instance; the device's compute-unit count and the kernel's occupancy do not
// change while the process runs).
template <typename K>
int64_t stream_grid(K kernel, int64_t total)
{
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    const auto key = std::make_pair(dev, reinterpret_cast<const void*>(kernel));
    int64_t slots;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(key);
        if (it != cache.end()) {
            slots = it->second;
        } else {
            int cus = 0, per_cu = 0;
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 320, 0) != hipSuccess)
                return -1;
            slots = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
            cache[key] = slots;
        }
    }
    return total < slots ? total : slots;
}

template <bool BF16, int VEC, int NCH, bool FUSED>
hipError_t launch_stream_one(const SelArgs& s, hipStream_t stream)
{
    auto kernel = select_stream_kernel<BF16, VEC, NCH, FUSED>;
    const int64_t grid = stream_grid(kernel, s.T * s.H);
    if (grid <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(320), 0, stream, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // rows of at most 128 causal blocks: one wavefront each
    return launch_wave<BF16, FUSED, true>(s, 4, stream);
}

template <bool BF16, int VEC, bool FUSED>
hipError_t launch_stream_vec(const SelArgs& s, int chunks, hipStream_t stream)
{
    switch (chunks) {
        case 1: return launch_stream_one<BF16, VEC, 1, FUSED>(s, stream);
        case 2: return launch_stream_one<BF16, VEC, 2, FUSED>(s, stream);
        case 4: return launch_stream_one<BF16, VEC, 4, FUSED>(s, stream);
        case 8: if constexpr (VEC * 8 <= 32) return launch_stream_one<BF16, VEC, 8, FUSED>(s, stream);
                break;
        case 16: if constexpr (VEC * 16 <= 32) return launch_stream_one<BF16, VEC, 16, FUSED>(s, stream);
                 break;
        case 32: if constexpr (VEC * 32 <= 32) return launch_stream_one<BF16, VEC, 32, FUSED>(s, stream);
                 break;
        default: break;
    }
    return hipErrorInvalidValue;
}

template <bool BF16, bool FUSED>
hipError_t launch_stream(const SelArgs& s, int vec, int chunks, hipStream_t stream)
{
    if (vec == 1) return launch_stream_vec<BF16, 1, FUSED>(s, chunks, stream);
    if constexpr (BF16) {
        if (vec == 8) return launch_stream_vec<true, 8, FUSED>(s, chunks, stream);
    } else {
        if (vec == 4) return launch_stream_vec<false, 4, FUSED>(s, chunks, stream);
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
    s.table_vec = ((uintptr_t)l.out_table % 16) == 0;
    const bool bf16 = l.dtype == KVBT_BF16;

    if (l.policy.path == 0) {
        if (bf16) return l.fused ? launch_wave<true, true, false>(s, s.rhpb, stream)
                                 : launch_wave<true, false, false>(s, s.rhpb, stream);
        return l.fused ? launch_wave<false, true, false>(s, s.rhpb, stream)
                       : launch_wave<false, false, false>(s, s.rhpb, stream);
    }
    int vec = l.policy.vec;
    int chunks = l.policy.chunks;
    if (vec > 1 && ((uintptr_t)l.scores % 16) != 0) {
        vec = 1;
        chunks = pow2_at_least((l.M + 255) / 256);
    }
    if (bf16) return l.fused ? launch_stream<true, true>(s, vec, chunks, stream)
                             : launch_stream<true, false>(s, vec, chunks, stream);
    return l.fused ? launch_stream<false, true>(s, vec, chunks, stream)
                   : launch_stream<false, false>(s, vec, chunks, stream);
}

hipError_t stream_slots(int dtype, int M, bool fused, int64_t* slots)
{
    kvbt_policy p;
    if (kvbt_launch_policy(M, M, dtype, 1, 1, 1, &p) != KVBT_OK) return hipErrorInvalidValue;
    const int64_t huge = (int64_t)1 << 40;
    SelArgs s = {};
    s.T = huge;
    s.H = 1;
    const bool bf16 = dtype == KVBT_BF16;
    int64_t g = -1;
    auto query = [&](auto kernel) { g = stream_grid(kernel, huge); };
    if (bf16) {
        if (p.vec == 8 && p.chunks == 4) fused ? query(select_stream_kernel<true, 8, 4, true>)
                                               : query(select_stream_kernel<true, 8, 4, false>);
        else if (p.vec == 8 && p.chunks == 1) fused ? query(select_stream_kernel<true, 8, 1, true>)
                                                    : query(select_stream_kernel<true, 8, 1, false>);
    } else {
        if (p.vec == 4 && p.chunks == 8) fused ? query(select_stream_kernel<false, 4, 8, true>)
                                               : query(select_stream_kernel<false, 4, 8, false>);
    }
    *slots = g;
    return g > 0 ? hipSuccess : hipErrorInvalidValue;
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
