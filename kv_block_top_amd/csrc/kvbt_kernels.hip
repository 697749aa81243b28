// kvbt_kernels.hip -- HIP kernels for gfx950 (CDNA4, wave64) of the top-k KV-block
// selector and the page-16 sparse block table, and their launchers.
//
// Selector launch paths (the policy only changes the geometry; results are the same
// on every path):
//   0  short rows (max_block <= 128): one wavefront per (row, head), several per
//      workgroup, no barrier; the tiles sit two per lane and a bitonic network picks
//      the best 16 of the 128 rank keys (rows longer than the hint loop over 128-tile
//      chunks);
//   1  long rows: one wavefront per (row, head). Rows of at most 128 tiles take the
//      short-row code; bf16 rows of 129..512 tiles load all their 128-tile chunks at
//      once, take each chunk's top 16 independently and merge the lists. Longer rows
//      (and fp32 rows past 128 tiles) are streamed from HBM in chunks of
//      64 lanes x 4 loads of 16 bytes (nontemporal buffer loads bounded by the row's
//      causal length), two chunks in flight. The four lanes of a quad read one
//      contiguous 64-byte segment per load; the exact maximum (in rank order) of each
//      segment is its group key, and each lane keeps the key of one group per chunk.
//      The k-th largest of the maxima of what each lane loaded is a threshold that every
//      element of the row's top-k reaches, and only the groups whose key reaches it
//      (about k of them) can hold such elements. Those segments are read again, the
//      elements that reach the threshold are compacted, and one sort with the forced
//      blocks (over 32 lanes when they fit, else 64) gives the result; each lane
//      fetches the block-table entry of its key before that sort. Rows with mass ties
//      at the threshold fall back, in the same wavefront, to an exact top-k over the
//      whole row, 128 elements at a time;
//   2  small batches of long rows: a workgroup per (row, head), one wavefront per chunk,
//      each chunk kept in registers and its hits staged in LDS, merged in the workgroup;
//   3  rows beyond 8192 tiles: 24-bit block ids in the keys, a workgroup per (row,
//      head), one wavefront per 8192-tile segment (each as in path 1; at most 8
//      wavefronts, each taking every 8th segment of longer rows), merged;
//   4  few (row, head) pairs with a caller's workspace: a row split across workgroups,
//      each slice's top-16 merged by the last slice to arrive, which leaves the
//      workspace zeroed;
//   5  topk above 16: one wavefront per (row, head) keeps a running top-64.
// All sorting networks exchange lanes through DPP and gfx950 permlane swaps only, and
// independent networks run stage by stage together. The kernels of paths 0-4 take what
// a wavefront needs before its first loads as leading scalar arguments, which the code
// object has preloaded into scalar registers at wave launch (see row_count_lead), and
// divide by launch-fixed counts with a multiply and a shift (kvbt_divide.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
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
    int rhpb;        // wave kernel: (row, head) pairs per workgroup
    int table_vec;   // out_table is 16-byte aligned
    int64_t front;   // streaming launch: (row, head) pairs visited first (decode rows x H)
    // cross-workgroup split (path 4): the caller's workspace
    uint32_t* ws_count;    // [T * H] arrival counters (one per 256-byte line), zero between calls
    uint64_t* ws_lists;    // [T * H, slices, 16] each slice's scored top-16 keys
    int slices;            // slices (workgroups) per (row, head)
    uint32_t h_mul, h_shift;   // make_divisor(H): (row, head) pair -> row
};

struct TabArgs {
    const int32_t* idx;
    int64_t T;
    int H;
    uint32_t h_mul, h_shift;   // make_divisor(H)
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

// Rank keys: compact keys for rows of at most 8192 tiles, 24-bit block ids beyond.
template <bool BF16, bool WIDE = false>
using KeyOf = typename std::conditional<
    WIDE, KeyWide, typename std::conditional<BF16, KeyBF16, KeyF32>::type>::type;

// Tiles per segment of a row longer than the fast path's 8192 tiles.
constexpr int kSegmentTiles = 8192;

// bf16 rows of 129 up to this many tiles take the preloaded-chunks code on the streaming
// launch path (kernels with NC > 0) instead of the threshold stream (with fp32 scores
// the 64-bit sorts make it slower than the stream).
constexpr int kChunkRowMax = 512;

// Exact top-k of a row of at most 128 * NCH tiles whose 2 * NCH tiles per lane
// (lane + 64 s) are already loaded (zero past nvp): the top 16 of each 128-tile chunk
// come from independent networks run stage by stage together, and the chunks' lists are
// merged pairwise, the merges of one level together. Same result as wave_select_row.
template <bool BF16, int NCH>
__device__ __forceinline__ typename KeyOf<BF16>::T wave_select_chunks(int nvp, int ni, int nl,
                                                                    const uint32_t (&raw)[2 * NCH])
{
    using KT = KeyOf<BF16>;
    using T = typename KT::T;
    static_assert((NCH & (NCH - 1)) == 0, "chunks are merged pairwise");
    const int lane = lane_id();
    const int lo_local = nvp - nl;
    T a[NCH], b[NCH];
#pragma unroll
    for (int s = 0; s < 2 * NCH; ++s) {
        const int e = s * kWave + lane;
        const bool forced = e < ni || e >= lo_local;
        const T k = e < nvp ? (forced ? KT::forced(e) : KT::scored(raw[s], e)) : T(0);
        if (s & 1) b[s >> 1] = k;
        else a[s >> 1] = k;
    }
    top16_of_128_n<NCH>(a, b);
    // a[c]: chunk c's best 16 in rank order
#pragma unroll
    for (int c = 0; c < NCH; ++c) a[c] = lane < 16 ? a[c] : T(0);
    return fold_top16_n<NCH>(a);
}

// Exact top-k of one (row, head) by one wavefront, over tiles [0, nvp) in chunks
// of 128. r0/r1 are the row's tiles lane and lane+64 (loaded by the caller, any
// value past nvp). Forced blocks get the forced key. Returns lane r = rank-r key
// for r < 16, 0 past the valid count.
template <bool BF16, bool WIDE = false>
__device__ __forceinline__ typename KeyOf<BF16, WIDE>::T wave_select_row(const void* scores, int64_t row_off,
                                                          int nvp, int ni, int nl,
                                                          uint32_t r0, uint32_t r1)
{
    using KT = KeyOf<BF16, WIDE>;
    using T = typename KT::T;
    const int lane = lane_id();
    const int lo_local = nvp - nl;
    // best 16 of the chunk of tiles base .. base + 127 (a, b: its tiles lane, lane + 64)
    auto chunk_top = [&](int base, uint32_t a, uint32_t b) -> T {
        T k[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int e = base + s * kWave + lane;
            const bool forced = e < ni || e >= lo_local;
            k[s] = e < nvp ? (forced ? KT::forced(e) : KT::scored(s ? b : a, e)) : T(0);
        }
        return top16_of_short(k[0], k[1], nvp - base);
    };
    T carry = chunk_top(0, r0, r1);
    carry = lane < 16 ? carry : T(0);
    // rows past one chunk are rare where this runs (the short-row launch, whose rows
    // the hint puts at 128 blocks or less): their loop is laid out away from the path
    // of the others
    if (__builtin_expect(nvp > 2 * kWave, 0)) {
        for (int base = 2 * kWave; base < nvp; base += 2 * kWave) {
            uint32_t raw[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int e = base + s * kWave + lane;
                raw[s] = e < nvp ? load_bits<BF16>(scores, row_off + e) : 0u;
            }
            carry = merge_top16(carry, chunk_top(base, raw[0], raw[1]));
        }
    }
    return carry;
}


// ---------------------------------------------------------------------------
// Long rows: one wavefront streams the row
// ---------------------------------------------------------------------------
// 32-bit words held per load: 16-byte loads keep their four words packed (two bf16
// scores per word); single-element loads hold the element widened to binary32.
template <int VEC>
constexpr int load_words() { return VEC == 1 ? 1 : 4; }

// Reads of one row through a buffer resource whose range is the row's first `nbytes`
// bytes: a load outside the range returns zeros and makes no memory access, so loads
// past the causal tiles need neither a branch nor an address clamp. Each load fetches
// VEC elements at element e0; NT marks a streaming load whose lines need not stay in the
// caches.
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

template <bool BF16, int VEC>
struct RowReader {
    static constexpr int kElem = BF16 ? 2 : 4;
    __amdgpu_buffer_rsrc_t rsrc;

    __device__ __forceinline__ RowReader(const void* row, int nbytes)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, nbytes,
                                                 kBufferWord3)) {}

    template <bool NT>
    __device__ __forceinline__ void load(int e0, uint32_t (&w)[load_words<VEC>()]) const
    {
        constexpr int aux = NT ? 2 : 0;   // cache policy: nontemporal
        const int off = e0 * kElem;
        if constexpr (VEC == 1) {
            if constexpr (BF16)
                w[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rsrc, off, 0, aux) << 16;
            else
                w[0] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, aux);
        } else {
            static_assert((!BF16 && VEC == 4) || (BF16 && VEC == 8), "vector widths: fp32 x4, bf16 x8");
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, aux);
            w[0] = x[0]; w[1] = x[1]; w[2] = x[2]; w[3] = x[3];
        }
    }
};

// Element v of a load as a binary32 bit pattern.
template <bool BF16, int VEC>
__device__ __forceinline__ uint32_t raw_elem(const uint32_t (&w)[load_words<VEC>()], int v)
{
    if constexpr (VEC == 1) return w[0];
    else if constexpr (BF16) return (v & 1) ? (w[v >> 1] & 0xFFFF0000u) : (w[v >> 1] << 16);
    else return w[v];
}

// Largest and smallest element of a full load, as signed integers (binary32 patterns).
// For bf16 pairs the high halves order like their whole words, so one max/min over the
// words gives the high-half extremes; the low halves are shifted up first.
template <bool BF16, int VEC>
__device__ __forceinline__ void load_minmax(const uint32_t (&w)[load_words<VEC>()], int& mx, int& mn)
{
    constexpr int W = load_words<VEC>();
    if constexpr (VEC == 1) {
        mx = mn = (int)w[0];
    } else {
        int hx = (int)w[0], hn = (int)w[0];
#pragma unroll
        for (int i = 1; i < W; ++i) {
            hx = max(hx, (int)w[i]);
            hn = min(hn, (int)w[i]);
        }
        if constexpr (BF16) {
            int lx = (int)(w[0] << 16), ln = lx;
#pragma unroll
            for (int i = 1; i < W; ++i) {
                lx = max(lx, (int)(w[i] << 16));
                ln = min(ln, (int)(w[i] << 16));
            }
            mx = max((int)((uint32_t)hx & 0xFFFF0000u), lx);
            mn = min((int)((uint32_t)hn & 0xFFFF0000u), ln);
        } else {
            mx = hx;
            mn = hn;
        }
    }
}

// Chunks in flight per wavefront on the streaming path (a third one measured no faster).
constexpr int kStreamDepth = 2;

// Loads per lane in one chunk: 64 lanes x U loads of VEC elements.
template <int VEC>
constexpr int chunk_loads() { return VEC == 1 ? 16 : 4; }

// Per-wavefront LDS of the long-row path.
template <typename T>
struct WaveShared {
    static constexpr int GCAP = 64;     // candidate groups
    static constexpr int MCAP = 64;     // candidate keys (with the forced blocks: one sort)
    uint32_t glist[GCAP];
    T mcand[MCAP];
};

// Exact top-16 of a long row by one wavefront (see the file comment). Element e of the
// row is loaded in chunk c, load u, lane l, slot v with e = ((c U + u) 64 + l) VEC + v.
// Groups: with 16-byte loads (QUAD), the four lanes of quad q read one contiguous
// 64-byte segment per load, and group (c, u, q) is that segment; lane 4q + p keeps the
// key of group (c, p, q) (U = 4). With single-element loads lane l's U elements of chunk
// c form group (c, l). Either way the 64 lanes keep keys of disjoint element sets.
// Returns lane r = rank-r key for r < 16 (0 past the valid count); on the fused call
// `phys` of lane r is the physical block of that key when *have_phys is set.
template <bool BF16, int VEC, int NC, bool FUSED, bool WIDE = false>
__device__ __forceinline__ uint64_t wave_stream_row(const SelArgs& a, int64_t row_off, int nvp,
                                                    const int32_t* bt_row,
                                                    WaveShared<typename KeyOf<BF16, WIDE>::T>& sh,
                                                    int& phys, bool& have_phys, int e_base = 0,
                                                    int len = -1, bool with_forced = true)
{
    using KT = KeyOf<BF16, WIDE>;
    using T = typename KT::T;
    using SH = WaveShared<T>;
    constexpr int U = chunk_loads<VEC>();
    constexpr bool QUAD = VEC > 1;
    static_assert(!QUAD || U == 4, "a quad keeps one group per load");
    constexpr int CHUNK = 64 * U * VEC;
    constexpr int W = load_words<VEC>();
    int lane = lane_id();
    if constexpr (WIDE) {
        // called once per segment in a loop: an opaque lane index keeps the per-lane
        // element indices from being hoisted out of that loop into live registers
        asm volatile("" : "+v"(lane));
    }
    const int ni = a.num_init, nl = a.num_local, topk = a.topk;
    const int lo_local = nvp - nl;
    // The streamed range is tiles [e_base, e_base + len) of the row (the whole causal
    // row unless a long row is taken one segment at a time); element e of the range is
    // block e_base + e. Without with_forced the result holds scored blocks only.
    if (len < 0) len = nvp;

    // stream the range, two chunks in flight; loads past it return zeros (masked below)
    // without touching memory
    const RowReader<BF16, VEC> rd(static_cast<const char*>(a.scores) + (row_off + e_base) * (BF16 ? 2 : 4),
                                  ((len + VEC - 1) / VEC) * VEC * (BF16 ? 2 : 4));
    constexpr int DEPTH = kStreamDepth;
    uint32_t buf[DEPTH][U][W];
    auto load_chunk = [&](int c, uint32_t (&b)[U][W]) {
#pragma unroll
        for (int u = 0; u < U; ++u) rd.template load<true>(((c * U + u) * 64 + lane) * VEC, b[u]);
    };
    // rank image of the largest element (signed extremes mx, mn), at least 1
    auto image_of = [](int mx, int mn) {
        return max(order_image(mx >= 0 ? (uint32_t)mx : (uint32_t)mn), 1u);
    };
    // Loads are issued for all NC chunks whatever the row length, so that the load
    // sequence has no branch and each wait covers exactly the chunk about to be used.
#pragma unroll
    for (int c = 0; c < DEPTH && c < NC; ++c) load_chunk(c, buf[c]);
    uint32_t gkey[NC];
    uint32_t lkey = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        gkey[c] = 0;
        if (c * CHUNK < len) {
            const bool full = (c + 1) * CHUNK <= len;
            uint32_t g = 0;
            int gx = INT32_MIN, gn = INT32_MAX;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = ((c * U + u) * 64 + lane) * VEC;
                int mx, mn;
                uint32_t img;
                if (full) {
                    load_minmax<BF16, VEC>(buf[c % DEPTH][u], mx, mn);
                    img = image_of(mx, mn);
                } else {
                    mx = INT32_MIN;
                    mn = INT32_MAX;
#pragma unroll
                    for (int v = 0; v < VEC; ++v) {
                        const int x = (int)raw_elem<BF16, VEC>(buf[c % DEPTH][u], v);
                        const bool ok = e0 + v < len;
                        mx = max(mx, ok ? x : INT32_MIN);
                        mn = min(mn, ok ? x : INT32_MAX);
                    }
                    img = e0 < len ? image_of(mx, mn) : 0u;
                }
                if constexpr (QUAD) {
                    lkey = max(lkey, img);
                    img = max(img, xor_lane<1>(img));
                    img = max(img, xor_lane<2>(img));
                    if ((lane & 3) == u) g = img;
                } else {
                    gx = max(gx, mx);
                    gn = min(gn, mn);
                    if (e0 < len) g = 1;
                }
            }
            if constexpr (!QUAD) {
                g = g ? image_of(gx, gn) : 0u;
                lkey = max(lkey, g);
            }
            gkey[c] = g;
        }
        if (c + DEPTH < NC) load_chunk(c + DEPTH, buf[c % DEPTH]);
    }

    // threshold: the topk-th largest lane key. A lane's key is the maximum of the
    // elements it loaded itself, so the keys are maxima of disjoint sets and at least
    // topk elements reach the threshold (short rows still give enough lanes a key)
    uint32_t tau = readlane(sort64_desc(lkey), topk - 1);
    if (tau == 0) tau = 1;

    // the groups whose maximum reaches tau, as the element index of their first load
    // (divided by VEC)
    int ng = 0;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const bool hit = gkey[c] >= tau;
        const uint64_t m = ballot(hit);
        if (m != 0) {
            const int pos = ng + (int)__builtin_amdgcn_mbcnt_hi(
                                     (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            const uint32_t code = QUAD ? (uint32_t)((c * U + (lane & 3)) * 64 + (lane & ~3))
                                       : (uint32_t)(c * 64 + lane);
            if (hit && pos < SH::GCAP) sh.glist[pos] = code;
            ng += __builtin_popcountll(m);
        }
    }
    // LDS accesses of one wavefront complete in order; keep the compiler from moving
    // the reads of other lanes' entries above the writes
    __builtin_amdgcn_wave_barrier();

    const int nf = ni + nl;      // disjoint: nvp > 128 >= ni + nl
    const int nfx = with_forced ? nf : 0;
    auto forced_key = [&](int i) { return KT::forced(i < ni ? i : lo_local + (i - ni)); };
    auto elem_key = [&](int e, uint32_t bits) -> T {
        const int g = e_base + e;
        const bool forced = g < ni || g >= lo_local;
        const bool cand = e < len && !forced && max(order_image(bits), 1u) >= tau;
        return cand ? KT::scored(bits, g) : T(0);
    };

    // read those groups again (four lanes per 64-byte group, or one lane per load of a
    // lane group) and keep the elements that reach tau
    constexpr int PER = QUAD ? 4 : U;   // loads per group
    int nc = 0;
    if (ng <= SH::GCAP) {
        for (int r0 = 0; r0 < ng * PER; r0 += kWave) {
            const int idx = r0 + lane;
            uint32_t bits[W];
            int e0 = len;
            if (idx < ng * PER) {
                const uint32_t code = sh.glist[idx / PER];
                const int part = idx % PER;
                e0 = QUAD ? ((int)code + part) * VEC
                          : (((int)(code >> 6) * U + part) * 64 + (int)(code & 63)) * VEC;
            }
            rd.template load<false>(e0, bits);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const T k = e0 + v < len ? elem_key(e0 + v, raw_elem<BF16, VEC>(bits, v)) : T(0);
                const uint64_t m = ballot(k != 0);
                if (m != 0) {
                    const int pos = nc + (int)__builtin_amdgcn_mbcnt_hi(
                                             (uint32_t)(m >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    if (k != 0 && pos < SH::MCAP) sh.mcand[pos] = k;
                    nc += __builtin_popcountll(m);
                }
            }
        }
    }
    __builtin_amdgcn_wave_barrier();

    if (ng <= SH::GCAP && nfx + nc <= kWave) {
        // one key per lane, tagged with its lane; each lane fetches its key's block
        const T key = lane < nfx ? forced_key(lane) : (lane < nfx + nc ? sh.mcand[lane - nfx] : T(0));
        int ph = 0;
        if constexpr (FUSED) {
            const int kid = KT::block(key);
            if (bt_row != nullptr && kid >= 0 && kid < a.max_blocks) ph = bt_row[kid];
        }
        // the keys sit in the first nfx + nc lanes: a 32-lane sort is enough when they fit
        const uint64_t tagged = ((uint64_t)key << 6) | (uint64_t)lane;
        const uint64_t sorted = nfx + nc <= 32 ? flip_sort<true, 2, 32>(tagged, lane)
                                               : sort64_desc(tagged);
        if constexpr (FUSED) phys = __builtin_amdgcn_ds_bpermute((int)(sorted & 63u) << 2, ph);
        have_phys = true;
        return lane < 16 ? (sorted >> 6) : 0;
    }
    // many equal scores at the threshold: exact top-k over the whole range
    have_phys = false;
    return (uint64_t)topk16_of_list<T>(nfx + len, [&](int i) -> T {
        if (i < nfx) return forced_key(i);
        const int e = i - nfx;
        return elem_key(e, load_bits<BF16>(a.scores, row_off + e_base + e));
    });
}

// ---------------------------------------------------------------------------
// Rows longer than the fast path's 8192 tiles (wide keys)
// ---------------------------------------------------------------------------
// Scored top-16 (rank order in lanes 0..15) of the 8192-tile segments first_seg,
// first_seg + stride, first_seg + 2 stride, ... of a row, each streamed with the
// threshold filter and merged.
template <bool BF16, int VEC, int NC>
__device__ __forceinline__ typename KeyOf<BF16, true>::T segments_top16(
    const SelArgs& a, int64_t row_off, int nvp, const int32_t* bt_row,
    WaveShared<typename KeyOf<BF16, true>::T>& sh, int first_seg, int stride = 1)
{
    using T = typename KeyOf<BF16, true>::T;
    T carry = 0;   // merging into an empty list returns the other list
#pragma unroll 1
    for (int s0 = first_seg * kSegmentTiles; s0 < nvp; s0 += stride * kSegmentTiles) {
        const int len = nvp - s0 < kSegmentTiles ? nvp - s0 : kSegmentTiles;
        int ph;
        bool hp;
        const T seg = (T)wave_stream_row<BF16, VEC, NC, false, true>(a, row_off, nvp, bt_row, sh,
                                                                     ph, hp, s0, len, false);
        carry = merge_top16(carry, seg);
    }
    return carry;
}

// The forced blocks (they outrank every score, in ascending id) followed by the scored
// top-16 `carry`, as the row's rank order in lanes 0..15. Requires nvp > 128.
template <typename KT>
__device__ __forceinline__ uint64_t forced_then(typename KT::T carry, int nvp, int ni, int nl)
{
    using T = typename KT::T;
    const int lane = lane_id();
    const int nf = ni + nl;
    const int src = lane >= nf ? lane - nf : 0;
    const T moved = (T)(((uint64_t)(uint32_t)shfl((int)(uint32_t)((uint64_t)carry >> 32), src) << 32) |
                        (uint32_t)shfl((int)(uint32_t)carry, src));
    const int fid = lane < ni ? lane : nvp - nl + (lane - ni);
    return lane < nf ? (uint64_t)KT::forced(fid) : (lane < 16 ? (uint64_t)moved : 0);
}

// ---------------------------------------------------------------------------
// Selector kernel: one wavefront per (row, head)
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

// The same from a kernel's leading scalar arguments, which the code object has preloaded
// into scalar registers at wave launch (kernel-argument preloading), so that no
// argument load stands between a wavefront's start and the loads of its row and row
// metadata: rows0 is the decode form's seq_lens (q >= 1), the explicit form's row_req
// (q == 0) or the standalone selector's num_valid_pages; (q_mul, q_shift) is
// make_divisor(q) and M is max_k_tiles.
template <bool FUSED>
__device__ __forceinline__ int row_count_lead(const SelArgs& a, const int32_t* rows0, int q,
                                              uint32_t q_mul, uint32_t q_shift, int M, int64_t t,
                                              int64_t& c, int& req)
{
    if constexpr (FUSED) {
        const RowInfo ri = q > 0 ? row_info_of(rows0, nullptr, nullptr, q, q_mul, q_shift, 0, t)
                                 : row_info_of(nullptr, rows0, a.rows.row_pos, 1, 0, 0, a.rows.B, t);
        c = ri.c;
        req = ri.req;
        return (int)clamp_count((c + kBlockTokens - 1) / kBlockTokens, M);
    } else {
        c = 0;
        req = -1;
        return (int)clamp_count(rows0[t], M);
    }
}

// NC = 0: short rows only (rows longer than 128 blocks loop over 128-tile chunks);
// the first chunk's tiles are then fetched together with the row metadata.
// NC > 0: rows longer than 128 blocks take the streaming path (NC chunks cover
// max_k_tiles). The launch visits the leading decode rows first, in buffer order
// (their lengths do not follow their position), then the other rows from the last
// (row, head) to the first, so that the longest rows of each prefill request start
// early and the short ones fill the end of the launch.
//
// What a wavefront needs before its first loads comes ahead of the argument block as
// plain scalars (see row_count_lead); (h_mul, h_shift) is make_divisor(H).
template <bool BF16, bool FUSED, int VEC, int NC>
__global__ __launch_bounds__(256) void select_wave_kernel(const void* scores, const int32_t* rows0,
                                                          int64_t total, int M, int rhpb,
                                                          uint32_t h_mul, uint32_t h_shift,
                                                          uint32_t q_mul, uint32_t q_shift, int q,
                                                          SelArgs a)
{
    using KT = KeyOf<BF16>;
    using T = typename KT::T;
    const int wave = uniform((int)(threadIdx.x >> 6));
    const int lane = lane_id();
    int64_t rh = (int64_t)blockIdx.x * rhpb + wave;
    if (rh >= total) return;
    if constexpr (NC > 0) {
        if (rh >= a.front) rh = total - 1 - (rh - a.front);
    }
    const int64_t t = divide_by((uint32_t)rh, h_mul, h_shift);
    const int64_t row_off = rh * (int64_t)M;

    const void* row = static_cast<const char*>(scores) + row_off * (BF16 ? 2 : 4);
    uint32_t r0 = 0, r1 = 0;
    if constexpr (NC == 0) {
        // the two round trips (row metadata, first tiles) overlap; tiles past the
        // causal count are masked below
        const RowReader<BF16, 1> rd(row, M * (BF16 ? 2 : 4));
        uint32_t w0[1], w1[1];
        rd.template load<false>(lane, w0);
        rd.template load<false>(lane + kWave, w1);
        r0 = w0[0];
        r1 = w1[0];
    }
    int64_t c;
    int req;
    const int nvp = uniform(row_count_lead<FUSED>(a, rows0, q, q_mul, q_shift, M, t, c, req));
    c = uniform(c);
    req = uniform(req);
    const int32_t* bt_row = FUSED && req >= 0 ? a.block_table + (int64_t)req * a.max_blocks : nullptr;

    uint64_t top;
    int phys = 0;
    bool have_phys = false;
    if (NC == 0 || nvp <= 2 * kWave) {
        if constexpr (NC > 0) {
            const RowReader<BF16, 1> rd(row, nvp * (BF16 ? 2 : 4));
            uint32_t w0[1], w1[1];
            rd.template load<false>(lane, w0);
            rd.template load<false>(lane + kWave, w1);
            r0 = w0[0];
            r1 = w1[0];
        }
        top = (uint64_t)wave_select_row<BF16>(a.scores, row_off, nvp, a.num_init, a.num_local,
                                              r0, r1);
    } else if (BF16 && nvp <= kChunkRowMax) {
        // up to kChunkRowMax tiles: all 128-tile chunks in one round trip, independent
        // top-16 networks (whose exchanges interleave), pairwise merges; the stream's
        // dependent round trips (threshold, candidate re-read) cost more than they save
        // here. (fp32 rows, or bf16 rows of 513..1024 tiles, measured slower this way.)
        if constexpr (NC > 0) {
            const RowReader<BF16, 1> rd(row, nvp * (BF16 ? 2 : 4));
            if (nvp <= 4 * kWave) {
                uint32_t raw[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    uint32_t w1[1];
                    rd.template load<false>(lane + s * kWave, w1);
                    raw[s] = w1[0];
                }
                top = (uint64_t)wave_select_chunks<BF16, 2>(nvp, a.num_init, a.num_local, raw);
            } else {
                uint32_t raw[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    uint32_t w1[1];
                    rd.template load<false>(lane + s * kWave, w1);
                    raw[s] = w1[0];
                }
                top = (uint64_t)wave_select_chunks<BF16, 4>(nvp, a.num_init, a.num_local, raw);
            }
        }
    } else {
        if constexpr (NC > 0) {
            __shared__ WaveShared<T> sh[4];
            top = wave_stream_row<BF16, VEC, NC, FUSED>(a, row_off, nvp, bt_row, sh[wave], phys,
                                                         have_phys);
        }
    }
    const int id = KT::block((T)top);
    if constexpr (NC > 0) {
        if (lane < a.topk) a.out_idx[rh * a.topk + lane] = id;
    }
    if constexpr (FUSED) {
        // short-row launches are only their latency chain: two store instructions per row
        int32_t* trow = a.out_table + rh * (int64_t)a.topk * kPagesPerBlock;
        if (have_phys)
            emit_table_phys(id, phys, c, a.max_blocks, a.topk, trow, a.out_ctx + rh,
                            a.table_vec != 0, NC > 0);
        else
            emit_table_sorted(id, c, bt_row, a.max_blocks, a.topk, trow, a.out_ctx + rh,
                              a.table_vec != 0, NC > 0);
    }
    // short-row launches write the indices last: a store ahead of the table's
    // block-table gather made the compiler wait for the store's completion before
    // issuing the gather (the 74-block batch 2.71 against 2.82 us; the streaming launch
    // measured slightly faster with the indices first)
    if constexpr (NC == 0) {
        if (lane < a.topk) a.out_idx[rh * a.topk + lane] = id;
    }
}

// ---------------------------------------------------------------------------
// Split selector: one workgroup of S wavefronts per (row, head), for batches with
// few (row, head) pairs and long rows. Wavefront w reads chunk w of the row (64 lanes x
// 4 loads of 16 bytes) over the row's capacity before the row metadata arrives and keeps
// it in registers. Every lane's maximum is the maximum of elements no other lane holds,
// so the topk-th largest of all the workgroup's lane maxima is reached by at least topk
// elements of the row: that is the threshold (each wavefront sorts its lanes' maxima,
// its 16 largest go to LDS, and the folds of a top-16 network over those sorted lists
// pick it; the largest of the wavefronts' own topk-th maxima, used before, let about a
// hundred candidates through on 8192-tile rows and took the slow list path). The loads
// holding an element that reaches it are staged in LDS from the
// registers, their elements compacted, and wavefront 0 sorts the forced blocks and all
// candidates at once. Rows longer than the S chunks, or with mass ties at the
// threshold, are finished exactly by wavefront 0 alone.
// ---------------------------------------------------------------------------
constexpr int kSplitMaxWaves = 8;

template <typename T>
struct SplitShared {
    static constexpr int SCAP = 64;     // staged loads per wavefront
    static constexpr int MCAP = 64;     // candidate keys per wavefront
    uint32_t top[kSplitMaxWaves][16];   // each wavefront's 16 largest lane maxima
    int nc[kSplitMaxWaves];
    uint32_t stage[kSplitMaxWaves][SCAP][4];
    int spos[kSplitMaxWaves][SCAP];
    T mc[kSplitMaxWaves][MCAP];
    WaveShared<T> one;                  // wavefront 0 finishing a row alone
};

template <bool BF16, bool FUSED, int VEC>
__global__ __launch_bounds__(64 * kSplitMaxWaves) void select_split_kernel(
    const void* scores, const int32_t* rows0, int M, uint32_t h_mul, uint32_t h_shift,
    uint32_t q_mul, uint32_t q_shift, int q, SelArgs a)
{
    using KT = KeyOf<BF16>;
    using T = typename KT::T;
    using SS = SplitShared<T>;
    static_assert(VEC > 1, "the split path reads 16-byte vectors");
    constexpr int U = chunk_loads<VEC>();
    constexpr int W = load_words<VEC>();
    constexpr int CHUNK = 64 * U * VEC;
    constexpr int ELEM = BF16 ? 2 : 4;
    __shared__ SS sh;
    const int S = uniform((int)(blockDim.x >> 6));
    const int wave = uniform((int)(threadIdx.x >> 6));
    const int lane = lane_id();
    const int64_t rh = blockIdx.x;
    const int64_t t = divide_by((uint32_t)rh, h_mul, h_shift);
    const int64_t row_off = rh * (int64_t)M;
    const void* row = static_cast<const char*>(scores) + row_off * ELEM;

    // this wavefront's chunk, requested before the causal count is known
    uint32_t buf[U][W];
    {
        const RowReader<BF16, VEC> cap(row, M * ELEM);
#pragma unroll
        for (int u = 0; u < U; ++u) cap.template load<true>(((wave * U + u) * 64 + lane) * VEC, buf[u]);
    }
    int64_t c;
    int req;
    const int nvp = uniform(row_count_lead<FUSED>(a, rows0, q, q_mul, q_shift, M, t, c, req));
    c = uniform(c);
    req = uniform(req);
    const int32_t* bt_row = FUSED && req >= 0 ? a.block_table + (int64_t)req * a.max_blocks : nullptr;
    const int ni = a.num_init, nl = a.num_local, topk = a.topk;
    const int nf = ni + nl;
    const int lo_local = nvp - nl;
    int32_t* trow = FUSED ? a.out_table + rh * (int64_t)topk * kPagesPerBlock : nullptr;

    uint64_t top;
    int phys = 0;
    bool have_phys = false;
    // the rows the launch was shaped for take the last branch; the other two are laid
    // out away from its code
    if (__builtin_expect(nvp <= 2 * kWave, 0)) {
        // short row: wavefront 0 alone (the branch is uniform over the workgroup)
        if (wave != 0) return;
        const RowReader<BF16, 1> rd(row, nvp * ELEM);
        uint32_t w0[1], w1[1];
        rd.template load<false>(lane, w0);
        rd.template load<false>(lane + kWave, w1);
        top = (uint64_t)wave_select_row<BF16>(a.scores, row_off, nvp, ni, nl, w0[0], w1[0]);
    } else if (__builtin_expect(nvp > S * CHUNK, 0)) {
        // longer than the chunks read: wavefront 0 streams the whole row
        if (wave != 0) return;
        top = wave_stream_row<BF16, VEC, 8, FUSED>(a, row_off, nvp, bt_row, sh.one, phys,
                                                    have_phys);
    } else {
        auto image_of = [](int mx, int mn) {
            return max(order_image(mx >= 0 ? (uint32_t)mx : (uint32_t)mn), 1u);
        };
        // the maximum of each load (0 if it holds no causal tile), and the lane's key
        uint32_t own[U];
        uint32_t lkey = 0;
        const bool full = (wave + 1) * CHUNK <= nvp;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e0 = ((wave * U + u) * 64 + lane) * VEC;
            int mx, mn;
            if (full) {
                load_minmax<BF16, VEC>(buf[u], mx, mn);
            } else {
                mx = INT32_MIN;
                mn = INT32_MAX;
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const int x = (int)raw_elem<BF16, VEC>(buf[u], v);
                    const bool in = e0 + v < nvp;
                    mx = max(mx, in ? x : INT32_MIN);
                    mn = min(mn, in ? x : INT32_MAX);
                }
            }
            own[u] = e0 < nvp ? image_of(mx, mn) : 0u;
            lkey = max(lkey, own[u]);
        }
        // the topk-th largest lane maximum of the workgroup (every wavefront finds it)
        const uint32_t sorted = wave * CHUNK < nvp ? sort64_desc(lkey) : 0u;
        if (lane < 16) sh.top[wave][lane] = sorted;
        __syncthreads();
        const uint32_t t0 = lane < 16 * S ? sh.top[lane >> 4][lane & 15] : 0u;
        const uint32_t t1 = kWave + lane < 16 * S ? sh.top[(kWave + lane) >> 4][lane & 15] : 0u;
        uint32_t tau = readlane(top16_of_sorted_rows(t0, t1), topk - 1);
        if (tau == 0) tau = 1;

        auto elem_key = [&](int e, uint32_t bits) -> T {
            const bool forced = e < ni || e >= lo_local;
            const bool cand = e < nvp && !forced && max(order_image(bits), 1u) >= tau;
            return cand ? KT::scored(bits, e) : T(0);
        };
        // stage the loads that hold an element reaching tau
        int nh = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool hit = own[u] >= tau;
            const uint64_t m = ballot(hit);
            if (m != 0) {
                const int pos = nh + (int)__builtin_amdgcn_mbcnt_hi(
                                         (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                if (hit && pos < SS::SCAP) {
#pragma unroll
                    for (int w = 0; w < W; ++w) sh.stage[wave][pos][w] = buf[u][w];
                    sh.spos[wave][pos] = ((wave * U + u) * 64 + lane) * VEC;
                }
                nh += __builtin_popcountll(m);
            }
        }
        __builtin_amdgcn_wave_barrier();
        // compact their elements that reach tau (forced blocks are added by wavefront 0)
        int nc = 0;
        if (nh <= SS::SCAP) {
            uint32_t bits[W];
#pragma unroll
            for (int w = 0; w < W; ++w) bits[w] = lane < nh ? sh.stage[wave][lane][w] : 0u;
            const int e0 = lane < nh ? sh.spos[wave][lane] : nvp;
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const T k = e0 + v < nvp ? elem_key(e0 + v, raw_elem<BF16, VEC>(bits, v)) : T(0);
                const uint64_t m = ballot(k != 0);
                if (m != 0) {
                    const int pos = nc + (int)__builtin_amdgcn_mbcnt_hi(
                                             (uint32_t)(m >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    if (k != 0 && pos < SS::MCAP) sh.mc[wave][pos] = k;
                    nc += __builtin_popcountll(m);
                }
            }
        } else {
            nc = SS::MCAP + 1;   // too many staged loads: mark the slice incomplete
        }
        if (lane == 0) sh.nc[wave] = nc;
        __syncthreads();
        if (wave != 0) return;

        // wavefront 0: forced blocks + every slice's candidates; off[w] is where slice w
        // starts in the concatenated list (uniform)
        int off[kSplitMaxWaves];
        int total = nf;
        bool complete = true;
#pragma unroll
        for (int w = 0; w < kSplitMaxWaves; ++w) {
            const int n = w < S ? uniform(sh.nc[w]) : 0;
            off[w] = total;
            complete = complete && n <= SS::MCAP;
            total += n;
        }
        auto forced_key = [&](int i) { return KT::forced(i < ni ? i : lo_local + (i - ni)); };
        // i-th key of the concatenated list (forced, then slice 0, slice 1, ...), i < total:
        // the last slice starting at or before i holds it (an empty slice is followed by
        // one starting at the same place, or ends the list)
        auto list_key = [&](int i) -> T {
            if (i < nf) return forced_key(i);
            int w = 0, base = off[0];
#pragma unroll
            for (int v = 1; v < kSplitMaxWaves; ++v) {
                const bool in = v < S && i >= off[v];
                w = in ? v : w;
                base = in ? off[v] : base;
            }
            return sh.mc[w][i - base];
        };
        if (__builtin_expect(complete && total <= kWave, 1)) {
            const T key = lane < total ? list_key(lane) : T(0);
            int ph = 0;
            if constexpr (FUSED) {
                const int kid = KT::block(key);
                if (bt_row != nullptr && kid >= 0 && kid < a.max_blocks) ph = bt_row[kid];
            }
            const uint64_t tagged = ((uint64_t)key << 6) | (uint64_t)lane;
            const uint64_t sorted = total <= 32 ? flip_sort<true, 2, 32>(tagged, lane)
                                                : sort64_desc(tagged);
            if constexpr (FUSED) phys = __builtin_amdgcn_ds_bpermute((int)(sorted & 63u) << 2, ph);
            have_phys = true;
            top = lane < 16 ? (sorted >> 6) : 0;
        } else if (complete) {
            top = (uint64_t)topk16_of_list<T>(total, list_key);
        } else {
            // many equal scores at the threshold: exact top-k over the whole row
            top = (uint64_t)topk16_of_list<T>(nf + nvp, [&](int i) -> T {
                if (i < nf) return forced_key(i);
                const int e = i - nf;
                return elem_key(e, load_bits<BF16>(a.scores, row_off + e));
            });
        }
    }
    const int id = KT::block((T)top);
    if (lane < topk) a.out_idx[rh * topk + lane] = id;
    if constexpr (FUSED) {
        if (have_phys)
            emit_table_phys(id, phys, c, a.max_blocks, topk, trow, a.out_ctx + rh, a.table_vec != 0);
        else
            emit_table_sorted(id, c, bt_row, a.max_blocks, topk, trow, a.out_ctx + rh,
                              a.table_vec != 0);
    }
}

// ---------------------------------------------------------------------------
// Segment selector for rows beyond the fast path: one workgroup of S wavefronts per
// (row, head); wavefront w streams 8192-tile segment w (and, for rows longer than S
// segments, w + S, w + 2S, ... as well). Each keeps the scored top-16 of its segments,
// wavefront 0 merges the S lists and places the forced blocks first.
// ---------------------------------------------------------------------------
template <bool BF16, bool FUSED, int VEC, int NC>
__global__ __launch_bounds__(64 * kSegmentMaxWaves) void select_segment_kernel(
    const int32_t* rows0, int M, uint32_t h_mul, uint32_t h_shift, uint32_t q_mul,
    uint32_t q_shift, int q, SelArgs a)
{
    using KT = KeyOf<BF16, true>;
    using T = typename KT::T;
    __shared__ WaveShared<T> sh[kSegmentMaxWaves];
    __shared__ T tops[kSegmentMaxWaves][16];
    const int S = uniform((int)(blockDim.x >> 6));
    const int wave = uniform((int)(threadIdx.x >> 6));
    const int lane = lane_id();
    const int64_t rh = blockIdx.x;
    const int64_t t = divide_by((uint32_t)rh, h_mul, h_shift);
    const int64_t row_off = rh * (int64_t)M;
    int64_t c;
    int req;
    const int nvp = uniform(row_count_lead<FUSED>(a, rows0, q, q_mul, q_shift, M, t, c, req));
    c = uniform(c);
    req = uniform(req);
    const int32_t* bt_row = FUSED && req >= 0 ? a.block_table + (int64_t)req * a.max_blocks : nullptr;

    uint64_t top;
    if (nvp <= 2 * kWave) {
        // short row: wavefront 0 alone (the branch is uniform over the workgroup)
        if (wave != 0) return;
        const RowReader<BF16, 1> rd(static_cast<const char*>(a.scores) + row_off * (BF16 ? 2 : 4),
                                    nvp * (BF16 ? 2 : 4));
        uint32_t w0[1], w1[1];
        rd.template load<false>(lane, w0);
        rd.template load<false>(lane + kWave, w1);
        top = (uint64_t)wave_select_row<BF16, true>(a.scores, row_off, nvp, a.num_init,
                                                    a.num_local, w0[0], w1[0]);
    } else {
        T seg = 0;
        const int s0 = wave * kSegmentTiles;
        if (s0 < nvp) {
            const int len = nvp - s0 < kSegmentTiles ? nvp - s0 : kSegmentTiles;
            int ph;
            bool hp;
            seg = (T)wave_stream_row<BF16, VEC, NC, false, true>(a, row_off, nvp, bt_row, sh[wave],
                                                                 ph, hp, s0, len, false);
        }
        // rows longer than S segments: wavefront w also takes segments w + S, w + 2S, ...
        if (S * kSegmentTiles < nvp)
            seg = merge_top16(seg, segments_top16<BF16, VEC, NC>(a, row_off, nvp, bt_row, sh[wave],
                                                                 wave + S, S));
        if (lane < 16) tops[wave][lane] = seg;
        __syncthreads();
        if (wave != 0) return;
        T carry = 0;
        for (int w = 0; w < S; ++w) carry = merge_top16(carry, lane < 16 ? tops[w][lane] : T(0));
        top = forced_then<KT>(carry, nvp, a.num_init, a.num_local);
    }
    const int id = KT::block((T)top);
    if (lane < a.topk) a.out_idx[rh * a.topk + lane] = id;
    if constexpr (FUSED)
        emit_table_sorted(id, c, bt_row, a.max_blocks, a.topk,
                          a.out_table + rh * (int64_t)a.topk * kPagesPerBlock, a.out_ctx + rh,
                          a.table_vec != 0);
}

// ---------------------------------------------------------------------------
// topk above 16, up to 64 (path 5): one wavefront per (row, head) keeps the row's
// running top-64 in rank order, one key per lane. The row is read in columns of 64
// elements (each lane loads a vector of VEC consecutive tiles; column v holds element v
// of every lane's vector). A column that holds a key above the running topk-th key is
// sorted and merged in: the element-wise maximum of the running list and the sorted
// column mirrored across lane 63 holds the top 64 of their union as a bitonic sequence,
// which xor stages 32..1 sort. Keys are 64-bit with 24-bit block ids, forced blocks
// first, so the result is the same total order as every other path.
// ---------------------------------------------------------------------------
constexpr int kWideTopkMax = 64;

// Page-16 table row of up to 64 selected blocks (lane r < topk holds the rank-r id, any
// value: -1, ids at or past min(cdiv(c, 128), max_blocks) and repeats are dropped). The
// kept ids are sorted ascending across the 64 lanes with their source lane, repeats
// removed, and each kept block pushed to the lane of its rank; lane r < topk writes
// entries 8r .. 8r + 7. A row without a request (bt_row null) keeps nothing.
__device__ __forceinline__ void emit_table_wide(int id, int64_t c, const int32_t* bt_row,
                                                int max_blocks, int topk, int32_t* table_row,
                                                int32_t* ctx_out, bool vec_store)
{
    const int lane = lane_id();
    const int64_t nvp_c = (c + kBlockTokens - 1) / kBlockTokens;
    const int64_t lim = nvp_c < max_blocks ? nvp_c : (int64_t)max_blocks;
    const bool ok = lane < topk && bt_row != nullptr && id >= 0 && id < lim;
    const int phys = ok ? bt_row[id] : 0;   // in flight during the sort
    const uint32_t sk = flip_sort<false, 2, 64>(ok ? ((uint32_t)id << 6) | (uint32_t)lane
                                                   : 0xFFFFFFFFu, lane);
    const uint32_t prev = (uint32_t)shfl((int)sk, lane > 0 ? lane - 1 : 0);
    const bool kept = sk != 0xFFFFFFFFu && !(lane > 0 && (prev >> 6) == (sk >> 6));
    const uint64_t km = ballot(kept);
    const int nkept = __builtin_popcountll(km);
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(km >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u));
    const int ph = __builtin_amdgcn_ds_bpermute((int)(sk & 63u) << 2, phys);
    int tb = 0;
    if (kept) {
        const int64_t rest = c - (int64_t)kBlockTokens * (sk >> 6);
        tb = rest < kBlockTokens ? (int)rest : kBlockTokens;
    }
    // kept lane of rank r goes to lane r; the others to lanes nkept .. 63, one each
    const int dst = kept ? below : 63 - (lane - below);
    const int ph_r = __builtin_amdgcn_ds_permute(dst << 2, ph);
    const int tb_r = __builtin_amdgcn_ds_permute(dst << 2, tb);
    uint32_t sum = (uint32_t)tb;
    sum += xor_lane<8>(sum);
    sum += xor_lane<4>(sum);
    sum += xor_lane<2>(sum);
    sum += xor_lane<1>(sum);
    const uint32_t total = readlane(sum, 0) + readlane(sum, 16) + readlane(sum, 32) +
                           readlane(sum, 48);
    if (lane < topk) {
        const int np = lane < nkept ? (tb_r + 15) >> 4 : 0;
        const uint32_t base = (uint32_t)ph_r * (uint32_t)kPagesPerBlock;
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
    if (lane == 0) *ctx_out = (int32_t)total;
}

template <bool BF16, bool FUSED, int VEC>
__global__ __launch_bounds__(256) void select_wide_topk_kernel(SelArgs a)
{
    using KT = KeyWide;
    using T = uint64_t;
    constexpr int W = load_words<VEC>();
    constexpr int ELEM = BF16 ? 2 : 4;
    const int wave = uniform((int)(threadIdx.x >> 6));
    const int lane = lane_id();
    const int64_t rh = (int64_t)blockIdx.x * 4 + wave;
    if (rh >= a.T * a.H) return;
    const int64_t t = divide_by((uint32_t)rh, a.h_mul, a.h_shift);
    const int64_t row_off = rh * (int64_t)a.M;
    int64_t c;
    int req;
    const int nvp = uniform(row_count<FUSED>(a, t, c, req));
    c = uniform(c);
    req = uniform(req);
    const int32_t* bt_row = FUSED && req >= 0 ? a.block_table + (int64_t)req * a.max_blocks : nullptr;
    const int ni = a.num_init, nl = a.num_local, topk = a.topk;
    const int lo_local = nvp - nl;
    // loads past the causal tiles return zeros without a memory access
    const RowReader<BF16, VEC> rd(static_cast<const char*>(a.scores) + row_off * ELEM,
                                  ((nvp + VEC - 1) / VEC) * VEC * ELEM);
    T run = 0;
    T kth = 0;   // the running topk-th key (0 while fewer are held)
#pragma unroll 1
    for (int base = 0; base < nvp; base += kWave * VEC) {
        uint32_t w[W];
        rd.template load<false>(base + lane * VEC, w);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const int e = base + lane * VEC + v;
            const bool forced = e < ni || e >= lo_local;
            const T k = e < nvp ? (forced ? KT::forced(e) : KT::scored(raw_elem<BF16, VEC>(w, v), e))
                                : T(0);
            if (ballot(k > kth) == 0) continue;   // nothing here reaches the top-k
            const T col = sort64_desc(k);
            const T r = xor_lane<63>(col);
            run = desc_xor_stages<32>(r > run ? r : run, lane);
            kth = readlane(run, topk - 1);
        }
    }
    const int id = KT::block(run);
    if (lane < topk) a.out_idx[rh * topk + lane] = id;
    if constexpr (FUSED)
        emit_table_wide(id, c, bt_row, a.max_blocks, topk,
                        a.out_table + rh * (int64_t)topk * kPagesPerBlock, a.out_ctx + rh,
                        a.table_vec != 0);
}

// Standalone table for topk above 16: one wavefront per (row, head), four per workgroup.
__global__ __launch_bounds__(256) void table_wide_kernel(TabArgs a)
{
    const int wave = (int)(threadIdx.x >> 6);
    const int lane = lane_id();
    const int64_t rh = (int64_t)blockIdx.x * 4 + wave;
    if (rh >= a.T * a.H) return;
    const RowInfo ri = row_info(a.rows, divide_by((uint32_t)rh, a.h_mul, a.h_shift));
    const int32_t* bt_row = ri.req >= 0 ? a.block_table + (int64_t)ri.req * a.max_blocks : nullptr;
    const int id = lane < a.topk ? a.idx[rh * a.topk + lane] : -1;
    emit_table_wide(id, ri.c, bt_row, a.max_blocks, a.topk,
                    a.out_table + rh * (int64_t)a.topk * kPagesPerBlock, a.out_ctx + rh,
                    a.table_vec != 0);
}

// ---------------------------------------------------------------------------
// Cross-workgroup split (path 4), for batches of few (row, head) pairs with long rows:
// one workgroup of one wavefront per slice of 64 lanes x 4 loads of 16 bytes (1024
// fp32 or 2048 bf16 tiles), so that one row is streamed by as many compute units as it
// has slices. Each slice keeps its loads in registers and takes its scored top-16 (the
// forced blocks are added at the end): every lane's maximum covers elements no other
// lane holds, so the k-th largest lane maximum is reached by at least k elements and
// bounds the slice's top-k from below; the loads holding an element that reaches it are
// staged in LDS straight from the registers, their elements compacted and sorted. The
// slice's 16 keys go to the caller's workspace, and an arrival counter per (row, head)
// picks the last slice to finish: it merges every slice's list, streams any tiles past
// the slices (rows longer than the launch hint), puts the forced blocks first, writes
// the outputs and sets the counter and the lists it read back to zero, so the workspace
// is all zeros again for the next call, of any batch shape (and for every replay of a
// captured graph) without a memset.
//
// The workspace is written and read only through the coherent accessors of
// kvbt_device.h (ws_store, ws_load and the two orderings).
// ---------------------------------------------------------------------------
constexpr int kXSplitMaxSlices = 64;

// Per-wavefront LDS of a slice.
struct XSliceShared {
    static constexpr int SCAP = 64;     // staged loads
    static constexpr int MCAP = 64;     // candidate keys
    uint32_t stage[SCAP][4];
    int spos[SCAP];
    uint64_t mc[MCAP];
};

constexpr int kXSplitMaxWaves = 8;      // wavefronts per slice workgroup

// Scored top-16 (rank order in lanes 0..15, 0 elsewhere) of the 64 x U x VEC tiles from
// `base` that this wavefront holds in `buf` (loaded with lane l holding tiles base +
// (u 64 + l) VEC .. + VEC of load u), scored ids being [ni, lo_local). Every lane's
// maximum covers elements no other lane holds, so the ks-th largest lane maximum bounds
// the chunk's top-ks from below; the loads holding an element that reaches it are staged
// in LDS from the registers, their elements compacted and sorted. Mass ties at the
// threshold read the chunk again for an exact top-16.
template <bool BF16, int VEC>
__device__ __forceinline__ uint64_t chunk_scored_top16(const SelArgs& a, int64_t row_off, int nvp,
                                                       int base, int ni, int lo_local, int ks,
                                                       const uint32_t (&buf)[chunk_loads<VEC>()][load_words<VEC>()],
                                                       XSliceShared& xs)
{
    using KT = KeyWide;
    using T = uint64_t;
    constexpr int U = chunk_loads<VEC>();
    constexpr int W = load_words<VEC>();
    constexpr int CHUNK = 64 * U * VEC;
    const int lane = lane_id();
    auto scored_at = [&](int e) { return e >= ni && e < lo_local; };
    auto image_of = [](int mx, int mn) {
        return max(order_image(mx >= 0 ? (uint32_t)mx : (uint32_t)mn), 1u);
    };
    uint32_t own[U];
    uint32_t lkey = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e0 = base + (u * 64 + lane) * VEC;
        int mx = INT32_MIN, mn = INT32_MAX;
        bool any = false;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const int x = (int)raw_elem<BF16, VEC>(buf[u], v);
            const bool ok = scored_at(e0 + v);
            mx = max(mx, ok ? x : INT32_MIN);
            mn = min(mn, ok ? x : INT32_MAX);
            any |= ok;
        }
        own[u] = any ? image_of(mx, mn) : 0u;
        lkey = max(lkey, own[u]);
    }
    uint32_t tau = readlane(sort64_desc(lkey), ks - 1);
    if (tau == 0) tau = 1;
    // stage the loads that hold an element reaching tau
    int nh = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool hit = own[u] >= tau;
        const uint64_t m = ballot(hit);
        if (m != 0) {
            const int pos = nh + (int)__builtin_amdgcn_mbcnt_hi(
                                     (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (hit && pos < XSliceShared::SCAP) {
#pragma unroll
                for (int w = 0; w < W; ++w) xs.stage[pos][w] = buf[u][w];
                xs.spos[pos] = base + (u * 64 + lane) * VEC;
            }
            nh += __builtin_popcountll(m);
        }
    }
    __builtin_amdgcn_wave_barrier();
    // compact their elements that reach tau
    int nc = 0;
    if (nh <= XSliceShared::SCAP) {
        uint32_t bits[W];
#pragma unroll
        for (int w = 0; w < W; ++w) bits[w] = lane < nh ? xs.stage[lane][w] : 0u;
        const int e0 = lane < nh ? xs.spos[lane] : nvp;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const uint32_t b = raw_elem<BF16, VEC>(bits, v);
            const bool cand = lane < nh && scored_at(e0 + v) && max(order_image(b), 1u) >= tau;
            const T k = cand ? KT::scored(b, e0 + v) : T(0);
            const uint64_t m = ballot(k != 0);
            if (m != 0) {
                const int pos = nc + (int)__builtin_amdgcn_mbcnt_hi(
                                         (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                if (k != 0 && pos < XSliceShared::MCAP) xs.mc[pos] = k;
                nc += __builtin_popcountll(m);
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    if (nh <= XSliceShared::SCAP && nc <= XSliceShared::MCAP) {
        const T x = lane < nc ? xs.mc[lane] : T(0);
        const T sorted = nc <= 32 ? flip_sort<true, 2, 32>(x, lane) : sort64_desc(x);
        return lane < 16 ? sorted : T(0);
    }
    const int n = nvp - base < CHUNK ? nvp - base : CHUNK;
    return topk16_of_list<T>(n, [&](int i) -> T {
        const int e = base + i;
        return scored_at(e) ? KT::scored(load_bits<BF16>(a.scores, row_off + e), e) : T(0);
    });
}

// A workgroup of S wavefronts per slice of S chunks of 64 lanes x 4 loads of 16 bytes;
// blockIdx = (row, head) x slices + slice.
template <bool BF16, bool FUSED>
__global__ __launch_bounds__(64 * kXSplitMaxWaves) void select_xsplit_kernel(
    const void* scores, const int32_t* rows0, int M, int nsl, uint32_t sl_mul, uint32_t sl_shift,
    uint32_t h_mul, uint32_t h_shift, uint32_t q_mul, uint32_t q_shift, int q, SelArgs a)
{
    using KT = KeyWide;
    using T = uint64_t;
    constexpr int VEC = BF16 ? 8 : 4;
    constexpr int U = chunk_loads<VEC>();
    constexpr int W = load_words<VEC>();
    constexpr int CHUNK = 64 * U * VEC;
    constexpr int ELEM = BF16 ? 2 : 4;
    constexpr int NCSEG = kSegmentTiles / CHUNK;   // streaming chunks per 8192-tile segment
    constexpr int NLOADS = kXSplitMaxSlices / 4;   // list loads per lane in the final merge
    __shared__ XSliceShared xs[kXSplitMaxWaves];
    __shared__ T tops[kXSplitMaxWaves][16];
    __shared__ WaveShared<T> one;
    const int S = uniform((int)(blockDim.x >> 6));
    const int wave = uniform((int)(threadIdx.x >> 6));
    const int lane = lane_id();
    const int64_t rh = divide_by(blockIdx.x, sl_mul, sl_shift);
    const int slice = (int)((int64_t)blockIdx.x - rh * nsl);
    const int64_t t = divide_by((uint32_t)rh, h_mul, h_shift);
    const int64_t row_off = rh * (int64_t)M;
    const void* row = static_cast<const char*>(scores) + row_off * ELEM;
    const int sbase = slice * S * CHUNK;   // first tile of this slice
    const int base = sbase + wave * CHUNK;  // first tile of this wavefront's chunk

    // the chunk's tiles, requested before the causal count is known (loads past the
    // row's capacity return zeros without a memory access)
    uint32_t buf[U][W];
    {
        const RowReader<BF16, VEC> cap(row, M * ELEM);
#pragma unroll
        for (int u = 0; u < U; ++u) cap.template load<true>(base + (u * 64 + lane) * VEC, buf[u]);
    }
    int64_t c;
    int req;
    const int nvp = uniform(row_count_lead<FUSED>(a, rows0, q, q_mul, q_shift, M, t, c, req));
    c = uniform(c);
    req = uniform(req);
    const int32_t* bt_row = FUSED && req >= 0 ? a.block_table + (int64_t)req * a.max_blocks : nullptr;
    const int ni = a.num_init, nl = a.num_local, topk = a.topk;
    const int lo_local = nvp - nl;
    int32_t* trow = FUSED ? a.out_table + rh * (int64_t)topk * kPagesPerBlock : nullptr;

    uint64_t top;
    if (nvp <= 2 * kWave) {
        // short row: wavefront 0 of slice 0 alone, without the workspace (the branch is
        // uniform over the row's workgroups)
        if (slice != 0 || wave != 0) return;
        const RowReader<BF16, 1> rd(row, nvp * ELEM);
        uint32_t w0[1], w1[1];
        rd.template load<false>(lane, w0);
        rd.template load<false>(lane + kWave, w1);
        top = (uint64_t)wave_select_row<BF16, true>(a.scores, row_off, nvp, ni, nl, w0[0], w1[0]);
    } else {
        // the slice's scored top-16 (nvp > 128 >= ni + nl: forced and scored ids are disjoint)
        const int ks = topk - ni - nl > 0 ? topk - ni - nl : 1;
        T mine = 0;
        if (base < nvp)
            mine = chunk_scored_top16<BF16, VEC>(a, row_off, nvp, base, ni, lo_local, ks, buf, xs[wave]);
        if (S > 1) {
            if (lane < 16) tops[wave][lane] = mine;
            __syncthreads();
            if (wave != 0) return;
            // up to eight sorted lists: four 16-lane rows in each of two registers
            const int la = lane >> 4, lb = la + 4;
            const T ra = la < S ? tops[la][lane & 15] : T(0);
            const T rb = lb < S ? tops[lb][lane & 15] : T(0);
            const T best = top16_of_sorted_rows(ra, rb);
            mine = lane < 16 ? best : T(0);
        }
        // publish the list (slices past the causal tiles have none), then arrive
        uint64_t* lists = a.ws_lists + rh * (int64_t)nsl * 16;
        if (sbase < nvp && lane < 16) ws_store(lists + slice * 16 + lane, mine);
        ws_order_release();
        uint32_t prev = 0;
        if (lane == 0)
            prev = __hip_atomic_fetch_add(a.ws_count + rh * kXSplitCounterStride, 1u,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = (uint32_t)uniform((int)prev);
        if (prev != (uint32_t)(nsl - 1)) return;
        ws_order_acquire();

        // the last slice to arrive: every list of a slice holding causal tiles, all
        // requested at once (four lists per load: lane l takes entry l % 16 of list
        // 4 i + l / 16), then folded eight at a time
        const int used = min(nsl, (nvp + S * CHUNK - 1) / (S * CHUNK));
        T r[NLOADS];
#pragma unroll
        for (int i = 0; i < NLOADS; ++i) {
            const int li = 4 * i + (lane >> 4);
            r[i] = 4 * i < used && li < used ? ws_load(lists + li * 16 + (lane & 15)) : T(0);
        }
        T carry = 0;
#pragma unroll
        for (int i = 0; i < NLOADS; i += 2) {
            if (4 * i < used) {
                const T best = top16_of_sorted_rows(r[i], r[i + 1]);
                carry = i == 0 ? (lane < 16 ? best : T(0)) : merge_top16(carry, best);
            }
        }
        // leave the workspace as it was found, all zeros: the counter, and the lists read
        // (another batch shape places its counters where these lists are)
        if (lane == 0)
            __hip_atomic_store(a.ws_count + rh * kXSplitCounterStride, 0u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int i = 0; i < NLOADS; ++i) {
            const int li = 4 * i + (lane >> 4);
            if (4 * i < used && li < used) ws_store(lists + li * 16 + (lane & 15), T(0));
        }
        // tiles past the slices (a row longer than the launch assumed), one 8192-tile
        // segment at a time
#pragma unroll 1
        for (int s0 = nsl * S * CHUNK; s0 < nvp; s0 += kSegmentTiles) {
            const int len = nvp - s0 < kSegmentTiles ? nvp - s0 : kSegmentTiles;
            int ph;
            bool hp;
            const T seg = (T)wave_stream_row<BF16, VEC, NCSEG, false, true>(
                a, row_off, nvp, bt_row, one, ph, hp, s0, len, false);
            carry = merge_top16(carry, seg);
        }
        top = forced_then<KT>(carry, nvp, ni, nl);
    }
    const int id = KT::block((T)top);
    if (lane < topk) a.out_idx[rh * topk + lane] = id;
    if constexpr (FUSED)
        emit_table_sorted(id, c, bt_row, a.max_blocks, topk, trow, a.out_ctx + rh,
                          a.table_vec != 0);
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
        const RowInfo ri = row_info(a.rows, divide_by((uint32_t)rh, a.h_mul, a.h_shift));
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

// The row description as the kernels' leading arguments take it (see row_count_lead).
template <bool FUSED>
const int32_t* lead_rows(const SelArgs& s)
{
    if (!FUSED) return s.rows.num_valid_pages;
    return s.rows.row_req == nullptr ? s.rows.seq_lens : s.rows.row_req;
}

template <bool FUSED>
int lead_q(const SelArgs& s)
{
    return FUSED && s.rows.row_req == nullptr ? s.rows.q : 0;
}

template <bool BF16, bool FUSED, int VEC, int NC>
hipError_t launch_wave(const SelArgs& args, int rhpb, hipStream_t stream)
{
    SelArgs s = args;
    s.rhpb = rhpb;
    const int64_t total = s.T * s.H;
    const int64_t blocks = (total + rhpb - 1) / rhpb;
    hipLaunchKernelGGL((select_wave_kernel<BF16, FUSED, VEC, NC>), dim3((unsigned)blocks),
                       dim3(kWave * rhpb), 0, stream, s.scores, lead_rows<FUSED>(s), total, s.M,
                       rhpb, s.h_mul, s.h_shift, s.rows.q_mul, s.rows.q_shift, lead_q<FUSED>(s),
                       s);
    return hipGetLastError();
}

// Rows longer than the fast path: wide keys, a workgroup of `waves` wavefronts per
// (row, head), one 8192-tile segment each.
template <bool BF16, bool FUSED, int VEC>
hipError_t launch_segments_vec(const SelArgs& s, int waves, hipStream_t stream)
{
    constexpr int NC = kSegmentTiles / (VEC == 1 ? 1024 : 64 * 4 * VEC);
    const int64_t total = s.T * s.H;
    hipLaunchKernelGGL((select_segment_kernel<BF16, FUSED, VEC, NC>), dim3((unsigned)total),
                       dim3(kWave * waves), 0, stream, lead_rows<FUSED>(s), s.M, s.h_mul,
                       s.h_shift, s.rows.q_mul, s.rows.q_shift, lead_q<FUSED>(s), s);
    return hipGetLastError();
}

template <bool BF16, bool FUSED>
hipError_t launch_wide(const SelArgs& s, int vec, int waves, hipStream_t stream)
{
    if (waves < 1 || waves > kSegmentMaxWaves) return hipErrorInvalidValue;
    if (vec == 1) return launch_segments_vec<BF16, FUSED, 1>(s, waves, stream);
    if constexpr (BF16) {
        if (vec == 8) return launch_segments_vec<true, FUSED, 8>(s, waves, stream);
    } else {
        if (vec == 4) return launch_segments_vec<false, FUSED, 4>(s, waves, stream);
    }
    return hipErrorInvalidValue;
}

template <bool BF16, bool FUSED, int VEC>
hipError_t launch_long_vec(const SelArgs& s, int chunks, hipStream_t stream)
{
    switch (chunks) {
        case 1: return launch_wave<BF16, FUSED, VEC, 1>(s, 4, stream);
        case 2: return launch_wave<BF16, FUSED, VEC, 2>(s, 4, stream);
        case 4: return launch_wave<BF16, FUSED, VEC, 4>(s, 4, stream);
        case 8: return launch_wave<BF16, FUSED, VEC, 8>(s, 4, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

template <bool BF16, bool FUSED>
hipError_t launch_long(const SelArgs& s, int vec, int chunks, hipStream_t stream)
{
    if (vec == 1) return launch_long_vec<BF16, FUSED, 1>(s, chunks, stream);
    if constexpr (BF16) {
        if (vec == 8) return launch_long_vec<true, FUSED, 8>(s, chunks, stream);
    } else {
        if (vec == 4) return launch_long_vec<false, FUSED, 4>(s, chunks, stream);
    }
    return hipErrorInvalidValue;
}

int pow2_at_least(int64_t x)
{
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

template <bool BF16, bool FUSED>
hipError_t launch_split(const SelArgs& s, int waves, hipStream_t stream)
{
    constexpr int VEC = BF16 ? 8 : 4;
    if (waves < 1 || waves > kSplitMaxWaves) return hipErrorInvalidValue;
    const int64_t total = s.T * s.H;
    hipLaunchKernelGGL((select_split_kernel<BF16, FUSED, VEC>), dim3((unsigned)total),
                       dim3(kWave * waves), 0, stream, s.scores, lead_rows<FUSED>(s), s.M, s.h_mul,
                       s.h_shift, s.rows.q_mul, s.rows.q_shift, lead_q<FUSED>(s), s);
    return hipGetLastError();
}

template <bool BF16, bool FUSED, int VEC>
hipError_t launch_wide_topk_vec(const SelArgs& s, hipStream_t stream)
{
    const int64_t total = s.T * s.H;
    hipLaunchKernelGGL((select_wide_topk_kernel<BF16, FUSED, VEC>), dim3((unsigned)((total + 3) / 4)),
                       dim3(4 * kWave), 0, stream, s);
    return hipGetLastError();
}

template <bool BF16, bool FUSED>
hipError_t launch_wide_topk(const SelArgs& s, bool vec, hipStream_t stream)
{
    if (vec) return launch_wide_topk_vec<BF16, FUSED, BF16 ? 8 : 4>(s, stream);
    return launch_wide_topk_vec<BF16, FUSED, 1>(s, stream);
}

template <bool BF16, bool FUSED>
hipError_t launch_xsplit(const SelArgs& s, int waves, hipStream_t stream)
{
    const int64_t total = s.T * s.H;
    const Divisor sd = make_divisor((uint32_t)s.slices);
    hipLaunchKernelGGL((select_xsplit_kernel<BF16, FUSED>), dim3((unsigned)(total * s.slices)),
                       dim3(kWave * waves), 0, stream, s.scores, lead_rows<FUSED>(s), s.M, s.slices,
                       sd.mul, sd.shift, s.h_mul, s.h_shift, s.rows.q_mul, s.rows.q_shift,
                       lead_q<FUSED>(s), s);
    return hipGetLastError();
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of the allocation-free fused call (kvbt_select_topk_and_build_table_noalloc):
// the cross-workgroup split's workspace as a file-scope device array, one copy per GPU,
// zero when the code object is loaded; every completed call leaves it all zeros again.
// Host code never uses the array's name as an address: its device address is looked up
// once per device (with that device current) and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KVBT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

hipError_t noalloc_scratch(void** out)
{
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

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
    const Divisor qd = make_divisor((uint32_t)s.rows.q), hd = make_divisor((uint32_t)l.H);
    s.rows.q_mul = qd.mul;
    s.rows.q_shift = qd.shift;
    s.h_mul = hd.mul;
    s.h_shift = hd.shift;
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
    s.front = l.num_decode_rows * l.H;
    s.ws_count = nullptr;
    s.ws_lists = nullptr;
    s.slices = 1;
    const bool bf16 = l.dtype == KVBT_BF16;

    if (l.policy.path == 5) {
        // topk above 16: 16-byte loads when rows are 16-byte multiples and the buffer is aligned
        const bool vec = l.policy.vec > 1 && ((uintptr_t)l.scores % 16) == 0;
        if (bf16) return l.fused ? launch_wide_topk<true, true>(s, vec, stream)
                                 : launch_wide_topk<true, false>(s, vec, stream);
        return l.fused ? launch_wide_topk<false, true>(s, vec, stream)
                       : launch_wide_topk<false, false>(s, vec, stream);
    }
    if (l.policy.path == 4) {
        // the workspace: counters first (one per (row, head), 256-byte aligned block),
        // then the slices' lists
        const int waves = l.policy.threads_per_block / kWave;
        if (l.workspace == nullptr || l.policy.slices < 1 || l.policy.slices > kXSplitMaxSlices ||
            waves < 1 || waves > kXSplitMaxWaves || ((uintptr_t)l.scores % 16) != 0)
            return hipErrorInvalidValue;
        s.slices = l.policy.slices;
        s.ws_count = static_cast<uint32_t*>(l.workspace);
        s.ws_lists = reinterpret_cast<uint64_t*>(static_cast<char*>(l.workspace) +
                                                 xsplit_counter_bytes(total));
        if (bf16) return l.fused ? launch_xsplit<true, true>(s, waves, stream)
                                 : launch_xsplit<true, false>(s, waves, stream);
        return l.fused ? launch_xsplit<false, true>(s, waves, stream)
                       : launch_xsplit<false, false>(s, waves, stream);
    }

    if (l.policy.path == 0) {
        if (bf16) return l.fused ? launch_wave<true, true, 1, 0>(s, s.rhpb, stream)
                                 : launch_wave<true, false, 1, 0>(s, s.rhpb, stream);
        return l.fused ? launch_wave<false, true, 1, 0>(s, s.rhpb, stream)
                       : launch_wave<false, false, 1, 0>(s, s.rhpb, stream);
    }
    const bool aligned = ((uintptr_t)l.scores % 16) == 0;
    if (l.M > kSegmentTiles) {
        const int vec = aligned ? l.policy.vec : 1;
        const int waves = l.policy.threads_per_block / kWave;
        if (bf16) return l.fused ? launch_wide<true, true>(s, vec, waves, stream)
                                 : launch_wide<true, false>(s, vec, waves, stream);
        return l.fused ? launch_wide<false, true>(s, vec, waves, stream)
                       : launch_wide<false, false>(s, vec, waves, stream);
    }
    if (l.policy.path == 2 && aligned) {
        if (bf16) return l.fused ? launch_split<true, true>(s, l.policy.chunks, stream)
                                 : launch_split<true, false>(s, l.policy.chunks, stream);
        return l.fused ? launch_split<false, true>(s, l.policy.chunks, stream)
                       : launch_split<false, false>(s, l.policy.chunks, stream);
    }
    int vec = l.policy.path == 1 ? l.policy.vec : 1;
    int chunks = l.policy.path == 1 ? l.policy.chunks : 0;
    if (vec == 1 || !aligned) {
        // single-element loads: chunks of 64 lanes x 16 loads
        vec = 1;
        chunks = pow2_at_least((l.M + 1023) / 1024);
    }
    if (bf16) return l.fused ? launch_long<true, true>(s, vec, chunks, stream)
                             : launch_long<true, false>(s, vec, chunks, stream);
    return l.fused ? launch_long<false, true>(s, vec, chunks, stream)
                   : launch_long<false, false>(s, vec, chunks, stream);
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
    const Divisor qd = make_divisor((uint32_t)s.rows.q), hd = make_divisor((uint32_t)l.H);
    s.rows.q_mul = qd.mul;
    s.rows.q_shift = qd.shift;
    s.h_mul = hd.mul;
    s.h_shift = hd.shift;
    s.block_table = l.block_table;
    s.max_blocks = l.max_blocks;
    s.out_table = l.out_table;
    s.out_ctx = l.out_ctx;
    s.table_vec = ((uintptr_t)l.out_table % 16) == 0;
    if (l.topk > kMaxTopk) {
        hipLaunchKernelGGL(table_wide_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0,
                           stream, s);
        return hipGetLastError();
    }
    const int64_t blocks = (total + 15) / 16;
    hipLaunchKernelGGL(table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, s);
    return hipGetLastError();
}

}  // namespace kvbt
