// kvbt_attn.hip -- sparse paged-attention decode over the page-16 sparse block table,
// for gfx950 (MI355X).
//
// The consumer of the sparse table (vLLM PR #47984 report, "[ROCm][MiniMax-M3][Spec
// Decode] Support speculative decode with AITER sparse PA", Summary and Implementation
// breakdown items 1-3): each (row, index head) attends over the ctx tokens its page
// list names, token i being slot i % 16 of page table[i / 16]; the G query heads of
// the head's group share those tokens. The pages print no kernel; this one is our own.
//
// Work: a workgroup per (row, index head), W wavefronts taking its pages round robin.
// A wavefront keeps the head group's queries as the B operand of the score MFMA and
// streams pages: per 16-token page, four v_mfma_f32_16x16x32_bf16 give the 16 x 16
// block of scores (tokens x query heads) straight from the page's keys -- the cache's
// K layout [page][head][D/8][16][8] hands every lane its 16 contiguous bytes -- then
// an online softmax per query head (running max, rescale), and eight
// v_mfma_f32_16x16x16_bf16 accumulate O^T += V^T P^T, the cache's V layout
// [page][head][D][16] giving each lane the 8 contiguous bytes of 4 tokens of one
// dimension that the score MFMA's output layout pairs with. Probabilities enter that
// MFMA as bf16 (rounded to nearest even); their sum is taken over the same rounded
// values, so the output is a convex combination of the values. The wavefronts' partial
// (max, sum, O) are merged in LDS in a fixed order. A batch of few (row, head) pairs may
// split each pair over 2-8 workgroups (the call with a workspace): each takes a
// contiguous share of the row's pages, and the last to finish merges the shares'
// partial results in split order through the caller's workspace.
//
// Each page is read through a buffer resource of its own: a page id outside
// [0, num_pages) gets an empty range, so its loads return zeros without touching
// memory (zero keys and values), and so do the prefetches past the row's last page.
// With one decode row per request no two workgroups read the same page, and the
// loads are nontemporal (random 4 KB pages then stream at the sequential read rate);
// the speculative rows of one request share most pages, so there they stay cacheable
// for the L2 hits the XCD-aware order sets up.
// The kernel is HBM bound (8 KB of keys and values per page and KV head against 16
// query heads at most); the MFMAs keep the arithmetic off the vector ALU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvbt_attn_launch.h"
#include "kvbt_device.h"

namespace kvbt {
namespace {

constexpr int kPageTokens = 16;
constexpr int kHeadDim = 128;
constexpr int kPageBytes = kPageTokens * kHeadDim * 2;   // one page of one KV head, K or V
constexpr int kBufferFlags = 0x00020000;                  // raw buffer, 32-bit data format

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int P>
__device__ __forceinline__ float xor_f(float x)
{
    return __uint_as_float(xor_lane<P>(__float_as_uint(x)));
}

// bf16 bits of x, rounded to nearest even
__device__ __forceinline__ uint32_t bf16_bits(float x)
{
    const __bf16 b = (__bf16)x;
    return (uint32_t)__builtin_bit_cast(unsigned short, b);
}

__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi)
{
    return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

__device__ __forceinline__ float bf16_value(uint32_t bits)
{
    return __uint_as_float(bits << 16);
}

// One page of one KV head as this lane holds it: keys for the score MFMA (4 x 16 B)
// and values for the output MFMA (8 x 8 B).
struct PageRegs {
    u32x4 k[4];
    u32x2 v[8];
};

struct Row {
    const unsigned char* kc;
    const unsigned char* vc;
    int64_t head_slab;      // h * kPageBytes
    int64_t page_stride;    // H * kPageBytes
    uint32_t num_pages;
    uint32_t tab0, tab1;    // table entries lane and lane + 64 of this row
    int pend;               // one past the last page this workgroup reads
};

// One page (id `id`, read only when `ok`) of the row's KV head into this lane's registers.
template <bool NT>
__device__ __forceinline__ void load_slab(PageRegs& r, const Row& w, uint32_t id, bool ok, int lane)
{
    constexpr int aux = NT ? 2 : 0;   // nontemporal: stream past the caches
    const uint32_t uid = ok ? id : 0u;
    const int64_t off = (int64_t)uid * w.page_stride + w.head_slab;
    const int nrec = ok ? kPageBytes : 0;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(w.kc + off),
                                                      (short)0, nrec, kBufferFlags);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(w.vc + off),
                                                      (short)0, nrec, kBufferFlags);
    // keys: step s holds dims 32s + 8g .. + 8 of token (lane & 15), g = lane >> 4
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        r.k[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rk, lane * 16, s * 1024, aux));
        __builtin_amdgcn_sched_barrier(0);
    }
    // values: block j holds tokens 4g .. 4g + 3 of dimension 16j + (lane & 15)
    const int vo = (lane & 15) * 32 + (lane >> 4) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        r.v[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                               rv, vo, j * 512, aux));
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Page p of the row's list (pages from w.pend on read as zeros without a load).
template <bool NT>
__device__ __forceinline__ void load_page(PageRegs& r, const Row& w, int p, int lane)
{
    // page id from the table (a uniform index into the two table registers)
    const int pp = p < w.pend ? p : 0;
    const uint32_t id = (uint32_t)__builtin_amdgcn_readlane((int)(pp < 64 ? w.tab0 : w.tab1),
                                                            pp & 63);
    load_slab<NT>(r, w, id, p < w.pend && id < w.num_pages, lane);
}

// Rescaling of the running sums is lazy: the reference max of a query head moves only
// when a page's scores exceed it by more than this many powers of two (or on the first
// page), decided for the whole wavefront at once, so the accumulators stay in place on
// almost every page. Unnormalised probabilities then stay below 2^8.
constexpr float kRescaleLog2 = 8.f;

// Page buffers per wavefront (32 VGPRs each).
constexpr int kDepth = 2;

struct Acc {
    floatx4 o[8];   // O^T: block j, element i = dim 16j + 4g + i of query head (lane & 15)
    float m;        // reference max of the scaled log2 scores of this lane's query head
    float l;        // running sum of the rounded probabilities (this lane's tokens)
};

template <bool FIRST>
__device__ __forceinline__ void attend_page(Acc& acc, const PageRegs& r, const bf16x8 (&qb)[4],
                                            float c2, int tok0, int ctx, int lane)
{
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k[k]), qb[k],
                                                   s, 0, 0, 0);
    // s[i]: score of token tok0 + 4g + i for query head (lane & 15)
    const int t0 = tok0 + (lane >> 4) * 4;
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = t0 + i < ctx ? s[i] * c2 : -__builtin_inff();
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, xor_f<16>(mx));
    mx = fmaxf(mx, xor_f<32>(mx));                 // finite: every page has a token
    if constexpr (FIRST) {
        acc.m = mx;                                // the sums are still zero
    } else if (__builtin_amdgcn_ballot_w64(mx > acc.m + kRescaleLog2) != 0) {
        const float m_new = fmaxf(acc.m, mx);
        const float alpha = __builtin_amdgcn_exp2f(acc.m - m_new);
        acc.l *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc.o[j] *= alpha;
        acc.m = m_new;
    }
    uint32_t pb[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pb[i] = bf16_bits(__builtin_amdgcn_exp2f(x[i] - acc.m));
        psum += bf16_value(pb[i]);
    }
    acc.l += psum;
    const short4_t pv = {(short)pb[0], (short)pb[1], (short)pb[2], (short)pb[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc.o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(short4_t, r.v[j]), pv, acc.o[j], 0, 0, 0);
}

// Split across workgroups (SPLIT): the S workgroups of one (row, head) take contiguous
// shares of its page list; each publishes its partial (max, sum, O) to the caller's
// workspace and increments the pair's arrival counter, and the last to arrive merges
// the S partial results in split order (a fixed order, whichever arrives last) and
// writes the outputs.
// Workspace layout, in 256-byte lines: the first 16 bytes of line k hold the arrival
// counter of pair k (lines past the batch's pairs leave theirs unused), the other 240
// bytes 15 slots of 16 bytes of partial results, numbered across lines. Partial results
// never touch a counter, and the last workgroup of a pair sets its counter back to
// zero, so the counters of every batch shape find zeros without any clearing.
constexpr int kPartSlotsPerLine = 15;
constexpr int kPartSlots = 8 * 64 + 8;   // one partial result: O (8 x 64 slots), (m, l)

__device__ __forceinline__ uint64_t* part_slot(void* ws, uint32_t slot)
{
    const uint32_t line = slot / kPartSlotsPerLine;
    const uint32_t in = slot - line * kPartSlotsPerLine;
    return (uint64_t*)((unsigned char*)ws + (uint64_t)line * 256 + 16 + in * 16);
}

__device__ __forceinline__ uint64_t pack2(float lo, float hi)
{
    return (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
}

// Four wavefronts per SIMD (at most 128 VGPRs; the kernel fits without spilling): with
// three, 64 long-context rows x 4 heads ran 44.5 against 43.0 us, the split 16 and 64
// spec-decode rows 11.4 and 18.8 against 11.1 and 18.0 us.
template <int W, bool OUT_BF16, bool NT, bool SPLIT>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(4))) void sparse_attn_kernel(AttnArgs a)
{
    __shared__ float sm_m[W > 1 ? W : 1][16];
    __shared__ float sm_l[W > 1 ? W : 1][16];
    __shared__ floatx4 sm_o[W > 1 ? W : 1][8][64];
    __shared__ uint32_t sm_arrived;

    const int lane = lane_id();
    const int wave = uniform((int)(threadIdx.x >> 6));
    // XCD-aware order: workgroups are dealt to the 8 XCDs round robin, so block b runs on
    // XCD b % 8; giving each XCD a contiguous range of (row, head) pairs keeps the rows of
    // one request, whose page lists overlap, on one L2 at about the same time (the S
    // workgroups of a split pair are neighbours in that order)
    const uint32_t nb = gridDim.x, b = blockIdx.x;
    const uint32_t xcd = b & 7u, full = nb >> 3, rem = nb & 7u;
    const uint32_t unit = xcd * full + (xcd < rem ? xcd : rem) + (b >> 3);
    const int64_t pair = SPLIT ? (int64_t)(unit / (uint32_t)a.splits) : (int64_t)unit;
    const int split = SPLIT ? uniform((int)(unit - (uint32_t)pair * (uint32_t)a.splits)) : 0;
    const int t = uniform((int)(pair / a.H));
    const int h = uniform((int)(pair - (int64_t)t * a.H));
    const int n = lane & 15;
    const int g = lane >> 4;

    const int64_t rh = (int64_t)t * a.H + h;
    int ctx = a.ctx[rh];
    ctx = ctx < 0 ? 0 : (ctx > kPageTokens * a.width ? kPageTokens * a.width : ctx);
    ctx = uniform(ctx);

    Row w;
    w.kc = (const unsigned char*)a.k_cache;
    w.vc = (const unsigned char*)a.v_cache;
    w.head_slab = (int64_t)h * kPageBytes;
    w.page_stride = (int64_t)a.H * kPageBytes;
    w.num_pages = (uint32_t)a.num_pages;
    // this workgroup's pages [p_lo, pend): the whole row, or split s's contiguous share
    const int npages = (ctx + kPageTokens - 1) / kPageTokens;
    int p_lo = 0;
    w.pend = npages;
    if constexpr (SPLIT) {
        p_lo = uniform(split * npages / a.splits);
        w.pend = uniform((split + 1) * npages / a.splits);
    }
    {
        const auto rt = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int32_t*>(a.table + rh * a.width), (short)0, a.width * 4, kBufferFlags);
        w.tab0 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rt, lane * 4, 0, 0);
        w.tab1 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rt, (lane + 64) * 4, 0, 0);
    }

    // queries of the group as the B operand: step k holds dims 32k + 8g .. + 8 of query
    // head n (zero for the padding heads n >= G, which fall outside the range)
    bf16x8 qb[4];
    {
        const int64_t q0 = ((int64_t)t * a.H + h) * a.G * (kHeadDim * 2);
        const auto rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void*>((const void*)((const unsigned char*)a.q + q0)), (short)0,
            a.G * kHeadDim * 2, kBufferFlags);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            qb[k] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rq, n * (kHeadDim * 2) + (32 * k + 8 * g) * 2,
                                                   0, 0));
    }

    Acc acc;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc.o[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    acc.m = -__builtin_inff();
    acc.l = 0.f;

    // pages p = wave, wave + W, ...: two page buffers, each refilled with the page two
    // steps ahead as soon as it has been used, so one page stays in flight while the
    // other is attended to. The loop takes two pages per turn and has no exit inside,
    // so its head is entered only with the other buffer's loads the most recent (an exit
    // between the two steps let the compiler wait for every load there).
    static_assert(kDepth == 2, "the loop below alternates two buffers");
    PageRegs buf0, buf1;
    load_page<NT>(buf0, w, p_lo + wave, lane);
    load_page<NT>(buf1, w, p_lo + wave + W, lane);
    int p = p_lo + wave;
    if (p < w.pend) {
        attend_page<true>(acc, buf0, qb, a.c2, p * kPageTokens, ctx, lane);
        load_page<NT>(buf0, w, p + 2 * W, lane);
        p += W;
        for (; p + W < w.pend; p += 2 * W) {
            attend_page<false>(acc, buf1, qb, a.c2, p * kPageTokens, ctx, lane);
            load_page<NT>(buf1, w, p + 2 * W, lane);
            attend_page<false>(acc, buf0, qb, a.c2, (p + W) * kPageTokens, ctx, lane);
            load_page<NT>(buf0, w, p + 3 * W, lane);
        }
        if (p < w.pend) attend_page<false>(acc, buf1, qb, a.c2, p * kPageTokens, ctx, lane);
    }
    acc.l += xor_f<16>(acc.l);
    acc.l += xor_f<32>(acc.l);

    // merge the wavefronts' partial results (fixed order) and write this lane's outputs,
    // or (split) publish them; wavefront v holds dimension blocks j = v * (8 / W) ...
    constexpr int kJPerWave = 8 / W;
    float mall, lsum;
    floatx4 ot[kJPerWave];          // relative to exp2(mall), not normalised
    if constexpr (W > 1) {
        if (lane < 16) {
            sm_m[wave][lane] = acc.m;
            sm_l[wave][lane] = acc.l;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) sm_o[wave][j][lane] = acc.o[j];
        __syncthreads();
        mall = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < W; ++v) mall = fmaxf(mall, sm_m[v][n]);
        float wscale[W];
        lsum = 0.f;
#pragma unroll
        for (int v = 0; v < W; ++v) {
            const float mv = sm_m[v][n];
            wscale[v] = mv == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mv - mall);
            lsum += wscale[v] * sm_l[v][n];
        }
#pragma unroll
        for (int jj = 0; jj < kJPerWave; ++jj) {
            ot[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < W; ++v) ot[jj] += wscale[v] * sm_o[v][wave * kJPerWave + jj][lane];
        }
    } else {
        mall = acc.m;
        lsum = acc.l;
#pragma unroll
        for (int jj = 0; jj < kJPerWave; ++jj) ot[jj] = acc.o[jj];
    }
    const int64_t orow = ((int64_t)t * a.H * a.G + (int64_t)h * a.G + n) * kHeadDim;
    auto write_out = [&](const floatx4 (&o)[kJPerWave], float inv_l) {
#pragma unroll
        for (int jj = 0; jj < kJPerWave; ++jj) {
            const int j = W == 1 ? jj : wave * kJPerWave + jj;
            const floatx4 v = o[jj] * inv_l;
            const int64_t e = orow + 16 * j + 4 * g;
            if constexpr (OUT_BF16) {
                u32x2 pk;
                pk[0] = bf16_pack(v[0], v[1]);
                pk[1] = bf16_pack(v[2], v[3]);
                *(u32x2*)((uint16_t*)a.out + e) = pk;
            } else {
                *(floatx4*)((float*)a.out + e) = v;
            }
        }
    };
    if constexpr (!SPLIT) {
        if (n < a.G) write_out(ot, lsum > 0.f ? 1.f / lsum : 0.f);
    } else {
        const int S = a.splits;
        // publish: O slot (j, lane) of this split's record, then (m, l) per query head
        const uint32_t base = ((uint32_t)pair * (uint32_t)S + (uint32_t)split) * kPartSlots;
        if (n < a.G) {
#pragma unroll
            for (int jj = 0; jj < kJPerWave; ++jj) {
                const int j = W == 1 ? jj : wave * kJPerWave + jj;
                uint64_t* d = part_slot(a.ws, base + j * 64 + lane);
                ws_store(d, pack2(ot[jj][0], ot[jj][1]));
                ws_store(d + 1, pack2(ot[jj][2], ot[jj][3]));
            }
            if (wave == 0 && lane < 16)
                ws_store(part_slot(a.ws, base + 512 + (lane >> 1)) + (lane & 1), pack2(mall, lsum));
        }
        // arrive once every wavefront's stores are complete; the last of the pair's
        // workgroups to arrive merges
        ws_order_release();
        __syncthreads();
        uint32_t* cnt = (uint32_t*)((unsigned char*)a.ws + pair * 256);
        if (threadIdx.x == 0)
            sm_arrived = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (uniform((int)sm_arrived) != S - 1) return;
        ws_order_acquire();
        if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (n >= a.G) return;
        // every split's (m, l) for this lane's query head, then the O blocks weighted and
        // summed in split order
        float ms[kAttnMaxSplits], ls[kAttnMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kAttnMaxSplits; ++sp) {
            ms[sp] = -__builtin_inff();
            ls[sp] = 0.f;
            if (sp >= S) continue;
            if (sp == split) {
                ms[sp] = mall;
                ls[sp] = lsum;
                continue;
            }
            const uint32_t bs = ((uint32_t)pair * (uint32_t)S + (uint32_t)sp) * kPartSlots;
            const uint64_t ml = ws_load(part_slot(a.ws, bs + 512 + (n >> 1)) + (n & 1));
            ms[sp] = __uint_as_float((uint32_t)ml);
            ls[sp] = __uint_as_float((uint32_t)(ml >> 32));
        }
        float mt = -__builtin_inff();
#pragma unroll
        for (int sp = 0; sp < kAttnMaxSplits; ++sp) mt = fmaxf(mt, ms[sp]);
        float lt = 0.f;
        floatx4 o[kJPerWave];
#pragma unroll
        for (int jj = 0; jj < kJPerWave; ++jj) o[jj] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sp = 0; sp < kAttnMaxSplits; ++sp) {
            if (sp >= S) continue;
            const float wsc = ms[sp] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ms[sp] - mt);
            lt += wsc * ls[sp];
            const uint32_t bs = ((uint32_t)pair * (uint32_t)S + (uint32_t)sp) * kPartSlots;
#pragma unroll
            for (int jj = 0; jj < kJPerWave; ++jj) {
                floatx4 ov;
                if (sp == split) {
                    ov = ot[jj];
                } else {
                    const int j = W == 1 ? jj : wave * kJPerWave + jj;
                    const uint64_t* d = part_slot(a.ws, bs + j * 64 + lane);
                    const uint64_t lo = ws_load(d), hi = ws_load(d + 1);
                    ov = floatx4{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                                 __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
                }
                o[jj] += wsc * ov;
            }
        }
        write_out(o, lt > 0.f ? 1.f / lt : 0.f);
    }
}

// ---------------------------------------------------------------------------
// Request-grouped decode (more than one row per request). The speculative rows of one
// request list mostly the same pages, so a workgroup takes up to kGroupRows rows of one
// request for one KV head: it lists the distinct pages of their page lists once (an LDS
// hash of the page ids, ordered by each page's first entry, row by row), then streams
// every distinct page once, nontemporally. Per page the score and output MFMAs run with
// the rows' query heads side by side in their 16 columns (CT column tiles of R = 16 / G
// rows), each column masked to the tokens its own row takes from that page (none when
// the row does not list it). If a row lists one page twice, every table entry becomes
// its own item instead, for that row alone: the results stay those of the definition
// for any table.
// ---------------------------------------------------------------------------
constexpr int kGroupRows = 4;                         // rows per workgroup at most
constexpr int kGroupEntries = kGroupRows * 128;       // table entries of a group at most
constexpr int kHashSlots = 1024;                      // at most half full
constexpr int64_t kGroupMinWorkgroups = 256;          // one per compute unit
// split per-row launches (a caller's workspace): below kSplitMaxPairs (row, head) pairs,
// 4 workgroups each up to kSplitFourPairs pairs, else 2
constexpr int64_t kSplitMaxPairs = 160;
constexpr int64_t kSplitFourPairs = 64;

template <int W>
struct GroupShared {
    union {
        struct {
            int32_t key[kHashSlots];     // page id (-2 for every invalid id), -1 empty
            int32_t first[kHashSlots];   // smallest entry (row * 128 + position) with it
            uint32_t count[kHashSlots];  // byte i: entries of row i with it
            uint32_t pos[kHashSlots];    // byte i: the position of that entry, 0xFF none
        } h;
        struct {                         // the wavefronts' partial results, one tile
            float m[W][16];
            float l[W][16];
            floatx4 o[W][8][64];
        } mg;
    } u;
    int2 item[kGroupEntries];            // distinct pages: id, positions (a byte per row)
    int wave_count[W];
    int dup;
};

__device__ __forceinline__ int pick4(int i, int v0, int v1, int v2, int v3)
{
    return i == 0 ? v0 : (i == 1 ? v1 : (i == 2 ? v2 : v3));
}

// One column tile of a page: as attend_page, for columns that may have no token on it
// (tok0 < 0: the column's row does not list the page).
__device__ __forceinline__ void attend_tile(Acc& acc, const PageRegs& r, const bf16x8 (&qb)[4],
                                            float c2, int tok0, int ctx, int lane)
{
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k[k]), qb[k],
                                                   s, 0, 0, 0);
    const int t0 = tok0 + (lane >> 4) * 4;
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = tok0 >= 0 && t0 + i < ctx ? s[i] * c2 : -__builtin_inff();
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, xor_f<16>(mx));
    mx = fmaxf(mx, xor_f<32>(mx));
    if (__builtin_amdgcn_ballot_w64(mx > acc.m + kRescaleLog2) != 0) {
        const float m_new = fmaxf(acc.m, mx);
        const float alpha = m_new == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(acc.m - m_new);
        acc.l *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc.o[j] *= alpha;
        acc.m = m_new;
    }
    uint32_t pb[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pb[i] = x[i] == -__builtin_inff() ? 0u : bf16_bits(__builtin_amdgcn_exp2f(x[i] - acc.m));
        psum += bf16_value(pb[i]);
    }
    acc.l += psum;
    const short4_t pv = {(short)pb[0], (short)pb[1], (short)pb[2], (short)pb[3]};
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc.o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(short4_t, r.v[j]), pv, acc.o[j], 0, 0, 0);
}

template <int W, int CT, bool OUT_BF16, bool NT>
__global__ __launch_bounds__(64 * W) void sparse_attn_group_kernel(AttnArgs a)
{
    __shared__ GroupShared<W> sh;
    constexpr int kThreads = 64 * W;
    constexpr int kPerThread = kGroupEntries / kThreads;
    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = uniform((int)(threadIdx.x >> 6));
    const int n = lane & 15;
    const int g = lane >> 4;
    // XCD-aware order over (group, head) pairs, as in the per-row kernel
    const uint32_t nb = gridDim.x, b = blockIdx.x;
    const uint32_t xcd = b & 7u, full = nb >> 3, rem = nb & 7u;
    const int64_t pair = (int64_t)(xcd * full + (xcd < rem ? xcd : rem) + (b >> 3));
    const int64_t grp = pair / a.H;
    const int h = uniform((int)(pair - grp * a.H));
    const int64_t req = grp / a.groups_per_req;
    const int sub = uniform((int)(grp - req * a.groups_per_req));
    const int64_t qr = a.rows_per_req;
    const int64_t row_lo = req * qr + (int64_t)sub * a.group_rows;
    int64_t row_hi = req * qr + (int64_t)(sub + 1) * a.group_rows;
    if (row_hi > (req + 1) * qr) row_hi = (req + 1) * qr;
    if (row_hi > a.T) row_hi = a.T;
    const int nrows = uniform((int)(row_hi > row_lo ? row_hi - row_lo : 0));
    if (nrows == 0) return;                      // the whole workgroup

    const int cmax = kPageTokens * a.width;
    int cr[kGroupRows];
#pragma unroll
    for (int i = 0; i < kGroupRows; ++i) {
        int c = i < nrows ? a.ctx[(row_lo + i) * a.H + h] : 0;
        c = c < 0 ? 0 : (c > cmax ? cmax : c);
        cr[i] = uniform(c);
    }

    // the distinct pages of the group's lists
    for (int e = tid; e < kHashSlots; e += kThreads) {
        sh.u.h.key[e] = -1;
        sh.u.h.first[e] = 0x7FFFFFFF;
        sh.u.h.count[e] = 0u;
        sh.u.h.pos[e] = 0xFFFFFFFFu;
    }
    if (tid == 0) sh.dup = 0;
    __syncthreads();
    uint32_t slot[kPerThread];
    int page[kPerThread];
#pragma unroll
    for (int m = 0; m < kPerThread; ++m) {
        const int e = tid + m * kThreads;
        const int i = e >> 7, k = e & 127;
        slot[m] = 0u;
        page[m] = -2;
        const int np = (pick4(i, cr[0], cr[1], cr[2], cr[3]) + kPageTokens - 1) / kPageTokens;
        if (i < nrows && k < np) {
            const int id = a.table[((row_lo + i) * a.H + h) * a.width + k];
            const int key = (uint32_t)id < (uint32_t)a.num_pages ? id : -2;
            uint32_t s = ((uint32_t)key * 2654435761u) >> 22;
            for (;;) {                           // ends: at most half the slots are used
                const int old = atomicCAS(&sh.u.h.key[s], -1, key);
                if (old == -1 || old == key) break;
                s = (s + 1) & (kHashSlots - 1);
            }
            atomicMin(&sh.u.h.first[s], e);
            const uint32_t before = atomicAdd(&sh.u.h.count[s], 1u << (8 * i));
            if ((before >> (8 * i)) & 0xFFu) sh.dup = 1;
            atomicAnd(&sh.u.h.pos[s], ~((0xFFu ^ (uint32_t)k) << (8 * i)));
            slot[m] = s;
            page[m] = key;
        }
    }
    __syncthreads();
    // items in entry order: a page's first entry owns it (every entry when a row lists
    // a page twice)
    const bool dup = uniform(sh.dup) != 0;
    int nitems = 0;
#pragma unroll
    for (int m = 0; m < kPerThread; ++m) {
        const int e = tid + m * kThreads;
        const int i = e >> 7, k = e & 127;
        const int np = (pick4(i, cr[0], cr[1], cr[2], cr[3]) + kPageTokens - 1) / kPageTokens;
        const bool act = i < nrows && k < np;
        const bool own = act && (dup || sh.u.h.first[slot[m]] == e);
        int2 it = {page[m], -1};
        if (own) {
            it.y = dup ? (int)(0xFFFFFFFFu ^ ((0xFFu ^ (uint32_t)k) << (8 * i)))
                       : (int)sh.u.h.pos[slot[m]];
        }
        const uint64_t bal = __builtin_amdgcn_ballot_w64(own);
        const int inwave = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (lane == 0) sh.wave_count[wave] = __builtin_popcountll(bal);
        __syncthreads();
        int at = nitems, total = 0;
#pragma unroll
        for (int v = 0; v < W; ++v) {
            const int cnt = sh.wave_count[v];
            at += v < wave ? cnt : 0;
            total += cnt;
        }
        if (own) sh.item[at + inwave] = it;
        nitems += total;
        __syncthreads();
    }
    nitems = uniform(nitems);

    // this lane's column in each tile: row, context, query head
    const int R = 16 / a.G;
    int crow[CT], cctx[CT];
    bf16x8 qb[CT][4];
    {
        const int64_t rowq = (int64_t)a.H * a.G * (kHeadDim * 2);    // bytes per row of q
        const unsigned char* q0 = (const unsigned char*)a.q + (row_lo * a.H + h) * a.G * (kHeadDim * 2);
        const int nrec = (int)((int64_t)(nrows - 1) * rowq + a.G * (kHeadDim * 2));
        const auto rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(q0), (short)0,
                                                          nrec, kBufferFlags);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const int ri = c * R + n / a.G;
            const bool ok = n < R * a.G && ri < nrows;
            crow[c] = ok ? ri : -1;
            cctx[c] = ok ? pick4(ri, cr[0], cr[1], cr[2], cr[3]) : 0;
            const int qo = ok ? (int)(ri * rowq) + (n % a.G) * (kHeadDim * 2) : nrec;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                qb[c][k] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rq, qo + (32 * k + 8 * g) * 2, 0, 0));
        }
    }

    Row w;
    w.kc = (const unsigned char*)a.k_cache;
    w.vc = (const unsigned char*)a.v_cache;
    w.head_slab = (int64_t)h * kPageBytes;
    w.page_stride = (int64_t)a.H * kPageBytes;
    w.num_pages = (uint32_t)a.num_pages;

    Acc acc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[c].o[j] = floatx4{0.f, 0.f, 0.f, 0.f};
        acc[c].m = -__builtin_inff();
        acc[c].l = 0.f;
    }
    auto load_item = [&](PageRegs& r, int j) {
        const int id = j < nitems ? uniform(sh.item[j].x) : -2;
        load_slab<NT>(r, w, (uint32_t)id, id >= 0, lane);
    };
    // items j = wave, wave + W, ...: two page buffers, each refilled with the item two
    // steps ahead as soon as it has been used. The loop takes two items per turn and has
    // no exit inside, so its head is entered only with the second buffer's loads the
    // most recent and the wait for the first buffer leaves those in flight (an exit
    // between the two steps let the compiler wait for every load there).
    static_assert(kDepth == 2, "the loop below alternates two buffers");
    PageRegs buf0, buf1;
    load_item(buf0, wave);
    load_item(buf1, wave + W);
    auto step = [&](PageRegs& r, int j) {
        const uint32_t posw = (uint32_t)uniform(sh.item[j].y);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const uint32_t pc = crow[c] >= 0 ? (posw >> (8 * crow[c])) & 0xFFu : 0xFFu;
            attend_tile(acc[c], r, qb[c], a.c2, pc == 0xFFu ? -1 : (int)pc * kPageTokens,
                        cctx[c], lane);
        }
        load_item(r, j + 2 * W);
    };
    int j = wave;
    for (; j + W < nitems; j += 2 * W) {
        step(buf0, j);
        step(buf1, j + W);
    }
    if (j < nitems) step(buf0, j);

    // merge the wavefronts' partial results tile by tile (fixed order) and write
    constexpr int kJPerWave = 8 / W;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        Acc& ac = acc[c];
        ac.l += xor_f<16>(ac.l);
        ac.l += xor_f<32>(ac.l);
        float wscale[W];
        float inv_l;
        if constexpr (W > 1) {
            if (lane < 16) {
                sh.u.mg.m[wave][lane] = ac.m;
                sh.u.mg.l[wave][lane] = ac.l;
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) sh.u.mg.o[wave][jj][lane] = ac.o[jj];
            __syncthreads();
            float mall = -__builtin_inff();
#pragma unroll
            for (int v = 0; v < W; ++v) mall = fmaxf(mall, sh.u.mg.m[v][n]);
            float lsum = 0.f;
#pragma unroll
            for (int v = 0; v < W; ++v) {
                const float mv = sh.u.mg.m[v][n];
                wscale[v] = mv == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mv - mall);
                lsum += wscale[v] * sh.u.mg.l[v][n];
            }
            inv_l = lsum > 0.f ? 1.f / lsum : 0.f;
        } else {
            wscale[0] = 1.f;
            inv_l = ac.l > 0.f ? 1.f / ac.l : 0.f;
        }
        if (crow[c] >= 0) {
            const int64_t orow = (((row_lo + crow[c]) * a.H + h) * a.G + n % a.G) * kHeadDim;
#pragma unroll
            for (int jj = 0; jj < kJPerWave; ++jj) {
                const int jd = W == 1 ? jj : wave * kJPerWave + jj;
                floatx4 o;
                if constexpr (W > 1) {
                    o = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int v = 0; v < W; ++v) o += wscale[v] * sh.u.mg.o[v][jd][lane];
                } else {
                    o = ac.o[jd];
                }
                o *= inv_l;
                const int64_t e = orow + 16 * jd + 4 * g;
                if constexpr (OUT_BF16) {
                    u32x2 pk;
                    pk[0] = bf16_pack(o[0], o[1]);
                    pk[1] = bf16_pack(o[2], o[3]);
                    *(u32x2*)((uint16_t*)a.out + e) = pk;
                } else {
                    *(floatx4*)((float*)a.out + e) = o;
                }
            }
        }
        if constexpr (W > 1) __syncthreads();     // before the next tile reuses the area
    }
}

template <int W, bool OUT_BF16, bool SPLIT>
hipError_t launch_wo(const AttnArgs& a, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.T * a.H * (SPLIT ? a.splits : 1))), block(64 * W);
    if (a.nt)
        hipLaunchKernelGGL((sparse_attn_kernel<W, OUT_BF16, true, SPLIT>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((sparse_attn_kernel<W, OUT_BF16, false, SPLIT>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int W, bool SPLIT = false>
hipError_t launch_w(const AttnArgs& a, hipStream_t stream)
{
    return a.out_bf16 ? launch_wo<W, true, SPLIT>(a, stream) : launch_wo<W, false, SPLIT>(a, stream);
}

template <int W, int CT, bool OUT_BF16>
hipError_t launch_group_wco(const AttnArgs& a, hipStream_t stream)
{
    const int64_t reqs = (a.T + a.rows_per_req - 1) / a.rows_per_req;
    const dim3 grid((unsigned)(reqs * a.groups_per_req * a.H)), block(64 * W);
    if (a.nt)
        hipLaunchKernelGGL((sparse_attn_group_kernel<W, CT, OUT_BF16, true>), grid, block, 0,
                           stream, a);
    else
        hipLaunchKernelGGL((sparse_attn_group_kernel<W, CT, OUT_BF16, false>), grid, block, 0,
                           stream, a);
    return hipGetLastError();
}

template <int W>
hipError_t launch_group_w(const AttnArgs& a, int ct, hipStream_t stream)
{
    if (ct == 1)
        return a.out_bf16 ? launch_group_wco<W, 1, true>(a, stream)
                          : launch_group_wco<W, 1, false>(a, stream);
    return a.out_bf16 ? launch_group_wco<W, 2, true>(a, stream)
                      : launch_group_wco<W, 2, false>(a, stream);
}

}  // namespace

bool attn_group_policy(int64_t T, int H, int G, int q, int* group_rows, int* groups_per_req)
{
    // rows of a request side by side in the MFMA columns: R = 16 / G rows per column
    // tile, at most two tiles and kGroupRows rows per workgroup; taken when the batch
    // gives every compute unit a workgroup (one compute unit streams random pages at
    // about 45 GB/s, so fewer and larger workgroups leave HBM idle: the 64-request
    // spec-decode table runs 52-56 us on the per-row kernel against 69 us grouped, while
    // 128 and 256 such requests run 89 and 175 us grouped against 100 and 196 us)
    if (q <= 1 || G < 1 || G > 16 || H < 1 || T < 1) return false;
    if ((int64_t)H * G * (kHeadDim * 2) * kGroupRows >= ((int64_t)1 << 31)) return false;
    const int R = 16 / G;
    int gr = q < kGroupRows ? q : kGroupRows;
    if (gr > 2 * R) gr = 2 * R;
    const int gpr = (q + gr - 1) / gr;
    const int64_t groups = (T + q - 1) / q * gpr * H;
    if (groups < kGroupMinWorkgroups) return false;
    if (group_rows) *group_rows = gr;
    if (groups_per_req) *groups_per_req = gpr;
    return true;
}

int64_t attn_split_bytes(int64_t pairs, int splits)
{
    const int64_t slots = pairs * splits * kPartSlots;
    if (slots >= ((int64_t)1 << 31)) return -1;
    const int64_t lines = (slots + kPartSlotsPerLine - 1) / kPartSlotsPerLine;
    return (lines > pairs ? lines : pairs) * 256;
}

int attn_split_policy(int64_t T, int H, int splits, int64_t workspace_bytes, int64_t* bytes)
{
    if (splits == 1 || T < 1 || H < 1) return 0;
    const int64_t pairs = T * H;
    int S = splits;
    if (splits == 0) {
        // the library's choice, for batches that leave most compute units without a
        // workgroup. Measured per call, per-row kernel against the split: the
        // spec-decode table's first 16 rows x 2 heads 20.3 against 11.3 us (4 each), its
        // first 48 rows 22.6 against 16.9 us (2; 19.4 with 4), its first 64 rows 23.7
        // against 18.1 us (2); 8 and 32 long-context rows x 4 heads 22.6 against 11.9
        // (4) and 28.3 against 24.3 us (2). From 192 pairs on the per-row kernel alone is
        // faster (its first 96 rows 24.5 against 28.9 us with 2; 512 pairs 54 against
        // 62 us). Three workgroups per pair ran slower than both two and four.
        if (pairs >= kSplitMaxPairs) return 0;
        S = pairs <= kSplitFourPairs ? 4 : 2;
    }
    const int64_t need = attn_split_bytes(pairs, S);
    if (need < 0 || pairs * S >= ((int64_t)1 << 32) || workspace_bytes < need)
        return splits == 0 ? 0 : -1;
    if (bytes) *bytes = need;
    return S;
}

hipError_t launch_sparse_attn_split(const AttnArgs& a, hipStream_t stream)
{
    if (a.splits < 2 || a.splits > kAttnMaxSplits || a.ws == nullptr) return hipErrorInvalidValue;
    switch (a.waves) {
        case 1: return launch_w<1, true>(a, stream);
        case 2: return launch_w<2, true>(a, stream);
        case 4: return launch_w<4, true>(a, stream);
        case 8: return launch_w<8, true>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sparse_attn(const AttnArgs& args, hipStream_t stream)
{
    int gr = 0, gpr = 0;
    if (attn_group_policy(args.T, args.H, args.G, args.rows_per_req, &gr, &gpr)) {
        AttnArgs a = args;
        a.group_rows = gr;
        a.groups_per_req = gpr;
        // pages streamed nontemporally when one workgroup holds all the rows of a
        // request (no other reads them), else cached
        a.nt = gpr == 1;
        const int R = 16 / a.G;
        const int ct = (gr + R - 1) / R;
        switch (a.waves) {
            case 1: return launch_group_w<1>(a, ct, stream);
            case 2: return launch_group_w<2>(a, ct, stream);
            case 4: return launch_group_w<4>(a, ct, stream);
            case 8: return launch_group_w<8>(a, ct, stream);
            default: return hipErrorInvalidValue;
        }
    }
    const AttnArgs& a = args;
    switch (a.waves) {
        case 1: return launch_w<1>(a, stream);
        case 2: return launch_w<2>(a, stream);
        case 4: return launch_w<4>(a, stream);
        case 8: return launch_w<8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvbt
