// Lightning Indexer for few query rows over long key caches (decode, a few
// streams each attending to a 256k-token cache): split the keys, stream them
// from HBM once, merge per row. The pages report that single-stream decode
// stayed a wall for their Metal kernels (first page, section details, second
// paragraph) and give no decode design; this one is built for HBM streaming.
//
//  * Grid = (P partitions of 8192 keys) x (rows). Eight wavefronts per
//    workgroup read the partition in 32 rounds of 256 consecutive keys, 32
//    keys per wavefront per round, the rounds of a full partition rotated by
//    its index so that the blocks of a row read staggered offsets. Pairs of a
//    wavefront's 32-key MFMA blocks combine their partial head sums in one
//    v_permlane32_swap.
//  * Keys go HBM -> VGPRs directly as MFMA B operands: the contraction index
//    d is assigned so that lane half h of k-step ks covers dims
//    h*64 + ks*8 .. +7, which makes every lane read 64 contiguous bytes of its
//    key (four 16-byte loads; the two halves of a wave cover each 128-byte fp8
//    row). Queries use the same assignment. E4M3 widens to bf16 in registers.
//    A ring of sub-blocks keeps three rounds of keys in flight while one is
//    scored (one for bf16 keys); the loop is unrolled and every load is
//    unconditional, so the compiler's wait counts stay exact instead of
//    draining the ring.
//  * The row's query (16 KB) and head weights are staged once in LDS and the
//    MFMA A operands read from there: the 96 registers this frees let the
//    compiler keep the loads in flight (registers, not memory, limited it).
//  * While the keys stream, every score's order key adds one count to a
//    4096-bin LDS histogram of its top 12 bits (sign, exponent, 3 mantissa
//    bits: eight bins per octave). These adds hide under the HBM wait. One
//    block scan of the histogram then gives the bin of the partition's k-th
//    largest key and of its m-th largest (m = ceil(k / full partitions)).
//  * The partition emits, in index order, every key at or above the lower
//    edge of the k-th key's bin: a superset of its top k, usually ~15% more,
//    with no exact selection. Every partition that holds m keys publishes
//    the lower edge of its m-th key's bin; the smallest of these is a lower
//    bound on the row's k-th key, because the full partitions alone hold at
//    least k keys at or above it.
//  * The last workgroup of a row to finish (device-scope arrival counter)
//    loads every candidate slot of the row in one batch, keeps those at or
//    above the bound (index order preserved by a block scan over 64-slot
//    groups) and selects the exact top k among them with block-wide radix
//    passes over 12-bit digits whose window starts at the highest bit in
//    which the live keys differ. The output is one ordered compaction.
#include "device_common.h"
#include "kernels.h"

#include <atomic>
#include <cstdlib>
#include <mutex>

namespace ds4idx {
namespace {

constexpr int H = kMfmaH;
constexpr int D = kMfmaD;
constexpr int NW = 8;
constexpr int THREADS = NW * 64;
constexpr int PL_MAX = 16384;            // longest partition (keys); see kSplitPartLens
constexpr int HBITS = 12;                // histogram digit width
constexpr int HBINS = 1 << HBITS;        // 4096 = 8 bins per thread
constexpr int HSHIFT = 32 - HBITS;       // partition histogram: top 12 key bits
constexpr int NLIST = 64;                // keys of one bin that a single wavefront ranks
constexpr int MSURV = 8192;              // merge survivors held in LDS
constexpr int MREG = MSURV / THREADS;    // survivors per thread
constexpr int GB = 16;                   // 64-slot groups per wavefront per merge batch
constexpr int MAX_SLOTS = 4096;          // full-list slots for k = 2048, the largest k
constexpr int HWORDS = HBINS + HBINS / 8;  // one pad word after every 8 bins
static_assert(HBINS == 8 * THREADS, "each thread owns eight histogram bins");
static_assert(HWORDS >= 2 * 2048, "the histogram words stage k <= 2048 output pairs");

// LDS word of histogram bin b. The scan gives each thread 8 consecutive bins;
// padding puts consecutive threads 9 words apart, so their reads fall in
// different banks (an 8-word stride costs several times the whole scan).
__device__ __forceinline__ int hidx(uint32_t b) { return (int)(b + (b >> 3)); }

// LDS word of the partition's key i: one pad word per 16 keys, so thread t
// reads its 16 consecutive keys at 17t .. 17t+15 without bank conflicts.
__device__ __forceinline__ int scx(int i) { return i + (i >> 4); }

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int QROW = D + 8;  // bf16 per LDS query row: 272 B keeps 16-byte reads conflict-free

// The scoring area of the LDS, for partitions of PART keys: the partition's
// score keys (sc_words words, at scx(i)), then for E4M3 keys each
// wavefront's ring of RING_SLOTS key sub-blocks (32 keys x 128 B, RING16
// 16-byte pieces each) and its two pair-scale slots (64 floats each), or for
// bf16 keys the row's query (H rows of QROW bf16). Two slots, one sub-block
// in flight while the other is scored, streamed the 8 x 262144-key decode as
// fast as three (61.6-64.2 against 63.6-64.3 us per call).
constexpr int RING16 = 256;
constexpr int RING_SLOTS = 2;
__host__ __device__ constexpr int sc_words(int part) { return part + part / 16; }
constexpr int RING_BYTES = NW * RING_SLOTS * RING16 * 16;
constexpr int PSCALE_BYTES = NW * 2 * 64 * 4;
__host__ __device__ constexpr int e4m3_area(int part) { return sc_words(part) * 4 + RING_BYTES + PSCALE_BYTES; }
__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }
constexpr int SCORE_BYTES = imax(imax(e4m3_area(8192), e4m3_area(12288)),
                                 imax(e4m3_area(16384), sc_words(PL_MAX) * 4 + H * QROW * 2));

struct SplitSmem {
    union {
        alignas(16) uint8_t area[SCORE_BYTES];  // scoring (see above)
        struct {
            uint32_t key[MSURV + MSURV / 16];  // merge survivors, index order (direct path: at scx)
            int idx[MSURV];
        } sv;
        struct {
            // partition lists, compacted before coalesced stores; the last 64
            // entries of each are per-lane trash slots (branch-free writes)
            uint64_t full[MAX_SLOTS + 64];
            uint64_t shortl[MAX_SLOTS + 64];
        } st;
        struct {
            // the planned partitioning of a ragged batch (plan_block only)
            long long pk[kSplitPlanRows + 1];  // clamped key prefix sums
            int pq[kSplitPlanRows + 1];        // clamped query prefix sums
            int own[kSplitPlanRows];           // the stream of each query row
        } pl;
    };
    float wl[H];                     // the row's head weights (scoring only)
    alignas(8) uint32_t hist[HWORDS];  // also the merge's output staging (k pairs)
    uint32_t lk[NLIST];              // keys of one bin, for exact ranking
    uint32_t gcnt[NW * GB];          // merge: survivors per 64-slot group
    uint32_t goff[NW * GB];          // merge: output offset per group
    uint32_t wcnt[2][NW];
    uint32_t wsum[NW];
    uint32_t wmax[NW];
    uint32_t red[2][NW];
    uint32_t pick[12];
    uint32_t nl;
    uint32_t pn[kSplitMaxParts];      // merge: full-list length per partition
    int last;
    long long plan_k0, plan_L;        // plan_block's result for this block
    int plan_r, plan_p, plan_n, plan_len, plan_base;
};

// A candidate slot: order key in the low word (0 = empty), key index in the high word.
__device__ __forceinline__ uint64_t slot(uint32_t key, long long index)
{
    return ((uint64_t)(uint32_t)index << 32) | key;
}

// Row (head within the 32-head block) of accumulator element i of a lane in
// a 32 x 32 MFMA result.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// After a barrier that published each wavefront's total in arr[0..NW): the
// sum over wavefronts below the calling one, and (`all`) over all of them.
// Lanes 0..7 scan the eight totals with row shifts; two reads pick the
// results, so no per-wavefront comparison masks stay live in SGPRs.
__device__ __forceinline__ uint32_t waves_before(const uint32_t *arr, uint32_t &all)
{
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t v = lane < NW ? arr[lane] : 0u;
    uint32_t x = v;
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);
    all = (uint32_t)__builtin_amdgcn_readlane((int)x, NW - 1);
    return (uint32_t)__builtin_amdgcn_readlane((int)(x - v), wid);
}

// Block-wide exclusive prefix sum of v; `total` receives the block sum. One
// barrier: sm.wsum must not be written again before the next barrier.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, SplitSmem &sm, uint32_t &total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const uint32_t x = wave_scan_incl(v, 0u, OpAdd{});
    if (lane == 63) sm.wsum[wid] = x;
    __syncthreads();
    const uint32_t before = waves_before(sm.wsum, total);
    return before + x - v;
}

// Block-wide AND and OR. One barrier.
__device__ __forceinline__ void block_and_or(uint32_t &a, uint32_t &o, SplitSmem &sm)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    a = wave_and(a);
    o = wave_or(o);
    if (lane == 0) {
        sm.red[0][wid] = a;
        sm.red[1][wid] = o;
    }
    __syncthreads();
    a = ~0u;
    o = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        a &= sm.red[0][w];
        o |= sm.red[1][w];
    }
}

struct Found {
    uint32_t bin;    // bin holding the target key
    uint32_t above;  // keys in higher bins
    uint32_t cnt;    // keys in the bin
};

// With sm.hist complete (a barrier passed): for each of up to three target
// ranks (1-based from the largest key; 0, or more than the keys counted, =
// no target) the bin holding that key. Thread t owns bins 4095 - 8t - j,
// j = 0..7, so one scan in thread order runs from the top. Returns the
// number of keys counted; with MAX, `bmax` receives the block maximum of
// `mx`. Two barriers.
template <int NT, bool MAX = false>
__device__ __forceinline__ uint32_t hist_find(SplitSmem &sm, const uint32_t (&tgt)[NT], Found (&f)[NT],
                                              uint32_t mx = 0u, uint32_t *bmax = nullptr)
{
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int top = HBINS - 1 - 8 * tid;
    const uint32_t *hb = &sm.hist[hidx((uint32_t)(top - 7))];
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = hb[7 - j];  // descending bins
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += c[j];
    const uint32_t x = wave_scan_incl(s, 0u, OpAdd{});
    if (MAX) mx = wave_max(mx);
    if (lane == 63) {
        sm.wsum[wid] = x;
        if (MAX) sm.wmax[wid] = mx;
    }
    __syncthreads();
    uint32_t total;
    uint32_t run = x - s + waves_before(sm.wsum, total);
    if (MAX) {
        const uint32_t m = lane < NW ? sm.wmax[lane] : 0u;
        *bmax = wave_max(m);
    }
    uint32_t incl[8];
    incl[0] = run + c[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) incl[j] = incl[j - 1] + c[j];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
        const uint32_t t = tgt[q];
        if (t <= total && run < t && t <= incl[7]) {  // one thread per target
            uint32_t j = 0, above = run, cnt = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool before = incl[i] < t;
                j += before ? 1u : 0u;
                above += before ? c[i] : 0u;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) cnt = (uint32_t)i == j ? c[i] : cnt;
            sm.pick[3 * q] = (uint32_t)top - j;
            sm.pick[3 * q + 1] = above;
            sm.pick[3 * q + 2] = cnt;
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NT; ++q) f[q] = Found{sm.pick[3 * q], sm.pick[3 * q + 1], sm.pick[3 * q + 2]};
    return total;
}

// One wavefront: the r-th largest (1-based, r <= n) of the n <= 64 keys in
// sm.lk, and how many of them are strictly larger. Wave-uniform results.
// Lane i counts the keys above and at or above its own, one broadcast key
// per step (n steps; the bins ranked here hold a few keys); key i is the
// r-th largest iff fewer than r keys exceed it and at least r reach it.
// A bit-serial radix over the keys' differing bits took ~1 us for a
// three-key bin, its ~24 ballot steps being one long dependency chain.
__device__ __forceinline__ void list_rank(const SplitSmem &sm, uint32_t n, uint32_t r, uint32_t &kth,
                                          uint32_t &gt_out)
{
    const int lane = threadIdx.x & 63;
    const bool live = lane < (int)n;
    const uint32_t mine = live ? sm.lk[lane] : 0u;
    uint32_t gt = 0, ge = 0;
    for (int j = 0; j < (int)n; ++j) {
        const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mine, j);
        gt += kj > mine ? 1u : 0u;
        ge += kj >= mine ? 1u : 0u;
    }
    const uint64_t m = wave_ballot(live && gt < r && r <= ge);
    const int src = m ? __builtin_ctzll(m) : 0;
    kth = (uint32_t)__builtin_amdgcn_readlane((int)mine, src);
    gt_out = (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
}

// Appends the calling wavefront's keys that satisfy `in` to sm.lk (order
// irrelevant; the caller knows there are at most NLIST of them).
__device__ __forceinline__ void list_append(SplitSmem &sm, bool in, uint32_t key)
{
    const int lane = threadIdx.x & 63;
    const uint64_t m = wave_ballot(in);
    if (m == 0) return;
    const int src = __builtin_ctzll(m);
    uint32_t base = 0;
    if (lane == src) base = atomicAdd(&sm.nl, (uint32_t)__builtin_popcountll(m));
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, src);
    const uint32_t pos = base + lanes_below(m);
    if (in && pos < (uint32_t)NLIST) sm.lk[pos] = key;
}

// Exact k-th largest key among the keys this block holds (0 = no key; more
// than k keys present). each(f) calls f(key) for every nonzero key of the
// calling thread. Returns tau, the k-th largest key, and ties, how many keys
// equal to tau belong to the top k (the lowest-index ones). Each pass takes
// the AND and OR of the keys still in play and histograms the 12 bits below
// their highest differing bit; a bin of at most 64 keys is ranked exactly by
// one wavefront.
template <class Each>
__device__ __forceinline__ void block_kth(Each each, uint32_t k, SplitSmem &sm, uint32_t &tau, uint32_t &ties)
{
    const int tid = threadIdx.x, wid = tid >> 6;
    uint32_t prefix = 0, pmask = 0, remaining = k;
    for (;;) {
        for (int b = tid; b < HWORDS; b += THREADS) sm.hist[b] = 0;
        if (tid == 0) sm.nl = 0;
        uint32_t a = ~0u, o = 0u;
        each([&](uint32_t u) {
            if ((u & pmask) == prefix) {
                a &= u;
                o |= u;
            }
        });
        block_and_or(a, o, sm);
        const uint32_t diff = (a ^ o) & ~pmask;
        if (diff == 0u) {  // every key still in play is equal: that is tau
            tau = a;
            ties = remaining;
            return;
        }
        const int hb = 31 - __builtin_clz(diff);
        const uint32_t above = hb == 31 ? 0u : (~0u << (hb + 1));
        prefix = (prefix & pmask) | (a & above & ~pmask);
        pmask |= above;
        const int lo = hb >= HBITS - 1 ? hb - (HBITS - 1) : 0;
        const uint32_t dmask = (2u << (hb - lo)) - 1u;
        each([&](uint32_t u) {
            if ((u & pmask) == prefix) atomicAdd(&sm.hist[hidx((u >> lo) & dmask)], 1u);
        });
        __syncthreads();
        Found fd[1];
        hist_find<1>(sm, {remaining}, fd);
        const Found f = fd[0];
        remaining -= f.above;
        prefix |= f.bin << lo;
        pmask |= dmask << lo;
        if (pmask == ~0u) {
            tau = prefix;
            ties = remaining;
            return;
        }
        if (f.cnt <= (uint32_t)NLIST) {
            each([&](uint32_t u) { list_append(sm, (u & pmask) == prefix, u); });
            __syncthreads();
            if (wid == 0) {
                uint32_t kth, gt;
                list_rank(sm, f.cnt, remaining, kth, gt);
                if ((threadIdx.x & 63) == 0) {
                    sm.pick[9] = kth;
                    sm.pick[10] = remaining - gt;
                }
            }
            __syncthreads();
            tau = sm.pick[9];
            ties = sm.pick[10];
            return;
        }
    }
}

// One 32-key sub-block of a wavefront in the MFMA layout: lane l holds key
// base + l%32, dims (l/32)*64 .. +63 (64 bytes of E4M3 codes or 128 bytes of
// bf16).
template <bool KFP8>
struct Raw {
    uint4 v[KFP8 ? 4 : 8];
};

// bf16 keys go HBM -> VGPRs in the MFMA layout. Every lane loads, whatever
// its key: keys at or past L read row L - 1 instead (L >= 1 wherever this is
// called), and their scores are dropped when stored. With no branch around
// the loads, every ring slot is filled by the same number of load
// instructions, so the compiler's wait counts before a slot is read stay
// exact instead of draining all loads in flight.
__device__ __forceinline__ void load_sub_bf16(Raw<false> &r, const uint8_t *Kr, long long kbase, long long L,
                                              int lane)
{
    const long long key = kbase + (lane & 31);
    const long long kc = key < L ? key : L - 1;
    const uint4 *src = reinterpret_cast<const uint4 *>(Kr + kc * 2 * D + (lane >> 5) * D);
#pragma unroll
    for (int j = 0; j < 8; ++j) r.v[j] = src[j];
}

// E4M3 keys go HBM -> LDS (global_load_lds_dwordx4) into a ring of 4 KB slots
// per wavefront, coalesced: instruction i moves keys base + 8i .. +7 whole,
// each 8 lanes one 128-byte row. In the MFMA layout, where every instruction
// touches 32 B of each of 32 rows, the same bytes stream ~8% slower. Key n's
// 16-byte piece p sits at slot piece 8n + (p ^ ring_swz(n)), ring_swz(n) =
// (n & 7) ^ ((n >> 3) & 1): lane l of instruction i (key n = 8i + l/8) lands
// at piece 8n + l%8, so it loads piece (l%8) ^ ring_swz(n); the fragment
// reads (one piece of each of 8 keys per 8 lanes) then hit eight distinct
// 16-byte positions mod 128 bytes in every 8 consecutive lanes, and 16
// distinct ones mod 256 bytes in every 16.
__device__ __forceinline__ int ring_swz(int n) { return (n & 7) ^ ((n >> 3) & 1); }

// One 4-byte word per lane straight into LDS (global_load_lds_dword: lane i's
// word lands at lds + 4 i), from a wavefront-uniform base plus a 32-bit
// per-lane byte offset; awaited like gather16_at.
__device__ __forceinline__ void gather4_at(const void *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

// B operand of k-step ks: dims half*64 + ks*8 .. +7 of the lane's half row.
template <bool KFP8>
__device__ __forceinline__ bf16x8 b_operand(const Raw<KFP8> &r, int ks)
{
    if (KFP8) {
        const uint4 &w = r.v[ks >> 1];
        const uint32_t lo = (ks & 1) ? w.z : w.x;
        const uint32_t hi = (ks & 1) ? w.w : w.y;
        const uint4 o = make_uint4(cvt2<false>(lo), cvt2<true>(lo), cvt2<false>(hi), cvt2<true>(hi));
        return __builtin_bit_cast(bf16x8, o);
    } else {
        return __builtin_bit_cast(bf16x8, r.v[ks]);
    }
}

// The head-weighted ReLU sum of one sub-block's two 32-head accumulators:
// this lane's 16 head rows of each head block.
__device__ __forceinline__ float head_sum(const f32x16 (&acc)[2], const float *wl, int lane)
{
    float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            s4[i & 3] = fmaf(wl[hb * 32 + acc_row(i, lane)], __builtin_amdgcn_fmed3f(acc[hb][i], 0.0f, 3.0e38f),
                             s4[i & 3]);
    return (s4[0] + s4[1]) + (s4[2] + s4[3]);
}

// Partial score of one sub-block with the query's A operands read from LDS
// (qa: head lane % 32, dims (lane / 32) * 64, rows QROW apart).
template <bool KFP8>
__device__ __forceinline__ float score_sub(const Raw<KFP8> &r, const uint16_t *qa, const float *wl, int lane)
{
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 bk = b_operand<KFP8>(r, ks);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
            acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                *reinterpret_cast<const bf16x8 *>(qa + hb * 32 * QROW + ks * 8), bk, acc[hb], 0, 0, 0);
    }
    return head_sum(acc, wl, lane);
}

// The same with the A operands in registers: qf[hb][ks] = head hb * 32 +
// lane % 32, dims (lane / 32) * 64 + ks * 8 .. +7.
__device__ __forceinline__ float score_sub_q(const Raw<true> &r, const bf16x8 (&qf)[2][8], const float *wl, int lane)
{
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 bk = b_operand<true>(r, ks);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[hb][ks], bk, acc[hb], 0, 0, 0);
    }
    return head_sum(acc, wl, lane);
}

// Planned partitions for a ragged batch of at most kSplitPlanRows query rows
// (and streams): the keys each row sees are split into n_r equal parts of at
// most T keys, T being the shortest multiple of 512 (at most PL_MAX) for which
// all the parts start in one round on the GPU's CUs; blocks take the parts in
// row order. Every block works the plan out alike from the prefix sums (no
// host synchronisation): rows are found as in wave_row_stream (the first
// stream whose clamped range holds the row), so malformed prefix sums give
// wrong rows but still one owner per row. Returns false for a block past the
// last part. The host launches at least sum_r ceil(L_r / PL_MAX) blocks.
__device__ bool plan_block(SplitSmem &sm, const Ragged &rg, int max_k, int tid, int lane, int wid, long long &r,
                           int &p, long long &L, long long &k0, int &nparts, int &plen, long long &lbase)
{
    const int B = rg.B, TQ = rg.total_q;
    for (int i = tid; i <= B; i += THREADS) {
        const int q = rg.cu_q[i];
        const long long k = rg.cu_k[i];
        sm.pl.pq[i] = q < 0 ? 0 : (q > TQ ? TQ : q);
        sm.pl.pk[i] = k < 0 ? 0 : (k > rg.total_k ? rg.total_k : k);
    }
    for (int i = tid; i < TQ; i += THREADS) sm.pl.own[i] = 0x7fffffff;
    __syncthreads();
    if (tid < B)
        for (int i = sm.pl.pq[tid]; i < sm.pl.pq[tid + 1]; ++i) atomicMin(&sm.pl.own[i], tid);
    __syncthreads();
    if (wid == 0) {
        constexpr int RPL = kSplitPlanRows / 64;  // rows per lane: lane + 64 i
        uint32_t lr[RPL];
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int row = lane + 64 * i;
            lr[i] = 0;
            if (row < TQ && sm.pl.own[row] != 0x7fffffff) {
                const int b = sm.pl.own[row];
                const int tb = sm.pl.pq[b + 1] > sm.pl.pq[b] ? sm.pl.pq[b + 1] - sm.pl.pq[b] : 0;
                const long long sb = sm.pl.pk[b + 1] > sm.pl.pk[b] ? sm.pl.pk[b + 1] - sm.pl.pk[b] : 0;
                const long long l = sb - tb + (row - sm.pl.pq[b]) + 1;
                // at most max_k <= PL_MAX * kSplitMaxParts (the host checks)
                lr[i] = l < 0 ? 0u : (uint32_t)(l < max_k ? l : max_k);
            }
        }
        // parts of row (lane + 64 i) at part length tk: one for a row with no key
        auto parts = [&](int i, uint32_t tk) {
            return lane + 64 * i < TQ ? (lr[i] == 0u ? 1u : (lr[i] + tk - 1u) / tk) : 0u;
        };
        auto total = [&](uint32_t tk) {
            uint32_t s = 0;
#pragma unroll
            for (int i = 0; i < RPL; ++i) s += parts(i, tk);
            return wave_total(wave_scan_incl(s, 0u, OpAdd{}));
        };
        // at most one round of CUs, and never more parts than blocks (at
        // PL_MAX there are at most as many parts as blocks)
        const uint32_t target = gridDim.x < (unsigned)kSplitCUs ? gridDim.x : (uint32_t)kSplitCUs;
        // Lengths are multiples of 512 keys: whole pairs of 256-key rounds,
        // as the scoring loop finishes its sub-blocks in pairs.
        constexpr int NT = PL_MAX / 512;
        int lo = 1, hi = NT;
        if (total(512u * NT) > target) lo = NT;
        while (lo < hi) {
            const int mid = (lo + hi) / 2;
            if (total(512u * (uint32_t)mid) <= target) hi = mid;
            else lo = mid + 1;
        }
        const uint32_t tk = 512u * (uint32_t)lo;
        const uint32_t j = blockIdx.x;
        uint32_t base = 0;
        int found = 0;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const uint32_t n = parts(i, tk);
            const uint32_t incl = wave_scan_incl(n, 0u, OpAdd{});
            const uint32_t first = base + incl - n;
            const uint64_t m = wave_ballot(!found && n > 0u && j >= first && j < first + n);
            if (m && lane == __builtin_ctzll(m)) {
                const int row = lane + 64 * i;
                const uint32_t per = (lr[i] + n - 1u) / n;  // <= tk
                sm.plan_r = row;
                sm.plan_p = (int)(j - first);
                sm.plan_n = (int)n;
                sm.plan_len = (int)((per + 511u) / 512u * 512u);
                sm.plan_base = (int)first;
                sm.plan_L = lr[i];
                sm.plan_k0 = sm.pl.own[row] != 0x7fffffff ? sm.pl.pk[sm.pl.own[row]] : 0;
            }
            found |= m != 0;
            base += wave_total(incl);
        }
        if (lane == 0 && !found) sm.plan_r = -1;
    }
    __syncthreads();
    if (sm.plan_r < 0) return false;
    r = sm.plan_r;
    p = sm.plan_p;
    L = sm.plan_L;
    k0 = sm.plan_k0;
    nparts = sm.plan_n;
    plen = sm.plan_len;
    lbase = sm.plan_base;
    return true;
}

// Ragged batches (VARLEN): row r belongs to the stream of rg whose query
// rows hold it (see StreamGeo); rows of no stream see no keys. Every
// partition of every row still takes part in the arrival, so the counters
// return to zero.
template <bool KFP8, bool VARLEN, int PART, bool PLAN = false>
__global__ __launch_bounds__(THREADS, 1) void split_indexer_kernel(
    const uint16_t *__restrict__ Q, const uint8_t *__restrict__ K, const float *__restrict__ Ks,
    const float *__restrict__ W, int T, int S, long long offset, int topk, int P, int slots, int s1,
    uint32_t *__restrict__ ctr, uint64_t *__restrict__ meta, uint64_t *__restrict__ full_list,
    uint64_t *__restrict__ short_list, int *__restrict__ idx, float *__restrict__ vals, Ragged rg)
{
    __shared__ SplitSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    // Ragged rows differ in length, so their later partitions are often
    // partial or empty. Blocks are taken partition-major there (every row's
    // partition 0, then every row's partition 1, ...): the full partitions
    // dispatch first, spread over the XCDs (consecutive blocks go to
    // consecutive XCDs), and the short ones fill the gaps. Uniform rows keep
    // the plain mapping.
    static_assert(!PLAN || (VARLEN && PART == PL_MAX), "planned parts are a ragged feature");
    int p;
    long long r;  // query row
    long long L, k0;  // keys this row sees; first key row of its stream
    int nparts = P, plen = PART;  // the row's partitions; this partition's length
    long long lbase = 0;          // list index of the row's first partition (planned parts)
    if constexpr (PLAN) {
        if (!plan_block(sm, rg, S, tid, lane, wid, r, p, L, k0, nparts, plen, lbase)) return;
    } else if constexpr (VARLEN) {
        const long long i = blockIdx.x + (long long)P * blockIdx.y;
        p = (int)(i / gridDim.y);
        r = i % gridDim.y;
        const int bs = wave_row_stream(rg.cu_q, rg.cu_k, rg.B, rg.total_q, rg.total_k, r, lane);
        L = 0;
        k0 = 0;
        if (bs >= 0) {
            const StreamGeo g = stream_geo(rg.cu_q, rg.cu_k, bs, rg.total_q, rg.total_k);
            const long long l = g.S - g.T + (r - g.q0) + 1;
            L = l < 0 ? 0 : l;  // l <= g.S always
            k0 = g.k0;
        }
    } else {
        p = blockIdx.x;
        r = blockIdx.y;
        const int b = (int)(r / T), t = (int)(r % T);
        L = offset + t + 1;
        k0 = (long long)b * S;
    }
    static_assert(PART % (NW * 32 * 4) == 0 && PART <= PL_MAX, "whole rounds, whole ring cycles");
    constexpr int NSUB = PART / (NW * 32);  // 32-key sub-blocks per wavefront
    const long long pbase = (long long)p * plen;
    const long long Lend = PLAN ? (L < pbase + plen ? L : pbase + plen) : L;  // this partition's end
    const long long lidx = PLAN ? lbase + p : r * P + p;  // this partition's lists

    // This wavefront's keys: the partition is read in PART / 256 rounds of
    // 256 consecutive keys, the eight wavefronts taking 32 keys each, and a
    // full partition starts its rounds at round p (mod PART / 256). At any
    // moment the blocks of a row then read different offsets of their
    // partitions, instead of all reading at multiples of the partition's
    // bytes apart: a read-only probe of this
    // geometry measured 48.4 against 53.2 us for the 8 x 262144-key decode
    // (and a wavefront owning 128 KB of its partition was as slow as the
    // latter). Sub-block sb of the wavefront covers keys
    // pbase + rot(sb) * 256 + wid * 32 .. +31; pairs (2j, 2j+1) share one half
    // swap. Slots past the wave's last sub-block reload that sub-block
    // (cached) rather than skip the load, so that every iteration issues the
    // same loads and the wait counts stay exact.
    constexpr int RKEYS = NW * 32;           // keys per round
    constexpr int NROUND = NSUB;             // rounds of the longest partition
    const int nround = PLAN ? plen / RKEYS : NROUND;  // rounds of a full partition
    const long long wbase = pbase + (long long)wid * 32;
    const bool full_part = Lend - pbase >= plen;
    const long long wrem = Lend - wbase;
    const int nsub = full_part ? nround
                     : wrem <= 0 ? 0 : (int)(((wrem + RKEYS - 1) / RKEYS + 1) & ~1LL);  // even: whole pairs
    const int rot0 = full_part ? p % nround : 0;
    auto sbase = [&](int sb) {
        const int rr = sb + rot0;
        return wbase + (long long)(rr >= nround ? rr - nround : rr) * RKEYS;
    };
    uint32_t *const sc = reinterpret_cast<uint32_t *>(sm.area);  // score keys at scx(key - pbase)
    // A finished pair: lanes 0..31 hold sub-block sb - 1's scores, lanes
    // 32..63 sub-block sb's; score key, LDS word and histogram count.
    auto store_pair = [&](int sb, float s) {
        const long long key = sbase(lane < 32 ? sb - 1 : sb) + (lane & 31);
        const uint32_t ok = ord_key(canon(s));
        sc[scx((int)(key - pbase))] = key < Lend ? ok : 0u;
        if (key < Lend && ok != 0u) atomicAdd(&sm.hist[hidx(ok >> HSHIFT)], 1u);
    };

    for (int i = tid; i < HWORDS; i += THREADS) sm.hist[i] = 0;
    if (tid == 0) sm.nl = 0;

    if constexpr (KFP8) {
        // ---- E4M3 keys: a ring of NBL 4 KB LDS slots per wavefront (see
        // ring_swz), NBL - 1 sub-blocks in flight while one is scored, and
        // with each even sub-block the scales of its pair (two 128-byte
        // pieces, one global_load_lds_dword) into one of two pair slots, laid
        // out so that lane l reads the scale of the key whose score it
        // finishes. The query's A operands live in registers. Every load in
        // the loop is a gather into LDS awaited with explicit counts.
        // Refilling a slot as soon as its fragments are in registers (with
        // three slots: three sub-blocks in flight during the MFMAs) was
        // slower, 70 against 64 us for the 8 x 262144-key decode: the extra
        // requests in flight served the eight XCDs very unevenly (their
        // blocks finished 45.6 to 55.8 us into the kernel).
        constexpr int NBL = RING_SLOTS;
        static_assert(e4m3_area(PART) <= SCORE_BYTES, "scoring area");
        static_assert(H == 64 && H * D * 2 == 2 * THREADS * 16, "weights: one word per lane; query: two pieces per thread");
        uint8_t *const rbytes = sm.area + sc_words(PART) * 4;
        const uint32_t ring0 = __builtin_amdgcn_readfirstlane(lds_addr(rbytes + wid * NBL * RING16 * 16));
        const float *const pscl = reinterpret_cast<const float *>(rbytes + RING_BYTES) + wid * 128;
        const uint32_t psc0 = __builtin_amdgcn_readfirstlane(lds_addr(pscl));
        const uint8_t *const Kp = uniform_ptr(K + (size_t)(k0 + pbase) * D);  // this partition's first key row
        const float *const Ksp = uniform_ptr(Ks + (size_t)(k0 + pbase));
        // Offsets are relative to pbase; keys at or past L read row L - 1.
        const int lim = (int)(L - 1 - pbase < (long long)PART + RKEYS ? L - 1 - pbase : (long long)PART + RKEYS);
        const uint32_t pc = (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);  // piece of instruction 0; ^16 for odd ones
        auto issue = [&](int t) {  // sub-block t (clamped to the last), and with an even t its pair's scales
            const int kb = (int)(sbase(t < nsub ? t : nsub - 1) - pbase);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kb + 8 * i + (lane >> 3);
                gather16_at(Kp, (uint32_t)(key < lim ? key : lim) * D + (pc ^ (uint32_t)((i & 1) << 4)),
                            ring0 + (uint32_t)((t % NBL) * RING16 * 16 + i * 1024));
            }
            if (!(t & 1)) {
                const int t0 = t < nsub ? t : nsub - 2;
                const int key = (int)(sbase(t0 + (lane >> 5)) - pbase) + (lane & 31);
                gather4_at(Ksp, (uint32_t)(key < lim ? key : lim) * 4, psc0 + (uint32_t)(((t >> 1) & 1) * 256));
            }
        };
        // Loads issued after sub-block sb's keys when it is awaited: its
        // pair's scales if sb is even, and sub-blocks sb + 1 .. sb + NBL - 1.
        static_assert(NBL <= 3, "a pair slot is refilled after the pair's scale is read");
        constexpr int CNT_EVEN = 1 + 4 * (NBL - 1) + (NBL - 1) / 2;
        constexpr int CNT_ODD = 4 * (NBL - 1) + NBL / 2;
        constexpr int CNT_PRO = 4 * (NBL - 1) + NBL / 2;  // the ring's first NBL - 1 sub-blocks

        // Head weights (wavefront 0) and the query (16 KB, into the score
        // area, which is not scored into before every wavefront holds its
        // fragments) first, then the ring's first sub-blocks. Query row h is
        // 16 pieces of 16 B, logical piece j at position j ^ (h % 16).
        if (wid == 0) gather4_at(uniform_ptr(W + r * H), (uint32_t)lane * 4, __builtin_amdgcn_readfirstlane(lds_addr(sm.wl)));
        const uint16_t *const Qr = uniform_ptr(Q + r * H * D);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int pos = j * THREADS + wid * 64 + lane, h = pos >> 4;
            gather16_at(Qr, (uint32_t)(h * 256 + (((lane & 15) ^ (h & 15)) << 4)),
                        __builtin_amdgcn_readfirstlane(lds_addr(sm.area + (j * THREADS + wid * 64) * 16)));
        }
        if (nsub > 0) {
#pragma unroll
            for (int t = 0; t < NBL - 1; ++t) issue(t);
            wait_vm<CNT_PRO>();
        } else {
            wait_vm<0>();
        }
        __syncthreads();
        bf16x8 qf[2][8];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int h = hb * 32 + (lane & 31), j = (lane >> 5) * 8 + ks;
                qf[hb][ks] = *reinterpret_cast<const bf16x8 *>(sm.area + h * 256 + ((j ^ (h & 15)) << 4));
            }
        __syncthreads();

        if (nsub > 0) {
            const int c = lane & 31, h4 = (lane >> 5) << 2;
            int ro[4];  // this lane's fragment pieces within a slot
#pragma unroll
            for (int j = 0; j < 4; ++j) ro[j] = 8 * c + ((h4 + j) ^ ring_swz(c));
            const uint4 *const rs = reinterpret_cast<const uint4 *>(rbytes) + wid * NBL * RING16;
            // Fully unrolled in pairs (nsub is even): slot and wait counts
            // are constants.
#pragma unroll
            for (int sb0 = 0; sb0 < NSUB; sb0 += 2) {
                if (sb0 >= nsub) continue;
                float part[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int sb = sb0 + i;
                    // the slot refilled now was last read one iteration ago
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                    issue(sb + NBL - 1);
                    if (i) wait_vm<CNT_ODD>();
                    else wait_vm<CNT_EVEN>();
                    Raw<true> rw;
#pragma unroll
                    for (int j = 0; j < 4; ++j) rw.v[j] = rs[(sb % NBL) * RING16 + ro[j]];
                    part[i] = score_sub_q(rw, qf, sm.wl, lane);
                }
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]),
                                                                 false, false);
                store_pair(sb0 + 1,
                           (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * pscl[((sb0 >> 1) & 1) * 64 + lane]);
            }
            wait_vm<0>();  // the reloads past the last sub-block: nothing may land in the area later
        }
    } else {
        // ---- bf16 keys: a ring of two sub-blocks in registers, loaded in
        // the MFMA layout before the query staging below, so the key stream
        // starts at once; the query's A operands are read from LDS.
        constexpr int NBUF = 2;
        static_assert(sc_words(PART) * 4 + H * QROW * 2 <= SCORE_BYTES, "scoring area");
        uint16_t *const qs = reinterpret_cast<uint16_t *>(sm.area + sc_words(PART) * 4);
        const uint8_t *Kr = K + (size_t)k0 * 2 * D;
        Raw<false> buf[NBUF];
        if (nsub > 0) load_sub_bf16(buf[0], Kr, sbase(0), L, lane);
        // The row's query (H x D bf16, 16 KB) into LDS: thread t copies two
        // 16-byte pieces, 16 per head row.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int piece = tid + THREADS * j;  // 0 .. H * D / 8 - 1
            const int h = piece >> 4, d8 = piece & 15;
            *reinterpret_cast<uint4 *>(&qs[h * QROW + d8 * 8]) =
                *reinterpret_cast<const uint4 *>(Q + (r * H + h) * D + d8 * 8);
        }
        if (tid < H) sm.wl[tid] = W[r * H + tid];
        __syncthreads();
        if (nsub > 0) {
            // A operands: head hb * 32 + lane % 32, dims (lane / 32) * 64 + ks * 8.
            const uint16_t *qa = &qs[(lane & 31) * QROW + (lane >> 5) * 64];
            float prev = 0.0f;
            for (int sb = 0; sb < nsub; sb += 2) {
                load_sub_bf16(buf[1], Kr, sbase(sb + 1), L, lane);
                prev = score_sub<false>(buf[0], qa, sm.wl, lane);
                load_sub_bf16(buf[0], Kr, sbase(sb + 2 < nsub ? sb + 2 : nsub - 1), L, lane);
                const float part = score_sub<false>(buf[1], qa, sm.wl, lane);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(prev), __float_as_uint(part), false,
                                                                 false);
                store_pair(sb + 1, __uint_as_float(sw[0]) + __uint_as_float(sw[1]));
            }
        }
    }
    // Rounds this wavefront did not score (a partial partition reads its
    // rounds in order, so they are the last ones) hold no key.
    for (int i = nsub + (lane >> 5); i < NROUND; i += 2) sc[scx(i * RKEYS + wid * 32 + (lane & 31))] = 0u;
    __syncthreads();
    // From here on thread t holds the keys of indices pbase + KPT t .. +KPT-1.
    constexpr int KPT = PART / THREADS;  // 16, 24 or 32
    uint32_t u[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) u[j] = sc[scx(KPT * tid + j)];
    const long long ibase = pbase + (long long)KPT * tid;

    // ---- bins of the partition's k-th, m-th and c1-th largest keys. The
    // full partitions of the row (PART keys each) alone hold fullp*m >= k
    // keys. Only nonzero keys are counted: the all-ones NaN pattern maps to
    // key 0, which reads as "no key" everywhere.
    const uint32_t fullp = (uint32_t)(L / plen);
    const uint32_t mth = fullp > 0 ? ((uint32_t)topk + fullp - 1) / fullp : 0u;  // 0: no bound
    // c1 = 4m. With planned parts the lists have room for 2k (the largest
    // m); fixed lengths size them for this m.
    const uint32_t c1 = PLAN && mth > 0 && 4 * mth < (uint32_t)(s1 / 4) ? 4 * mth : (uint32_t)(s1 / 4);
    uint32_t mykmax = 0, kmax;
#pragma unroll
    for (int j = 0; j < KPT; ++j) mykmax = u[j] > mykmax ? u[j] : mykmax;
    Found fd[3];
    const uint32_t nkeys = hist_find<3, true>(sm, {(uint32_t)topk, mth, c1}, fd, mykmax, &kmax);
    const Found fk = fd[0], fm = fd[1], f1 = fd[2];
    const bool has_m = mth > 0 && nkeys >= mth;
    const bool all = nkeys <= (uint32_t)topk;
    // Keys at or above `edge` form the full candidate list: all keys when
    // the partition holds at most k, else everything from the k-th key's bin
    // up. Keys at or above `edge1` (from the c1-th key's bin up) form the
    // short list, which serves the merge whenever edge1 <= the row bound.
    const uint32_t edge = all ? 1u : (fk.bin << HSHIFT);
    const uint32_t F = all ? nkeys : fk.above + fk.cnt;
    const uint32_t edge1 = nkeys < c1 ? 1u : (f1.bin << HSHIFT);
    const uint32_t n1 = nkeys < c1 ? nkeys : f1.above + f1.cnt;
    const bool short_ok = n1 <= (uint32_t)s1;
    const long long cb = lidx * (long long)slots;
    const long long cb1 = lidx * (long long)s1;
    // This partition's bound, published with the short list's edge, the
    // largest key and the full list's length: the lower edge of its m-th
    // key's bin (m keys at or above it; ~0 = no bound from this partition).
    // Ranking that bin's keys for the exact m-th key gave a slightly higher
    // bound, but cost ~1.5 us on the last partition's critical path, while
    // the merge reads every short-list slot whatever the bound.
    const uint32_t nfull = F <= (uint32_t)slots ? F : (uint32_t)topk;
    auto publish_meta = [&]() {
        if (wid != 0) return;
        const uint32_t tp = has_m ? (fm.bin << HSHIFT) : ~0u;
        if (lane == 0) {
            store_agent(&meta[2 * lidx], ((uint64_t)(short_ok ? edge1 : ~0u) << 32) | tp);
            store_agent(&meta[2 * lidx + 1], ((uint64_t)nfull << 32) | kmax);
        }
    };
    const bool direct = F <= (uint32_t)slots;
    // Each thread counts its candidates for both lists; one scan places
    // them, and the lists are compacted in index order
    // in LDS, then written with coalesced stores: the full list when it fits
    // (else below, after an exact selection), the short list with its unused
    // slots empty.
    uint32_t cf = 0, cs = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        cf += u[j] >= edge ? 1u : 0u;
        cs += u[j] >= edge1 ? 1u : 0u;
    }
    uint32_t tf;
    const uint32_t exfs = block_excl_scan(cf | (cs << 16), sm, tf);  // counts < 2^14
    // The counts are exact, so positions stay below F <= slots and n1 <= s1.
    // Every key is written, those not in a list to this lane's trash slot:
    // with no branch per key, the compiler does not move the writes out of
    // line into blocks at the far end of the kernel's code.
    const uint32_t ib = (uint32_t)ibase;
    if (direct) {
        uint32_t pf = exfs & 0xffffu;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool in = u[j] >= edge;
            sm.st.full[in ? pf : (uint32_t)(MAX_SLOTS + lane)] = ((uint64_t)(ib + j) << 32) | u[j];
            pf += in ? 1u : 0u;
        }
    }
    if (short_ok) {
        uint32_t ps = exfs >> 16;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const bool in = u[j] >= edge1;
            sm.st.shortl[in ? ps : (uint32_t)(MAX_SLOTS + lane)] = ((uint64_t)(ib + j) << 32) | u[j];
            ps += in ? 1u : 0u;
        }
    }
    __syncthreads();
    if (direct)
        for (int i = tid; i < (int)F; i += THREADS) store_agent(&full_list[cb + i], sm.st.full[i]);
    if (short_ok)
        for (int i = tid; i < s1; i += THREADS)
            store_agent(&short_list[cb1 + i], i < (int)n1 ? sm.st.shortl[i] : (uint64_t)0);
    publish_meta();
    if (!direct) {
        // Too many keys share the k-th key's bin: exact selection of k.
        uint32_t tau, ties;
        block_kth(
            [&](auto f) {
#pragma unroll
                for (int j = 0; j < KPT; ++j)
                    if (u[j] != 0u) f(u[j]);
            },
            (uint32_t)topk, sm, tau, ties);
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            ngt += u[j] > tau ? 1u : 0u;
            neq += (u[j] != 0u && u[j] == tau) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan(ngt | (neq << 16), sm, tot);  // counts < 2^14
        uint32_t eqb = ex >> 16;
        uint32_t o = (ex & 0xffffu) + (eqb < ties ? eqb : ties);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            bool keep = u[j] > tau;
            if (u[j] != 0u && u[j] == tau) keep = eqb++ < ties;
            if (keep) {
                if (o < (uint32_t)slots) store_agent(&full_list[cb + o], slot(u[j], ibase + j));
                ++o;
            }
        }
    }

    // ---- arrival: the last workgroup of the row merges. The candidate lists
    // travel through device-coherent (agent-scope) stores and loads, which
    // bypass the per-XCD L2's non-coherent lines; waiting for every store to
    // complete before the counter increment orders them, with no cache-wide
    // writeback or invalidate.
    for (int i = tid; i < HWORDS; i += THREADS) sm.hist[i] = 0;  // for the merge
    if (tid == 0) sm.nl = 0;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        sm.last = __hip_atomic_fetch_add(&ctr[r], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (uint32_t)(nparts - 1);
    __syncthreads();
    if (!sm.last) return;

    int *io = idx + r * topk;
    float *vo = vals ? vals + r * topk : nullptr;
    const long long lrow = PLAN ? lbase : r * P;  // list index of the row's first partition
    const uint64_t *rs = short_list + lrow * s1;
    const uint64_t *rf = full_list + lrow * slots;
    const int G1 = nparts * (s1 / 64), GF = nparts * (slots / 64);

    // Survivors of the bound from a slot grid (every partition's list padded
    // to `per` slots with empty ones) in slot = index order: 64-slot group g,
    // wavefront w takes groups w + 8i. Returns false when they exceed MSURV.
    uint32_t Fs = 0;
    auto collect_batch = [&](const uint64_t (&v)[GB], uint32_t bound) {
        uint32_t mycnt = 0;
#pragma unroll
        for (int i = 0; i < GB; ++i) {
            const uint32_t key = (uint32_t)v[i];
            const uint32_t c = (uint32_t)__builtin_popcountll(wave_ballot(key != 0u && key >= bound));
            mycnt = lane == i ? c : mycnt;
        }
        if (lane < GB) sm.gcnt[wid + NW * lane] = mycnt;
        __syncthreads();
        uint32_t tot;
        const uint32_t ex = block_excl_scan(tid < NW * GB ? sm.gcnt[tid] : 0u, sm, tot);
        if (tid < NW * GB) sm.goff[tid] = Fs + ex;
        __syncthreads();
        if (Fs + tot > (uint32_t)MSURV) return false;
#pragma unroll
        for (int i = 0; i < GB; ++i) {
            const uint32_t key = (uint32_t)v[i];
            const bool keep = key != 0u && key >= bound;
            const uint64_t mk = wave_ballot(keep);
            if (mk != 0) {
                const uint32_t pos = sm.goff[wid + NW * i] + lanes_below(mk);
                if (keep) {
                    sm.sv.key[pos] = key;
                    sm.sv.idx[pos] = (int)(v[i] >> 32);
                }
            }
        }
        Fs += tot;
        return true;
    };
    auto load_batch = [&](uint64_t (&v)[GB], const uint64_t *grid, int G, int g0) {
#pragma unroll
        for (int i = 0; i < GB; ++i) {
            const int g = g0 + wid + NW * i;
            v[i] = g < G ? load_agent(&grid[(long long)g * 64 + lane]) : (uint64_t)0;
        }
    };
    // The full lists: slot j of partition q holds a key only for j < sm.pn[q].
    const int gpp = slots / 64;
    auto load_full_batch = [&](uint64_t (&v)[GB], int g0) {
#pragma unroll
        for (int i = 0; i < GB; ++i) {
            const int g = g0 + wid + NW * i;
            const bool in = g < GF && (g % gpp) * 64 + lane < (int)sm.pn[g < GF ? g / gpp : 0];
            v[i] = in ? load_agent(&rf[(long long)g * 64 + lane]) : (uint64_t)0;
        }
    };
    auto collect_short = [&](uint32_t bnd) {
        for (int g0 = 0; g0 < G1; g0 += NW * GB) {
            uint64_t v[GB];
            load_batch(v, rs, G1, g0);
            if (!collect_batch(v, bnd)) return false;
        }
        return true;
    };
    auto collect_full = [&](uint32_t bnd) {
        for (int g0 = 0; g0 < GF; g0 += NW * GB) {
            uint64_t v[GB];
            load_full_batch(v, g0);
            if (!collect_batch(v, bnd)) return false;
        }
        return true;
    };

    // The first batch of short lists is in flight with the partitions'
    // bounds. Row bound: the smallest published m-th key; the short lists
    // serve when every partition's short-list edge is at or below it.
    uint64_t v0[GB];
    load_batch(v0, rs, G1, 0);
    uint32_t tq = ~0u, eq1 = 0u, mq = 0u;
    for (int q = lane; q < nparts; q += 64) {
        const uint64_t a = load_agent(&meta[2 * (lrow + q)]);
        const uint64_t b = load_agent(&meta[2 * (lrow + q) + 1]);
        const uint32_t t = (uint32_t)a, e1 = (uint32_t)(a >> 32), km = (uint32_t)b;
        tq = t < tq ? t : tq;
        eq1 = e1 > eq1 ? e1 : eq1;
        mq = km > mq ? km : mq;
        if (wid == 0) sm.pn[q] = (uint32_t)(b >> 32);  // full-list lengths, for the other paths
    }
    uint32_t bound = wave_min(tq);
    if (bound == ~0u) bound = 0u;
    const uint32_t kmax_row = wave_max(mq);
    const bool use_short = bound != 0u && wave_max(eq1) <= bound;

    uint32_t m_out;
    if (use_short && G1 <= NW * GB) {
        // Select straight from the loaded short lists, in the order they
        // were loaded: thread t holds slots 512 i + t (i < GB), so chunk
        // (i, wavefront) holds slots 512 i + 64 w .. +63, and chunks taken in
        // (i, w) order run through the slots in index order. Every key in play
        // lies in [bound, row maximum], so they share the bits above the
        // highest bit in which those two differ: the 12 bits below it are the
        // first digit, with no reduction pass.
        const int hb = 31 - __builtin_clz((bound ^ kmax_row) | 1u);
        const int lo = hb >= HBITS - 1 ? hb - (HBITS - 1) : 0;
        const uint32_t dmask = (2u << (hb - lo)) - 1u;
        const uint32_t prefix = hb == 31 ? 0u : (bound & (~0u << (hb + 1)));
        uint32_t kk[GB];  // slots past the lists were loaded as 0 (no key)
#pragma unroll
        for (int i = 0; i < GB; ++i) {
            const uint32_t key = (uint32_t)v0[i];
            kk[i] = key >= bound ? key : 0u;
            if (kk[i] != 0u) atomicAdd(&sm.hist[hidx((kk[i] >> lo) & dmask)], 1u);
        }
        __syncthreads();
        Found fd[1];
        const uint32_t total = hist_find<1>(sm, {(uint32_t)topk}, fd);
        uint32_t tau = 0, ties = 0;  // at most k keys in play: all are kept
        if (total > (uint32_t)topk) {
            const Found f = fd[0];
            const uint32_t rem = (uint32_t)topk - f.above;
            if (lo == 0) {
                tau = prefix | f.bin;
                ties = rem;
            } else if (f.cnt <= (uint32_t)NLIST) {
                uint32_t cm = 0;
#pragma unroll
                for (int i = 0; i < GB; ++i) cm += (kk[i] != 0u && ((kk[i] >> lo) & dmask) == f.bin) ? 1u : 0u;
                if (cm != 0u) {
                    uint32_t pm = atomicAdd(&sm.nl, cm);
#pragma unroll
                    for (int i = 0; i < GB; ++i)
                        if (kk[i] != 0u && ((kk[i] >> lo) & dmask) == f.bin) sm.lk[pm++] = kk[i];
                }
                __syncthreads();
                if (wid == 0) {
                    uint32_t kth, gt;
                    list_rank(sm, f.cnt, rem, kth, gt);
                    if (lane == 0) {
                        sm.pick[9] = kth;
                        sm.pick[10] = rem - gt;
                    }
                }
                __syncthreads();
                tau = sm.pick[9];
                ties = sm.pick[10];
            } else {
                block_kth(
                    [&](auto fn) {
#pragma unroll
                        for (int i = 0; i < GB; ++i)
                            if (kk[i] != 0u) fn(kk[i]);
                    },
                    (uint32_t)topk, sm, tau, ties);
            }
        }
        // Ordered output. Each chunk counts its keys above tau and equal to
        // it (ballots); every wavefront scans the 128 chunk counts itself, so
        // one barrier serves. A key's place is the keys above tau before it
        // plus the ties before it, capped at the ties kept (the lowest
        // indices); the stores come straight from the loaded lists.
        uint32_t mycnt = 0;
#pragma unroll
        for (int i = 0; i < GB; ++i) {
            const uint32_t ng = (uint32_t)__builtin_popcountll(wave_ballot(kk[i] > tau));
            const uint32_t ne = (uint32_t)__builtin_popcountll(wave_ballot(kk[i] != 0u && kk[i] == tau));
            mycnt = lane == i ? ng | (ne << 16) : mycnt;  // counts <= 64
        }
        if (lane < GB) sm.gcnt[NW * lane + wid] = mycnt;
        __syncthreads();
        // lane l: chunks 2l and 2l + 1, i.e. (i, w) = (l / 4, 2 (l % 4)) and the next
        const uint32_t c0 = sm.gcnt[2 * lane], c1 = sm.gcnt[2 * lane + 1];
        const uint32_t inc = wave_scan_incl(c0 + c1, 0u, OpAdd{});  // packed: each half < 2^14
        const uint32_t ex0 = inc - c0 - c1, ex1 = inc - c1;
#pragma unroll
        for (int i = 0; i < GB; ++i) {
            const int e = NW * i + wid;  // this wavefront's chunk of slot row i
            const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)((e & 1) ? ex1 : ex0), e >> 1);
            const bool gt = kk[i] > tau, eq = kk[i] != 0u && kk[i] == tau;
            const uint32_t gb = (base & 0xffffu) + lanes_below(wave_ballot(gt));
            const uint32_t eb = (base >> 16) + lanes_below(wave_ballot(eq));
            if (gt || (eq && eb < ties)) {
                const uint32_t pos = gb + (eb < ties ? eb : ties);
                io[pos] = (int)(v0[i] >> 32);
                if (vo) vo[pos] = key_float(kk[i]);
            }
        }
        m_out = total < (uint32_t)topk ? total : (uint32_t)topk;
    } else {
        __syncthreads();  // sm.pn
        const bool ok = use_short ? collect_short(bound) : collect_full(bound);
        __syncthreads();
        if (ok) {
            // Thread t owns the contiguous run [t*ch, t*ch + ch) of survivors.
            const int ch = (int)((Fs + THREADS - 1) / THREADS);
            const int e0 = tid * ch;
            uint32_t su[MREG];
    #pragma unroll
            for (int i = 0; i < MREG; ++i) {
                const int e = e0 + i;
                su[i] = (i < ch && e < (int)Fs) ? sm.sv.key[e] : 0u;
            }
            uint32_t tau = 0, ties = 0;  // with at most k survivors every one is kept
            if (Fs > (uint32_t)topk) {
                block_kth(
                    [&](auto f) {
    #pragma unroll
                        for (int i = 0; i < MREG; ++i)
                            if (su[i] != 0u) f(su[i]);
                    },
                    (uint32_t)topk, sm, tau, ties);
            }
            uint32_t ngt = 0, neq = 0;
    #pragma unroll
            for (int i = 0; i < MREG; ++i) {
                ngt += su[i] > tau ? 1u : 0u;
                neq += (su[i] != 0u && su[i] == tau) ? 1u : 0u;
            }
            uint32_t tot;
            const uint32_t ex = block_excl_scan(ngt | (neq << 16), sm, tot);  // counts < 2^14
            uint32_t eqb = ex >> 16;
            uint32_t pos = (ex & 0xffffu) + (eqb < ties ? eqb : ties);
    #pragma unroll
            for (int i = 0; i < MREG; ++i) {
                bool keep = su[i] > tau;
                if (su[i] != 0u && su[i] == tau) keep = eqb++ < ties;
                if (keep && pos < (uint32_t)topk) {
                    io[pos] = sm.sv.idx[e0 + i];
                    if (vo) vo[pos] = key_float(su[i]);
                    ++pos;
                }
            }
            m_out = Fs < (uint32_t)topk ? Fs : (uint32_t)topk;
        } else {
            // The bound left too many survivors (many equal scores): the same
            // selection over every full-list slot, read from the workspace.
            const int E = nparts * slots;
            auto valid = [&](int e) { return (uint32_t)(e % slots) < sm.pn[e / slots]; };
            auto each = [&](auto f) {
                for (int e = tid; e < E; e += THREADS) {
                    const uint32_t key = valid(e) ? (uint32_t)load_agent(&rf[e]) : 0u;
                    if (key != 0u) f(key);
                }
            };
            uint32_t n = 0;
            each([&](uint32_t) { ++n; });
            uint32_t N;
            block_excl_scan(n, sm, N);
            __syncthreads();
            uint32_t tau = 0, ties = 0;
            if (N > (uint32_t)topk) block_kth(each, (uint32_t)topk, sm, tau, ties);
            const int ch = (E + THREADS - 1) / THREADS;
            const int e0 = tid * ch, e1 = e0 + ch < E ? e0 + ch : E;
            uint32_t ngt = 0, neq = 0;
            for (int e = e0; e < e1; ++e) {
                const uint32_t key = valid(e) ? (uint32_t)load_agent(&rf[e]) : 0u;
                ngt += key > tau ? 1u : 0u;
                neq += (key != 0u && key == tau) ? 1u : 0u;
            }
            uint32_t tot;
            const uint32_t gtb = block_excl_scan(ngt, sm, tot);
            __syncthreads();
            uint32_t eqb = block_excl_scan(neq, sm, tot);
            uint32_t pos = gtb + (eqb < ties ? eqb : ties);
            for (int e = e0; e < e1; ++e) {
                const uint64_t sv = valid(e) ? load_agent(&rf[e]) : (uint64_t)0;
                const uint32_t key = (uint32_t)sv;
                bool keep = key > tau;
                if (key != 0u && key == tau) keep = eqb++ < ties;
                if (keep && pos < (uint32_t)topk) {
                    io[pos] = (int)(sv >> 32);
                    if (vo) vo[pos] = key_float(key);
                    ++pos;
                }
            }
            m_out = N < (uint32_t)topk ? N : (uint32_t)topk;
        }
    }
    for (int j = (int)m_out + tid; j < topk; j += THREADS) {
        io[j] = -1;
        if (vo) vo[j] = -INFINITY;
    }
    if (tid == 0) ctr[r] = 0u;
}

template <bool KFP8, bool VARLEN>
hipError_t launch_t(const Problem &p, const SplitShape &sh, const Ragged &rg, const void *Q, const void *K,
                    const float *Ks, const float *W, int k, int *idx, float *vals, void *ws, hipStream_t st)
{
    const int P = split_parts(sh);
    SplitWorkspace w = split_workspace(ws, sh, k);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(P, (unsigned)sh.rows), dim3(THREADS), 0, st,
                           static_cast<const uint16_t *>(Q), static_cast<const uint8_t *>(K), Ks, W, p.T, p.S,
                           p.offset, k, P, split_slots(k), split_short_slots(sh, k), w.ctr, w.meta, w.full_list,
                           w.short_list, idx, vals, rg);
    };
    if constexpr (VARLEN) {
        if (sh.plan) {
            // One block per planned part; S carries the most keys a row may see.
            hipLaunchKernelGGL((split_indexer_kernel<KFP8, true, PL_MAX, true>), dim3(sh.plan), dim3(THREADS), 0,
                               st, static_cast<const uint16_t *>(Q), static_cast<const uint8_t *>(K), Ks, W, 0,
                               (int)sh.max_len, 0LL, k, sh.plan, split_slots(k), split_short_slots(sh, k), w.ctr,
                               w.meta, w.full_list, w.short_list, idx, vals, rg);
            return hipGetLastError();
        }
    }
    if (sh.part == kSplitPartLens[2]) go(split_indexer_kernel<KFP8, VARLEN, kSplitPartLens[2]>);
    else if (sh.part == kSplitPartLens[1]) go(split_indexer_kernel<KFP8, VARLEN, kSplitPartLens[1]>);
    else go(split_indexer_kernel<KFP8, VARLEN, kSplitPartLens[0]>);
    return hipGetLastError();
}

std::atomic<int> g_split_len{-1};  // -1: not read from the environment yet; 0: automatic

bool supported_len(int len)
{
    for (int l : kSplitPartLens)
        if (len == l) return true;
    return false;
}

int split_len_now()
{
    int v = g_split_len.load(std::memory_order_relaxed);
    if (v >= 0) return v;
    int init = 0;
    if (const char *e = std::getenv("DS4IDX_SPLIT")) {
        const int x = std::atoi(e);
        if (supported_len(x)) init = x;
    }
    int expected = -1;
    g_split_len.compare_exchange_strong(expected, init);
    return g_split_len.load(std::memory_order_relaxed);
}

// Partition length: the override if set, else the shortest length whose
// partitions (`blocks(len)`, at most) all start in one round on the GPU's
// compute units, else the shortest. One workgroup runs per CU, so a batch
// that needs a second round of partitions pays for a whole second round.
template <class Blocks>
int pick_part(Blocks blocks)
{
    const int o = split_len_now();
    if (o) return o;
    for (int l : kSplitPartLens)
        if (blocks((long long)l) <= kSplitCUs) return l;
    return kSplitPartLens[0];
}

}  // namespace

int set_split_len(int len)
{
    if (len != 0 && !supported_len(len)) return -1;
    const int prev = split_len_now();
    g_split_len.store(len, std::memory_order_relaxed);
    return prev;
}

int get_split_len() { return split_len_now(); }

SplitShape split_shape(const Problem &p)
{
    const long long rows = (long long)p.B * p.T, max_len = p.offset + p.T;
    const int part = pick_part([&](long long l) { return rows * ((max_len + l - 1) / l); });
    return SplitShape{rows, max_len, p.offset + 1, part};
}

SplitShape split_shape(const VarlenProblem &p)
{
    // The stream lengths are on the device. With one query per stream the
    // nonempty partitions number at most total_k / len + B, exactly
    // B ceil(max_k / len) when every stream holds max_k keys; with several
    // queries per stream there is no such bound here.
    if (split_len_now() == 0 && p.total_q >= 1 && p.total_q <= kSplitPlanRows && p.B <= kSplitPlanRows &&
        p.max_k <= (long long)PL_MAX * kSplitMaxParts) {
        // Planned parts. A row seeing L <= max_k keys takes at most
        // ceil(L / PL_MAX) parts in any plan, so this many blocks suffice;
        // at least one per CU, so that short rows spread over all of them.
        const long long need = p.total_q * ((p.max_k + PL_MAX - 1) / PL_MAX);
        const long long blocks = need > kSplitCUs ? need : kSplitCUs;
        return SplitShape{p.total_q, p.max_k, p.max_k, PL_MAX, (int)blocks};
    }
    const int part = pick_part([&](long long l) {
        if (p.total_q != p.B) return (long long)p.total_q * ((p.max_k + l - 1) / l);
        if (p.total_k == (long long)p.B * p.max_k) return (long long)p.B * ((p.max_k + l - 1) / l);
        return (p.total_k + l - 1) / l + p.B;
    });
    return SplitShape{p.total_q, p.max_k, p.max_k, part};
}

int split_parts(const SplitShape &sh) { return (int)((sh.max_len + sh.part - 1) / sh.part); }

int split_slots(int k) { return (2 * k + 63) / 64 * 64; }

int split_short_slots(const SplitShape &sh, int k)
{
    if (sh.plan) return split_slots(k);  // the kernel takes c1 = 4m per row, m up to k
    // Room for the keys from the bin of the c1-th largest up, c1 = 4m (m =
    // ceil(k / full partitions) of the row with the fewest): the kernel takes
    // c1 = slots / 4, so the bin may hold up to 3 c1 further keys.
    const long long fullp = sh.short_len / sh.part;
    if (fullp < 1) return 64;
    const long long m = (k + fullp - 1) / fullp;
    const long long s = (16 * m + 63) / 64 * 64;
    return (int)(s < split_slots(k) ? s : split_slots(k));
}

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Candidate lists: one per partition of every row, or per planned block.
static size_t split_lists(const SplitShape &sh)
{
    return sh.plan ? (size_t)sh.plan : (size_t)sh.rows * (size_t)split_parts(sh);
}

size_t split_workspace_bytes(const SplitShape &sh, int k)
{
    const size_t rows = (size_t)sh.rows, n = split_lists(sh);
    return align256(rows * 4) + align256(n * 16) + align256(n * (size_t)split_slots(k) * 8) +
           align256(n * (size_t)split_short_slots(sh, k) * 8);
}

SplitWorkspace split_workspace(void *ws, const SplitShape &sh, int k)
{
    const size_t rows = (size_t)sh.rows, n = split_lists(sh);
    char *c = static_cast<char *>(ws);
    SplitWorkspace w;
    w.ctr = reinterpret_cast<uint32_t *>(c);
    c += align256(rows * 4);
    w.meta = reinterpret_cast<uint64_t *>(c);
    c += align256(n * 16);
    w.full_list = reinterpret_cast<uint64_t *>(c);
    c += align256(n * (size_t)split_slots(k) * 8);
    w.short_list = reinterpret_cast<uint64_t *>(c);
    return w;
}

hipError_t launch_split_select(const Problem &p, const void *Q, const void *K, const float *Ks,
                               const float *W, int k, int *idx, float *vals, void *ws, hipStream_t st)
{
    const SplitShape sh = split_shape(p);
    if (p.k_dtype == FP8) return launch_t<true, false>(p, sh, Ragged{}, Q, K, Ks, W, k, idx, vals, ws, st);
    return launch_t<false, false>(p, sh, Ragged{}, Q, K, Ks, W, k, idx, vals, ws, st);
}

// ---- the allocation-free entry point's scratch memory
//
// One fixed array per GPU, in the code object's device memory, so that the
// allocation-free select needs no workspace from its caller. Host code never
// uses the array's name as an address (on the host it is only a stand-in):
// the device address comes from hipGetSymbolAddress, once per device with
// that device current, and is kept per device.
namespace {

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *__restrict__ p, long long n)
{
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

}  // namespace

void *noalloc_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

// Zero n words on the stream with a fill kernel (no memset node, so the call
// can be captured into a graph and replayed).
hipError_t launch_zero_words(uint32_t *p, long long n, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    const long long blocks = (n + 255) / 256;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_split_select_varlen(const VarlenProblem &p, const int *cu_q, const long long *cu_k,
                                      const void *Q, const void *K, const float *Ks, const float *W, int k,
                                      int *idx, float *vals, void *ws, hipStream_t st)
{
    const SplitShape sh = split_shape(p);
    const Ragged rg{cu_q, cu_k, p.B, p.total_q, p.total_k};
    const Problem none{};
    if (p.k_dtype == FP8) return launch_t<true, true>(none, sh, rg, Q, K, Ks, W, k, idx, vals, ws, st);
    return launch_t<false, true>(none, sh, rg, Q, K, Ks, W, k, idx, vals, ws, st);
}

}  // namespace ds4idx
