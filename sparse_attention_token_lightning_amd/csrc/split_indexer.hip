// Lightning Indexer for few query rows over long key caches (decode, a few
// streams each attending to a 256k-token cache): split the keys, stream them
// from HBM once, merge per row. The pages report that single-stream decode
// stayed a wall for their Metal kernels (first page, section details, second
// paragraph) and give no decode design; this one is built for HBM streaming.
//
//  * Grid = (P partitions of 8192 keys) x (rows). Eight wavefronts per
//    workgroup, each scoring 1024 keys in rounds of 64 (two 32-key MFMA
//    blocks whose partial head sums pair up in one v_permlane32_swap).
//  * Keys go HBM -> VGPRs directly as MFMA B operands: the contraction index
//    d is assigned so that lane half h of k-step ks covers dims
//    h*64 + ks*8 .. +7, which makes every lane read 64 contiguous bytes of its
//    key (four 16-byte loads; the two halves of a wave cover each 128-byte fp8
//    row). Queries use the same assignment. E4M3 widens to bf16 in registers.
//    The next round's keys are in flight while the current one is scored.
//  * The partition's exact top-k is found by block-wide radix selection over
//    an order-preserving 32-bit key held in registers (16 per lane). Each
//    digit pass first reduces the AND and OR of the keys still in play and
//    starts its 8-bit window at their highest differing bit, so bits that
//    every live key shares cost nothing and the histogram spreads over
//    bins instead of piling onto one (the candidates of a row are all top
//    scores and share their high bits). The selected keys go, in index
//    order, to the workspace.
//  * The last workgroup of a row to finish (device-scope arrival counter)
//    merges the row's P candidate lists: they are staged through LDS with
//    coalesced loads, each thread keeps a contiguous run in registers, the
//    same selection runs, and one block-wide scan orders the output. The
//    counter is reset for the next call.
#include "device_common.h"
#include "kernels.h"
#include "wave_select.h"

namespace ds4idx {
namespace {

constexpr int H = kMfmaH;
constexpr int D = kMfmaD;
constexpr int NW = 8;
constexpr int THREADS = NW * 64;
constexpr int ROUNDS = 16;
constexpr int WAVE_KEYS = ROUNDS * 64;
constexpr int PART = NW * WAVE_KEYS;  // 8192
constexpr int MREG = 32;              // merge keys held per thread
constexpr int MSTAGE = THREADS * MREG;  // candidates the merge stages in LDS
constexpr int MEXT = 32;              // largest per-partition order statistic kept for the row bound
constexpr int MSURV = 2048;           // survivors of the bound that one wavefront selects from

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

struct SplitSmem {
    union {
        uint32_t sc[NW][WAVE_KEYS];            // partition score keys, 0 = no key
        uint32_t fin[NW][MEXT];                // per-wavefront top-m keys (after sc is read)
        uint32_t stage[MSTAGE + MSTAGE / 32];  // merge staging, one pad word per 32
    };
    int stage_i[MSTAGE + MSTAGE / 32];        // merge staging: key indices
    uint32_t fs[MSURV];                       // merge survivors: keys
    int fe[MSURV];                            // merge survivors: key indices
    uint32_t pt[kSplitMaxParts];              // partitions' m-th largest keys
    uint32_t red[3][NW];
    uint32_t hist[NW][256];
    uint32_t tot[256];
    uint32_t wsum[NW];
    uint32_t pick[2];
    uint32_t pn[kSplitMaxParts];
    int last;
};

template <class V>
__device__ __forceinline__ void store_agent(V *p, V v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class V>
__device__ __forceinline__ V load_agent(const V *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// Block-wide exclusive prefix sum of v; `total` receives the block sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, SplitSmem &sm, uint32_t &total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const uint32_t x = wave_scan_incl(v, 0u, OpAdd{});
    if (lane == 63) sm.wsum[wid] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t c = sm.wsum[w];
        before += (w < wid) ? c : 0u;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

// Block-wide sum, AND and OR.
__device__ __forceinline__ void block_reduce3(uint32_t &s, uint32_t &a, uint32_t &o, SplitSmem &sm)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    s = wave_sum(s);
    a = wave_and(a);
    o = wave_or(o);
    if (lane == 0) {
        sm.red[0][wid] = s;
        sm.red[1][wid] = a;
        sm.red[2][wid] = o;
    }
    __syncthreads();
    s = 0u;
    a = ~0u;
    o = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        s += sm.red[0][w];
        a &= sm.red[1][w];
        o |= sm.red[2][w];
    }
    __syncthreads();
}

// After every thread has added its keys to its wavefront's histogram, find
// the digit of the k-th largest key and how many keys of that digit are
// still wanted (sm.pick).
__device__ __forceinline__ void pick_digit(SplitSmem &sm, uint32_t remaining)
{
    const int tid = threadIdx.x, lane = tid & 63;
    __syncthreads();
    if (tid < 256) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += sm.hist[w][tid];
        sm.tot[tid] = s;
    }
    __syncthreads();
    if (tid < 64) {
        uint32_t c[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) c[q] = sm.tot[4 * lane + q];
        const uint32_t tot = c[0] + c[1] + c[2] + c[3];
        const uint32_t incl = wave_scan_incl(tot, 0u, OpAdd{});
        uint32_t above = wave_total(incl) - incl;
        int found = -1;
        uint32_t rem = 0;
#pragma unroll
        for (int q = 3; q >= 0; --q) {
            if (found < 0 && above < remaining && remaining <= above + c[q]) {
                found = q;
                rem = remaining - above;
            }
            above += c[q];
        }
        const int src = __builtin_ctzll(wave_ballot(found >= 0));
        if (lane == src) {
            sm.pick[0] = (uint32_t)(4 * lane + found);
            sm.pick[1] = rem;
        }
    }
    __syncthreads();
}

// Exact k-th largest key among the keys this block holds (0 = no key; more
// than k keys present). each(f) calls f(key) for every key of the calling
// thread. Returns tau, the k-th largest key, and ties, how many keys equal
// to tau belong to the top k (the lowest-index ones).
template <class Each>
__device__ void block_select(Each each, uint32_t k, SplitSmem &sm, uint32_t &tau, uint32_t &ties)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t prefix = 0, pmask = 0, remaining = k;
    {
        // When at least k scores are >= +0, the k-th largest is too.
        uint32_t nn = 0, a = 0, o = 0;
        each([&](uint32_t u) { nn += u >= 0x80000000u ? 1u : 0u; });
        block_reduce3(nn, a, o, sm);
        if (nn >= k) prefix = pmask = 0x80000000u;
    }
    while (pmask != ~0u) {
        uint32_t n = 0, a = ~0u, o = 0u;
        each([&](uint32_t u) {
            if ((u & pmask) == prefix) {
                a &= u;
                o |= u;
            }
        });
        block_reduce3(n, a, o, sm);
        const uint32_t diff = (a ^ o) & ~pmask;
        if (diff == 0u) {  // every key still in play is equal: that is tau
            prefix = a;
            break;
        }
        const int hb = 31 - __builtin_clz(diff);
        const uint32_t above = hb == 31 ? 0u : (~0u << (hb + 1));
        prefix = (prefix & pmask) | (a & above & ~pmask);
        pmask |= above;
        const int lo = hb >= 7 ? hb - 7 : 0;
        const uint32_t dmask = (2u << (hb - lo)) - 1u;
        for (int b = lane; b < 256; b += 64) sm.hist[wid][b] = 0;
        wave_lds_sync();
        each([&](uint32_t u) {
            if ((u & pmask) == prefix) atomicAdd(&sm.hist[wid][(u >> lo) & dmask], 1u);
        });
        pick_digit(sm, remaining);
        prefix |= sm.pick[0] << lo;
        pmask |= dmask << lo;
        remaining = sm.pick[1];
    }
    tau = prefix;
    ties = remaining;
}

// This lane's half of one key row of a 32-key sub-block (key = base + lane%32,
// dims half*64 .. +63): 64 bytes of E4M3 codes or 128 bytes of bf16; for the
// first sub-block of a pair also the scale of key base + lane.
template <bool KFP8>
struct Raw {
    uint4 v[KFP8 ? 4 : 8];
    float scale;
};

template <bool KFP8, bool SCALE>
__device__ __forceinline__ void load_sub(Raw<KFP8> &r, const uint8_t *Kr, const float *Ksr,
                                         long long kbase, long long L, int lane)
{
    constexpr int NV = KFP8 ? 4 : 8;
    constexpr int ROWB = KFP8 ? D : 2 * D;
    const long long key = kbase + (lane & 31);
    if (key < L) {
        const uint4 *src = reinterpret_cast<const uint4 *>(Kr + key * ROWB + (lane >> 5) * (ROWB / 2));
#pragma unroll
        for (int j = 0; j < NV; ++j) r.v[j] = src[j];
    } else {
#pragma unroll
        for (int j = 0; j < NV; ++j) r.v[j] = make_uint4(0, 0, 0, 0);
    }
    if (KFP8 && SCALE) {
        const long long sk = kbase + lane;
        r.scale = sk < L ? Ksr[sk] : 1.0f;
    }
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

// Partial score of one sub-block: this lane's 16 head rows of each head block.
template <bool KFP8>
__device__ __forceinline__ float score_sub(const Raw<KFP8> &r, const bf16x8 (&a)[2][8],
                                           const float (&wv)[2][16])
{
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 bk = b_operand<KFP8>(r, ks);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
            acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[hb][ks], bk, acc[hb], 0, 0, 0);
    }
    float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            s4[i & 3] = fmaf(wv[hb][i], __builtin_amdgcn_fmed3f(acc[hb][i], 0.0f, 3.0e38f), s4[i & 3]);
    return (s4[0] + s4[1]) + (s4[2] + s4[3]);
}

template <bool KFP8>
__global__ __launch_bounds__(THREADS, 1) void split_indexer_kernel(
    const uint16_t *__restrict__ Q, const uint8_t *__restrict__ K, const float *__restrict__ Ks,
    const float *__restrict__ W, int T, int S, long long offset, int topk, int P,
    uint32_t *__restrict__ ctr, uint32_t *__restrict__ cand_n, uint32_t *__restrict__ cand_t,
    float *__restrict__ cand_s, int *__restrict__ cand_i, int *__restrict__ idx,
    float *__restrict__ vals)
{
    __shared__ SplitSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int p = blockIdx.x;
    const long long r = blockIdx.y;  // b * T + t
    const int b = (int)(r / T), t = (int)(r % T);
    const long long L = offset + t + 1;
    const long long pbase = (long long)p * PART;
    const long long nvalid = L - pbase < 0 ? 0 : (L - pbase > PART ? PART : L - pbase);

    // ---- score this wavefront's 1024 keys into sm.sc
    const long long wbase = pbase + (long long)wid * WAVE_KEYS;
    const long long wkeys = L - wbase < 0 ? 0 : (L - wbase > WAVE_KEYS ? WAVE_KEYS : L - wbase);
    if (wkeys > 0) {
        bf16x8 a[2][8];
        float wv[2][16];
        const int half = lane >> 5;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const bf16x8 *qp = reinterpret_cast<const bf16x8 *>(
                Q + ((r * H + hb * 32 + (lane & 31)) * D + half * 64));
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) a[hb][ks] = qp[ks];
#pragma unroll
            for (int i = 0; i < 16; ++i) wv[hb][i] = W[r * H + hb * 32 + acc_row(i, lane)];
        }
        const uint8_t *Kr = K + (size_t)b * S * (KFP8 ? D : 2 * D);
        const float *Ksr = KFP8 ? Ks + (size_t)b * S : nullptr;
        // Sub-blocks of 32 keys; pairs (2j, 2j+1) share one half swap. A ring
        // of NBUF raw sub-blocks keeps NBUF-1 loads in flight.
        constexpr int NBUF = KFP8 ? 4 : 2;
        const int nsub = (int)((wkeys + 63) / 64) * 2;
        Raw<KFP8> buf[NBUF];
#pragma unroll
        for (int i = 0; i < NBUF - 1; ++i) {
            if (i < nsub) {
                if (i & 1) load_sub<KFP8, false>(buf[i], Kr, Ksr, wbase + 32 * i, L, lane);
                else load_sub<KFP8, true>(buf[i], Kr, Ksr, wbase + 32 * i, L, lane);
            }
        }
        float prev = 0.0f, pscale = 1.0f;
        for (int sb0 = 0; sb0 < nsub; sb0 += NBUF) {
#pragma unroll
            for (int i = 0; i < NBUF; ++i) {
                const int sb = sb0 + i;
                if (sb < nsub) {
                    if (!(i & 1)) pscale = buf[i].scale;
                    const int nx = sb + NBUF - 1;
                    if (nx < nsub) {
                        if ((i + NBUF - 1) & 1)
                            load_sub<KFP8, false>(buf[(i + NBUF - 1) % NBUF], Kr, Ksr, wbase + 32 * nx, L, lane);
                        else
                            load_sub<KFP8, true>(buf[(i + NBUF - 1) % NBUF], Kr, Ksr, wbase + 32 * nx, L, lane);
                    }
                    const float part = score_sub<KFP8>(buf[i], a, wv);
                    if (i & 1) {
                        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(prev),
                                                                         __float_as_uint(part), false, false);
                        float sc = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                        if (KFP8) sc *= pscale;
                        const long long key = wbase + 32 * (sb - 1) + lane;
                        sm.sc[wid][32 * (sb - 1) + lane] = key < L ? ord_key(canon(sc)) : 0u;
                    } else {
                        prev = part;
                    }
                }
            }
        }
    }
    for (int i = (int)(((wkeys + 63) / 64) * 64) + lane; i < WAVE_KEYS; i += 64) sm.sc[wid][i] = 0u;
    wave_lds_sync();
    uint32_t u[ROUNDS];
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j) u[j] = sm.sc[wid][j * 64 + lane];

    // ---- exact top-k of this partition, in index order (wave, round, lane)
    const uint32_t want = (uint32_t)(nvalid < topk ? nvalid : topk);
    const bool select_all = nvalid <= topk;
    uint32_t tau = 0, ties = 0;
    if (!select_all) {
        block_select(
            [&](auto f) {
#pragma unroll
                for (int j = 0; j < ROUNDS; ++j)
                    if (u[j] != 0u) f(u[j]);
            },
            (uint32_t)topk, sm, tau, ties);
    }
    uint32_t neq = 0;
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j)
        neq += (uint32_t)__builtin_popcountll(wave_ballot(!select_all && u[j] != 0u && u[j] == tau));
    uint32_t total;
    uint32_t eq_before = block_excl_scan(lane == 0 ? neq : 0u, sm, total);
    eq_before = (uint32_t)__builtin_amdgcn_readlane((int)eq_before, 0);
    uint32_t keepbits = 0, nkeep = 0;
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j) {
        const bool valid = u[j] != 0u;
        const bool eq = !select_all && valid && u[j] == tau;
        const uint64_t meq = wave_ballot(eq);
        const bool keep = valid && (select_all || u[j] > tau || (eq && eq_before + lanes_below(meq) < ties));
        eq_before += (uint32_t)__builtin_popcountll(meq);
        const uint64_t mk = wave_ballot(keep);
        keepbits |= keep ? (1u << j) : 0u;
        nkeep += (uint32_t)__builtin_popcountll(mk);
    }
    uint32_t out = block_excl_scan(lane == 0 ? nkeep : 0u, sm, total);
    out = (uint32_t)__builtin_amdgcn_readlane((int)out, 0);
    const long long cbase = (r * P + p) * (long long)topk;
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j) {
        const bool keep = (keepbits >> j) & 1u;
        const uint64_t mk = wave_ballot(keep);
        const uint32_t pos = out + lanes_below(mk);
        if (keep && pos < want) {
            store_agent(&cand_s[cbase + pos], key_float(u[j]));
            store_agent(&cand_i[cbase + pos], (int)(pbase + (long long)wid * WAVE_KEYS + j * 64 + lane));
        }
        out += (uint32_t)__builtin_popcountll(mk);
    }
    if (tid == 0) store_agent(&cand_n[r * P + p], want);
    // Unused slots hold the key-0 pattern (all bits set), which reads as "no key".
    for (int i = (int)want + tid; i < topk; i += THREADS) store_agent(&cand_s[cbase + i], __uint_as_float(~0u));

    // ---- this partition's m-th largest key, m = ceil(k / P). With every
    // partition holding m keys at or above its own m-th, the row holds at
    // least P*m >= k keys at or above the smallest of them: a lower bound on
    // the row's k-th key that lets the merge skip most candidates.
    const int mth = (topk + P - 1) / P;
    if (mth <= MEXT) {
        uint32_t top[MEXT];
        wave_mth_key<ROUNDS>(u, mth, lane, top);  // this wavefront's m largest keys
        if (lane == 0)
            for (int i = 0; i < mth; ++i) sm.fin[wid][i] = top[i];
        __syncthreads();
        if (wid == 0) {
            uint32_t fu[(NW * MEXT) / 64];
#pragma unroll
            for (int j = 0; j < (NW * MEXT) / 64; ++j) {
                const int i = j * 64 + lane;
                fu[j] = (i % MEXT) < mth ? sm.fin[i / MEXT][i % MEXT] : 0u;
            }
            const uint32_t tp = wave_mth_key<(NW * MEXT) / 64>(fu, mth, lane, nullptr);
            if (lane == 0) store_agent(&cand_t[r * P + p], tp);  // 0: fewer than m keys, no bound
        }
    } else if (tid == 0) {
        store_agent(&cand_t[r * P + p], 0u);
    }

    // ---- arrival: the last workgroup of the row merges. The candidate lists
    // travel through device-coherent (agent-scope) stores and loads, which
    // bypass the per-XCD L2's non-coherent lines; waiting for every store to
    // complete before the counter increment orders them, with no cache-wide
    // writeback or invalidate.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        sm.last = __hip_atomic_fetch_add(&ctr[r], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (uint32_t)(P - 1);
    __syncthreads();
    if (!sm.last) return;

    const int E = P * topk;  // <= kSplitMaxParts * DS4IDX_MAX_TOPK
    const float *rs = cand_s + r * E;
    const int *ri = cand_i + r * E;
    int *io = idx + r * topk;
    float *vo = vals ? vals + r * topk : nullptr;
    // Element e = (partition, position) in index order; thread t owns the
    // contiguous run [t*chunk, (t+1)*chunk), which keeps the output order.
    const int chunk = (E + THREADS - 1) / THREADS;
    const int e0 = tid * chunk;
    uint32_t m_out = 0;  // selected count (the rest of the row is padding)
    if (chunk <= MREG) {
        // One batch of device-coherent loads, all in flight before any is used:
        // every other workgroup's stores completed before its counter increment.
        // Unused slots carry the no-key pattern, so no per-partition counts.
        float vs[MREG];
        int vi[MREG];
#pragma unroll
        for (int j = 0; j < MREG; ++j) {
            const int e = tid + THREADS * j;
            vs[j] = e < E ? load_agent(&rs[e]) : __uint_as_float(~0u);
            vi[j] = e < E ? load_agent(&ri[e]) : 0;
        }
        const uint32_t ptv = tid < P ? load_agent(&cand_t[r * P + tid]) : ~0u;
        const uint32_t wb = wave_min(ptv);
        if (lane == 0) sm.red[0][wid] = wb;
#pragma unroll
        for (int j = 0; j < MREG; ++j) {
            const int e = tid + THREADS * j;
            if (e < E) {
                sm.stage[e + (e >> 5)] = ord_key(vs[j]);
                sm.stage_i[e + (e >> 5)] = vi[j];
            }
        }
        __syncthreads();
        uint32_t bound = ~0u;  // keys below it cannot be among the row's top k (0: no bound)
#pragma unroll
        for (int w = 0; w < NW; ++w) bound = sm.red[0][w] < bound ? sm.red[0][w] : bound;
        uint32_t mu[MREG];
#pragma unroll
        for (int i = 0; i < MREG; ++i) {
            const int e = e0 + i;
            mu[i] = (i < chunk && e < E) ? sm.stage[e + (e >> 5)] : 0u;
        }
        // Survivors of the bound, kept in (partition, position) = index order.
        uint32_t nsurv = 0;
#pragma unroll
        for (int i = 0; i < MREG; ++i) nsurv += (mu[i] != 0u && mu[i] >= bound) ? 1u : 0u;
        uint32_t F;
        const uint32_t sbase = block_excl_scan(nsurv, sm, F);
        // With a bound, F >= k whenever the row has k keys; without one, F = all keys.
        const uint32_t m = F < (uint32_t)topk ? F : (uint32_t)topk;
        const bool all = F <= (uint32_t)topk;
        m_out = m;
        if (F <= (uint32_t)topk) {
            // Everything that survives is selected (F = min(N, k) here).
            uint32_t pos = sbase;
#pragma unroll
            for (int i = 0; i < MREG; ++i) {
                if (mu[i] != 0u && mu[i] >= bound) {
                    if (pos < m) {
                        io[pos] = sm.stage_i[(e0 + i) + ((e0 + i) >> 5)];
                        if (vo) vo[pos] = key_float(mu[i]);
                    }
                    ++pos;
                }
            }
        } else if (F <= (uint32_t)MSURV) {
            uint32_t pos = sbase;
#pragma unroll
            for (int i = 0; i < MREG; ++i) {
                if (mu[i] != 0u && mu[i] >= bound) {
                    sm.fs[pos] = mu[i];
                    sm.fe[pos] = sm.stage_i[(e0 + i) + ((e0 + i) >> 5)];
                    ++pos;
                }
            }
            __syncthreads();
            if (wid == 0) {  // one wavefront, no block barriers: exact top-k of the survivors
                uint32_t fu[MSURV / 64];
#pragma unroll
                for (int j = 0; j < MSURV / 64; ++j) {
                    const int i = j * 64 + lane;
                    fu[j] = i < (int)F ? sm.fs[i] : 0u;
                }
                uint32_t ties;
                const uint32_t tau = wave_kth_key<MSURV / 64>(fu, (uint32_t)topk, sm.hist[0], lane, ties);
                uint32_t out = 0, tr = 0;
#pragma unroll
                for (int j = 0; j < MSURV / 64; ++j) {
                    const int i = j * 64 + lane;
                    const bool eq = fu[j] != 0u && fu[j] == tau;
                    const uint64_t meq = wave_ballot(eq);
                    const bool keep = fu[j] != 0u && (fu[j] > tau || (eq && tr + lanes_below(meq) < ties));
                    const uint64_t mk = wave_ballot(keep);
                    const uint32_t o = out + lanes_below(mk);
                    if (keep && o < m) {
                        io[o] = sm.fe[i];
                        if (vo) vo[o] = key_float(fu[j]);
                    }
                    out += (uint32_t)__builtin_popcountll(mk);
                    tr += (uint32_t)__builtin_popcountll(meq);
                }
            }
        } else {
            // Too many survivors (adversarial rows): block-wide selection of all.
            uint32_t mtau = 0, mties = 0;
            if (!all) {
                block_select(
                    [&](auto f) {
#pragma unroll
                        for (int i = 0; i < MREG; ++i)
                            if (mu[i] != 0u) f(mu[i]);
                    },
                    (uint32_t)topk, sm, mtau, mties);
            }
            uint32_t my_eq = 0;
#pragma unroll
            for (int i = 0; i < MREG; ++i) my_eq += (!all && mu[i] != 0u && mu[i] == mtau) ? 1u : 0u;
            uint32_t run = block_excl_scan(my_eq, sm, total);
            uint64_t keepmask = 0;
            uint32_t my_keep = 0;
#pragma unroll
            for (int i = 0; i < MREG; ++i) {
                const bool valid = mu[i] != 0u;
                const bool eq = !all && valid && mu[i] == mtau;
                const bool keep = valid && (all || mu[i] > mtau || (eq && run < mties));
                run += eq ? 1u : 0u;
                keepmask |= keep ? (1ull << i) : 0ull;
                my_keep += keep ? 1u : 0u;
            }
            uint32_t pos = block_excl_scan(my_keep, sm, total);
#pragma unroll
            for (int i = 0; i < MREG; ++i) {
                if ((keepmask >> i) & 1ull) {
                    if (pos < m) {
                        io[pos] = sm.stage_i[(e0 + i) + ((e0 + i) >> 5)];
                        if (vo) vo[pos] = key_float(mu[i]);
                    }
                    ++pos;
                }
            }
        }
    } else {
        // Long candidate lists: the same selection, reading the workspace.
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // drop stale L2 lines, then plain loads
        for (int q = tid; q < P; q += THREADS) sm.pn[q] = cand_n[r * P + q];
        __syncthreads();
        uint32_t N = 0;
        for (int q = 0; q < P; ++q) N += sm.pn[q];
        const uint32_t m = N < (uint32_t)topk ? N : (uint32_t)topk;
        const bool all = N <= (uint32_t)topk;
        m_out = m;
        auto valid_at = [&](int e) {
            const int q = e / topk;
            return (uint32_t)(e - q * topk) < sm.pn[q];
        };
        uint32_t mtau = 0, mties = 0;
        if (!all) {
            block_select(
                [&](auto f) {
                    for (int e = tid; e < E; e += THREADS)
                        if (valid_at(e)) f(ord_key(rs[e]));
                },
                (uint32_t)topk, sm, mtau, mties);
        }
        const int e1 = e0 + chunk < E ? e0 + chunk : E;
        uint32_t my_eq = 0;
        for (int e = e0; e < e1; ++e)
            if (valid_at(e)) my_eq += (!all && ord_key(rs[e]) == mtau) ? 1u : 0u;
        const uint32_t eq_base = block_excl_scan(my_eq, sm, total);
        uint32_t my_keep = 0, run = eq_base;
        for (int e = e0; e < e1; ++e) {
            if (!valid_at(e)) continue;
            const uint32_t uu = ord_key(rs[e]);
            const bool eq = !all && uu == mtau;
            my_keep += (all || uu > mtau || (eq && run < mties)) ? 1u : 0u;
            run += eq ? 1u : 0u;
        }
        uint32_t pos = block_excl_scan(my_keep, sm, total);
        run = eq_base;
        for (int e = e0; e < e1; ++e) {
            if (!valid_at(e)) continue;
            const float sv = rs[e];
            const uint32_t uu = ord_key(sv);
            const bool eq = !all && uu == mtau;
            const bool keep = all || uu > mtau || (eq && run < mties);
            run += eq ? 1u : 0u;
            if (keep && pos < m) {
                io[pos] = ri[e];
                if (vo) vo[pos] = sv;
            }
            pos += keep ? 1u : 0u;
        }
    }
    for (int j = (int)m_out + tid; j < topk; j += THREADS) {
        io[j] = -1;
        if (vo) vo[j] = -INFINITY;
    }
    if (tid == 0) ctr[r] = 0u;
}

template <bool KFP8>
hipError_t launch_t(const Problem &p, const void *Q, const void *K, const float *Ks, const float *W,
                    int k, int *idx, float *vals, void *ws, hipStream_t st)
{
    const int rows = p.B * p.T;
    const int P = split_parts(p);
    SplitWorkspace w = split_workspace(ws, p, k);
    hipLaunchKernelGGL((split_indexer_kernel<KFP8>), dim3(P, rows), dim3(THREADS), 0, st,
                       static_cast<const uint16_t *>(Q), static_cast<const uint8_t *>(K), Ks, W,
                       p.T, p.S, p.offset, k, P, w.ctr, w.cand_n, w.cand_t, w.cand_s, w.cand_i, idx, vals);
    return hipGetLastError();
}

}  // namespace

int split_parts(const Problem &p)
{
    const long long maxL = p.offset + p.T;
    return (int)((maxL + PART - 1) / PART);
}

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

size_t split_workspace_bytes(const Problem &p, int k)
{
    const size_t rows = (size_t)p.B * p.T, P = (size_t)split_parts(p);
    return align256(rows * 4) + 2 * align256(rows * P * 4) + 2 * align256(rows * P * (size_t)k * 4);
}

SplitWorkspace split_workspace(void *ws, const Problem &p, int k)
{
    const size_t rows = (size_t)p.B * p.T, P = (size_t)split_parts(p);
    char *c = static_cast<char *>(ws);
    SplitWorkspace w;
    w.ctr = reinterpret_cast<uint32_t *>(c);
    c += align256(rows * 4);
    w.cand_n = reinterpret_cast<uint32_t *>(c);
    c += align256(rows * P * 4);
    w.cand_t = reinterpret_cast<uint32_t *>(c);
    c += align256(rows * P * 4);
    w.cand_s = reinterpret_cast<float *>(c);
    c += align256(rows * P * (size_t)k * 4);
    w.cand_i = reinterpret_cast<int *>(c);
    return w;
}

hipError_t launch_split_select(const Problem &p, const void *Q, const void *K, const float *Ks,
                               const float *W, int k, int *idx, float *vals, void *ws, hipStream_t st)
{
    if (p.k_dtype == FP8) return launch_t<true>(p, Q, K, Ks, W, k, idx, vals, ws, st);
    return launch_t<false>(p, Q, K, Ks, W, k, idx, vals, ws, st);
}

}  // namespace ds4idx
