// Lightning Indexer scorer + streaming top-k on gfx950 matrix cores.
//
// The pages' Metal kernels (a threadgroup-tiled scorer, a register-blocked
// K-resident scorer and a streaming top-512 that replaced a bitonic sort and
// merge cascade; first page, section details, first and second paragraphs)
// are prior art for a different GPU. This kernel is laid out for CDNA4:
//
//  * Work split. A 512-thread workgroup owns 8 consecutive query tokens of one
//    batch row; each of its eight wavefronts owns one token and keeps its
//    query (64 heads x 128 dims, bf16) resident in VGPRs as MFMA A operands
//    for the whole key loop. Two wavefronts share each SIMD, so one's LDS
//    waits and epilogue overlap the other's matrix work.
//  * Keys. Tiles of 128 keys are staged global -> registers -> LDS, double
//    buffered, once per workgroup. E4M3 codes are widened to bf16 on the way
//    into LDS (exact: every E4M3 value is a bf16 value). A key row is 256 B
//    with its 16-byte pieces permuted by the row (piece p of row r at
//    p ^ (r & 15)), so the 16 rows one fragment read touches spread over all
//    the banks; rows padded to 272 B instead conflicted on this part (19% of
//    CU cycles in bank-conflict stalls, 4% swizzled). The per-token fp32
//    scale is kept aside and applied once to the head-reduced score (allowed
//    since the scale is positive, so it commutes with the ReLU).
//  * Contraction. v_mfma_f32_16x16x32_bf16 with heads on M (four 16-head
//    tiles) and keys on N, fp32 accumulation. A 64-key pair is two 32-key
//    halves of 2 key tiles x 4 head tiles: each of the 4 k-steps over
//    D = 128 issues a half's 8 independent MFMAs on two B fragments read
//    once from LDS, interleaved one MFMA to two VALU instructions with the
//    reduction of the other half, at raised wavefront priority. The
//    wavefront keeps its own matrix work going first, and the other
//    wavefront of the SIMD fills the gaps (with two 32x32 tiles per head
//    block the epilogue did not overlap and cost a fifth of the time).
//  * Epilogue in registers. Each lane holds 4 heads of each of 4 head tiles
//    for 4 keys: ReLU (one v_med3), times w[t,h] (fp32), summed in-lane.
//    v_permlane32_swap and v_permlane16_swap then add the other three lane
//    groups' heads so that lane l holds the score of key l of the pair. The
//    causal mask (key <= offset + t) is applied per lane.
//  * Streaming top-k per token. A candidate buffer of CAP (score, index)
//    slots per token lives in LDS. A score enters only if it reaches the
//    token's running threshold (ballot + mbcnt place it in ascending key
//    order). At a tile's end, when some token's buffer is nearly full, every
//    wavefront whose buffer holds more than RAISE_LO entries raises its
//    threshold, all in the same tile, so the workgroup stalls at one barrier
//    for all of them: to the highest 8-bit histogram edge that keeps k
//    entries at or above it, compacting the buffer stably; nothing that can
//    still reach the top k is dropped. If that frees too little, the exact k-th
//    key is found by radix selection and the buffer cut to exactly k
//    entries; later keys, all with higher indices, must then beat it
//    strictly, so equal scores keep going to the lower index. At the end the
//    exact selection runs once more and the buffer, already in index order,
//    is the output. No sort anywhere.
#include "device_common.h"
#include "kernels.h"
#include "wave_select.h"

#include <atomic>
#include <cstdlib>

namespace ds4idx {
namespace {

constexpr int H = kMfmaH;   // indexer heads
constexpr int D = kMfmaD;   // head dim
constexpr int NWAVE = 8;    // wavefronts per workgroup, one query token each
constexpr int TQ = NWAVE;
constexpr int KT = 128;     // keys per LDS tile
constexpr int KROW = D;  // bf16 per LDS key row (256 B); 16-byte piece p of row r at p ^ (r & 15)
constexpr int CAP = 1280;   // candidate slots per token
// A tile adds at most 2 pairs (128 entries) to a buffer between two tile
// ends: a raise is called for above RAISE_HI, and every buffer above
// RAISE_LO (> k, so a raise is possible) takes part.
constexpr int RAISE_HI = CAP - 64 - 128;
constexpr int RAISE_LO = 768;
static_assert(kMfmaMaxK < RAISE_LO && RAISE_LO < RAISE_HI, "a raise keeps k of more than k entries");
constexpr int THREADS = NWAVE * 64;

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

constexpr int KROW8 = D + 16;  // bytes per LDS key row of raw E4M3 codes (fp8 x fp8 scorer)

struct alignas(16) Smem {
    uint16_t k[2][KT * KROW];
    float scale[2][KT];
    float cs[TQ][CAP];
    int ci[TQ][CAP];
    uint32_t hist[NWAVE][256];
    alignas(8) uint8_t rneed[2][NWAVE];  // per tile parity: this wavefront's buffer is above RAISE_HI
    int last;  // split parts: this block arrived last for its 8 tokens
};

// v_mfma_f32_16x16x32_bf16 operand layout: lane l supplies row (A) or column
// (B) l % 16 and the 8 contraction elements (l / 16) * 8 .. +7; the result
// element i of lane l is row 4 * (l / 16) + i, column l % 16.

// max(x, 0) in one instruction (scores stay far below the upper clamp).
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, 3.0e38f); }

constexpr int CREG = CAP / 64;  // buffer entries per lane when held in registers

// Lane `lane` holds buffer entries i = j*64 + lane (j < CREG) in registers;
// entries past n read as key 0 (no key: below every finite score's key).
__device__ __forceinline__ void load_buffer(const float *cs, const int *ci, int n, int lane,
                                            uint32_t (&u)[CREG], int (&iv)[CREG])
{
#pragma unroll
    for (int j = 0; j < CREG; ++j) {
        const int i = j * 64 + lane;
        u[j] = i < n ? ord_key(cs[i]) : 0u;
        iv[j] = i < n ? ci[i] : 0;
    }
}

// Stable in-place compaction of the register-held buffer: keep(key, rank
// among equal-to-tie keys) decides; returns the new count.
template <class Keep>
__device__ __forceinline__ int wave_compact(float *cs, int *ci, const uint32_t (&u)[CREG],
                                            const int (&iv)[CREG], uint32_t tie, int lane, Keep keep)
{
    uint32_t out = 0, ties = 0;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < CREG; ++j) {
        const bool valid = u[j] != 0u;
        const bool eq = valid && u[j] == tie;
        const uint64_t meq = wave_ballot(eq);
        const bool k = valid && keep(u[j], eq, ties + lanes_below(meq));
        const uint64_t mk = wave_ballot(k);
        if (k) {
            const uint32_t pos = out + lanes_below(mk);
            cs[pos] = key_float(u[j]);
            ci[pos] = iv[j];
        }
        out += (uint32_t)__builtin_popcountll(mk);
        ties += (uint32_t)__builtin_popcountll(meq);
    }
    wave_lds_sync();
    return (int)out;
}

// Wavefront-wide: reduce the candidate buffer (cs, ci)[0..n) with n > k to
// exactly its top-k, keeping index order; returns the k-th score. The k-th
// largest order key is found digit by digit: each pass takes the AND and OR
// of the keys still in play and starts its 8-bit window at their highest
// differing bit, so shared high bits cost no pass.
__device__ __forceinline__ float wave_keep_topk(float *cs, int *ci, int n, int k, uint32_t *hist, int lane)
{
    uint32_t u[CREG];
    int iv[CREG];
    load_buffer(cs, ci, n, lane, u, iv);
    uint32_t ties;
    const uint32_t tau = wave_kth_key<CREG>(u, (uint32_t)k, hist, lane, ties);
    wave_compact(cs, ci, u, iv, tau, lane,
                 [&](uint32_t key, bool eq, uint32_t rank) { return key > tau || (eq && rank < ties); });
    return key_float(tau);
}

// Wavefront-wide, cheap: raise the admission threshold without finding the
// exact k-th key. The AND/OR of all entries gives the bits they share; one
// 8-bit histogram over the window just below them finds the highest bin edge
// with at least k entries at or above it; a stable pass keeps exactly those.
// Nothing that can still reach the top k is dropped (k entries already sit at
// or above the edge). Returns the new count (n when no edge frees space);
// `edge` receives the order key from which later scores are admitted.
__device__ __forceinline__ int wave_raise_threshold(float *cs, int *ci, int n, int k, uint32_t *hist, int lane,
                                    uint32_t &edge)
{
    uint32_t u[CREG];
    int iv[CREG];
    load_buffer(cs, ci, n, lane, u, iv);
    uint32_t a = ~0u, o = 0u;
#pragma unroll
    for (int j = 0; j < CREG; ++j)
        if (u[j] != 0u) {
            a &= u[j];
            o |= u[j];
        }
    a = wave_and(a);
    o = wave_or(o);
    const uint32_t diff = a ^ o;
    if (diff == 0u) return n;
    const int hb = 31 - __builtin_clz(diff);
    const uint32_t above = hb == 31 ? 0u : (~0u << (hb + 1));
    const int lo = hb >= 7 ? hb - 7 : 0;
    const uint32_t dmask = (2u << (hb - lo)) - 1u;
    uint32_t higher;
    const uint32_t bin = wave_digit<CREG>(u, a & above, above, lo, dmask, (uint32_t)k, hist, lane, higher);
    uint32_t e = (a & above) | (bin << lo);
    if (e < 0x00800000u) e = 0x00800000u;  // never below -FLT_MAX: a NaN threshold admits nothing
    const int kept = wave_compact(cs, ci, u, iv, 0xffffffffu, lane,
                                  [&](uint32_t key, bool, uint32_t) { return key >= e; });
    edge = e;
    return kept;
}

template <bool KFP8>
struct TileRegs {
    uint4 v[KFP8 ? 2 : 4];
};

// Thread tid stages key (tid / 4) of the tile, bytes quarter (tid % 4) of the row.
template <bool KFP8>
__device__ __forceinline__ void load_tile(TileRegs<KFP8> &r, float &sc, const uint8_t *Kb,
                                          const float *Ksb, int S, int tile, int tid)
{
    const int key = tile * KT + (tid >> 2);
    const int part = tid & 3;
    constexpr int ROWB = KFP8 ? D : 2 * D;
    constexpr int NV = KFP8 ? 2 : 4;
    if (key < S) {
        const uint4 *src = reinterpret_cast<const uint4 *>(Kb + (size_t)key * ROWB + part * (ROWB / 4));
#pragma unroll
        for (int j = 0; j < NV; ++j) r.v[j] = src[j];
        sc = (KFP8 && part == 0) ? Ksb[key] : 1.0f;
    } else {
#pragma unroll
        for (int j = 0; j < NV; ++j) r.v[j] = make_uint4(0, 0, 0, 0);
        sc = 1.0f;
    }
}

// Two E4M3 codes (the low or high 16 bits of w) -> two bf16 (exact).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// fp8 x fp8 scorer: the codes stay raw, 144-byte rows (32-byte fragment reads
// of 8 consecutive rows fall in distinct banks).
__device__ __forceinline__ void store_tile_raw(Smem &sm, int buf, const TileRegs<true> &r, float sc, int tid)
{
    const int key = tid >> 2, part = tid & 3;
    uint4 *dst = reinterpret_cast<uint4 *>(reinterpret_cast<uint8_t *>(&sm.k[buf][0]) + key * KROW8 + part * 32);
    dst[0] = r.v[0];
    dst[1] = r.v[1];
    if (part == 0) sm.scale[buf][key] = sc;
}

template <bool KFP8>
__device__ __forceinline__ void store_tile(Smem &sm, int buf, const TileRegs<KFP8> &r, float sc, int tid)
{
    const int key = tid >> 2, part = tid & 3, sw = key & 15;
    uint4 *row = reinterpret_cast<uint4 *>(&sm.k[buf][key * KROW]);
    if (KFP8) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 w = r.v[j];
            row[(4 * part + 2 * j) ^ sw] = make_uint4(fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x),
                                                      fp8x2_to_bf16x2<false>(w.y), fp8x2_to_bf16x2<true>(w.y));
            row[(4 * part + 2 * j + 1) ^ sw] = make_uint4(fp8x2_to_bf16x2<false>(w.z), fp8x2_to_bf16x2<true>(w.z),
                                                          fp8x2_to_bf16x2<false>(w.w), fp8x2_to_bf16x2<true>(w.w));
        }
        if (part == 0) sm.scale[buf][key] = sc;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) row[(4 * part + j) ^ sw] = r.v[j];
    }
}

// Key parts (SPLITK): each wavefront holds its token's exact selection among
// this part's keys (cs/ci, cnt entries in index order). It is published with
// device-scope stores; after every wavefront's stores have completed and the
// workgroup has passed a barrier, one lane counts the part in; the workgroup
// that sees the last count merges, each wavefront its token: the parts'
// lists, concatenated in part order (= index order), go into registers, the
// exact k-th key comes from register radix passes, and an ordered ballot
// compaction writes the row. The same instruction-level handoff as the
// split-key kernel's (see there).
__device__ __forceinline__ void parts_finish(Smem &sm, float *cs, int *ci, int cnt, int topk, bool tok_ok,
                                             long long q0, int tok, int t0, int part, int nparts,
                                             const PrefillParts &pw, int *__restrict__ idx,
                                             float *__restrict__ vals)
{
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const long long row = q0 + tok;
    if (tok_ok) {
        wave_lds_sync();
        if (cnt > topk) {
            wave_keep_topk(cs, ci, cnt, topk, sm.hist[wid], lane);
            cnt = topk;
        }
        uint64_t *lst = pw.list + ((size_t)row * kPrefillMaxParts + part) * topk;
        for (int i = lane; i < cnt; i += 64) store_agent(&lst[i], ((uint64_t)(uint32_t)ci[i] << 32) | ord_key(cs[i]));
        if (lane == 0) store_agent(&pw.cnt[row * kPrefillMaxParts + part], (uint32_t)cnt);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint32_t *ctr = pw.ctr + (q0 + t0);  // one counter per 8-token block: its first row
    if (tid == 0)
        sm.last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nparts - 1);
    __syncthreads();
    if (!sm.last) return;
    if (tok_ok) {
        constexpr int MC = kPrefillMaxParts * kMfmaMaxK / 64;  // entries per lane
        uint32_t pc[kPrefillMaxParts], tot = 0;
#pragma unroll
        for (int q = 0; q < kPrefillMaxParts; ++q) {
            pc[q] = q < nparts ? load_agent(&pw.cnt[row * kPrefillMaxParts + q]) : 0u;
            tot += pc[q];
        }
        const uint64_t *rl = pw.list + (size_t)row * kPrefillMaxParts * topk;
        uint32_t u[MC];
        int iv[MC];
#pragma unroll
        for (int j = 0; j < MC; ++j) {
            const uint32_t e = (uint32_t)(j * 64 + lane);
            uint32_t base = 0;
            int q = 0;
#pragma unroll
            for (int qq = 0; qq < kPrefillMaxParts - 1; ++qq)
                if (q == qq && e >= base + pc[qq]) {
                    base += pc[qq];
                    q = qq + 1;
                }
            u[j] = 0u;
            iv[j] = 0;
            if (e < tot) {
                const uint64_t v = load_agent(&rl[(size_t)q * topk + (e - base)]);
                u[j] = (uint32_t)v;
                iv[j] = (int)(v >> 32);
            }
        }
        uint32_t tau = 0, ties = 0;  // at most k entries: every one is kept
        if (tot > (uint32_t)topk) tau = wave_kth_key<MC>(u, (uint32_t)topk, sm.hist[wid], lane, ties);
        int *io = idx + row * topk;
        float *vo = vals ? vals + row * topk : nullptr;
        uint32_t out = 0, eqseen = 0;
#pragma unroll
        for (int j = 0; j < MC; ++j) {
            const uint32_t key = u[j];
            const bool eq = key != 0u && key == tau;
            const uint64_t meq = wave_ballot(eq);
            const bool keep = key != 0u && (key > tau || (eq && eqseen + lanes_below(meq) < ties));
            const uint64_t mk = wave_ballot(keep);
            if (keep) {
                const uint32_t pos = out + lanes_below(mk);
                io[pos] = iv[j];
                if (vo) vo[pos] = key_float(key);
            }
            out += (uint32_t)__builtin_popcountll(mk);
            eqseen += (uint32_t)__builtin_popcountll(meq);
        }
        for (int j = (int)out + lane; j < topk; j += 64) {
            io[j] = -1;
            if (vo) vo[j] = -INFINITY;
        }
    }
    if (tid == 0) *ctr = 0u;
}

// Ragged batches (VARLEN): the streams of rg (see StreamGeo); the grid's x
// dimension covers every stream's 8-token blocks, and blocks past the last
// one exit at once.
// QFP8: the fp8 x fp8 scorer. Q holds E4M3 codes with one fp32 scale per
// (token, head) in QS; the scale is positive, so it commutes with the ReLU and
// joins the head weight. Keys stay raw E4M3 in LDS and each 16 x 16 tile is
// one v_mfma_scale_f32_16x16x128_f8f6f4 over all 128 dims (unit block
// scales): the same lane mapping for both operands (lane l: row or column
// l % 16, bytes 32 (l / 16) .. +31) pairs their contraction elements.
template <bool KFP8, bool SCORE, bool VARLEN, bool QFP8, bool SPLITK = false>
__global__ __launch_bounds__(THREADS, 1) void mfma_indexer_kernel(
    const uint16_t *__restrict__ Q, const uint8_t *__restrict__ K, const float *__restrict__ Ks,
    const float *__restrict__ W, int T, int S, long long offset, int topk, int *__restrict__ idx,
    float *__restrict__ vals, float *__restrict__ scores, const float *__restrict__ QS, Ragged rg,
    PrefillParts pp_ws = PrefillParts{})
{
    static_assert(!QFP8 || (KFP8 && !SCORE && !VARLEN), "the fp8 x fp8 scorer is the E4M3-key select");
    static_assert(!SPLITK || (VARLEN && !SCORE && !QFP8), "key parts are a ragged-select feature");
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    // This block's stream: first query row q0, first key row k0, Tb queries
    // over Sb cached keys, query t seeing keys <= offb + t.
    long long q0, k0, offb;
    int Tb, Sb, t0;
    int part = 0, nparts = 1;  // key part of this block (SPLITK), of nparts
    if constexpr (VARLEN) {
        int j = 0;
        const int bs = wave_block_stream(rg.cu_q, rg.cu_k, rg.B, rg.total_q, rg.total_k, TQ, blockIdx.x, lane, j,
                                         SPLITK ? pp_ws.kpart : 0, kPrefillMaxParts);
        if (bs < 0) return;  // the same for every wavefront of the block
        const StreamGeo g = stream_geo(rg.cu_q, rg.cu_k, bs, rg.total_q, rg.total_k);
        q0 = g.q0;
        k0 = g.k0;
        Sb = (int)(g.S < 0x7fffffffLL ? g.S : 0x7fffffffLL);
        Tb = g.T < Sb ? g.T : Sb;  // rows past the cache (malformed input) are dropped
        offb = (long long)g.S - g.T;
        if constexpr (SPLITK) {
            nparts = stream_parts(g.S, pp_ws.kpart, kPrefillMaxParts);
            part = j % nparts;
            j /= nparts;
        }
        t0 = ((Tb + TQ - 1) / TQ - 1 - j) * TQ;  // longest rows of the stream first
    } else {
        const int nblk = (T + TQ - 1) / TQ;
        t0 = (nblk - 1 - (int)blockIdx.x) * TQ;  // longest rows first
        q0 = (long long)blockIdx.y * T;
        k0 = (long long)blockIdx.y * S;
        Tb = T;
        Sb = S;
        offb = offset;
    }
    const int tok = t0 + wid;
    const bool tok_ok = tok < Tb;
    const long long lim = tok_ok ? offb + tok : -1;  // last key this token sees

    // Query as MFMA A operands: a[m][ks] = Q[tok, head 16m + lane%16,
    // dims 32ks + (lane/16)*8 .. +7]. B operands use the same dim mapping.
    // wv[m][i] = W[tok, head 16m + 4(lane/16) + i], the heads of this lane's
    // accumulator elements.
    bf16x8 a[4][4];
    i32x8 a8[4];  // QFP8: a8[m] = codes of head 16m + lane%16, dims 32 (lane/16) .. +31
    float wv[4][4];
    {
        const long long qrow = (q0 + (tok_ok ? tok : 0)) * H;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if constexpr (QFP8) {
                const uint4 *qp = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(Q) +
                                                                  (qrow + m * 16 + (lane & 15)) * D + (lane >> 4) * 32);
                const uint4 lo = tok_ok ? qp[0] : make_uint4(0, 0, 0, 0);
                const uint4 hi = tok_ok ? qp[1] : make_uint4(0, 0, 0, 0);
                a8[m] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            } else {
                const bf16x8 *qp = reinterpret_cast<const bf16x8 *>(
                    Q + (qrow + m * 16 + (lane & 15)) * D + (lane >> 4) * 8);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) a[m][ks] = tok_ok ? qp[ks * 4] : bf16x8{};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long long hrow = qrow + m * 16 + 4 * (lane >> 4) + i;
                wv[m][i] = tok_ok ? (QFP8 ? W[hrow] * QS[hrow] : W[hrow]) : 0.0f;
            }
        }
    }

    const long long blk_last = offb + (t0 + TQ < Tb ? t0 + TQ : Tb) - 1;  // last key any token sees
    const long long nkeys = SCORE ? (long long)Sb : blk_last + 1;
    // Tiles tlo .. thi-1: every tile of the visible keys, or with key parts
    // (SPLITK) those of part `part`: keys part*kpart .. (part+1)*kpart - 1,
    // the last part taking the rest (kpart is a multiple of KT).
    int tlo = 0, thi = (int)((nkeys + KT - 1) / KT);
    if constexpr (SPLITK) {
        if (nparts > 1) {
            const int per = pp_ws.kpart / KT;
            tlo = part * per;
            if (part < nparts - 1) thi = thi < tlo + per ? thi : tlo + per;
            if (thi < tlo) thi = tlo;
        }
    }
    const int ntiles = thi - tlo;
    const uint8_t *Kb = K + (size_t)k0 * (KFP8 ? D : 2 * D);
    const float *Ksb = KFP8 ? Ks + (size_t)k0 : nullptr;
    float *cs = sm.cs[wid];
    int *ci = sm.ci[wid];
    int cnt = 0;
    float thr = -INFINITY;  // a score enters the buffer iff score >= thr

    TileRegs<KFP8> tr;
    float tsc;
    load_tile<KFP8>(tr, tsc, Kb, Ksb, Sb, tlo, tid);
    if constexpr (QFP8) store_tile_raw(sm, 0, tr, tsc, tid);
    else store_tile<KFP8>(sm, 0, tr, tsc, tid);
    __syncthreads();

    // Half-pair software pipeline. A 64-key pair is two 32-key halves of 8
    // output tiles each (acc[s] for keys 32s..32s+31 of the pair). The MFMAs
    // of one half run while the VALU reduces the other (the previous half),
    // k-step by k-step with a scheduling fence after each, so the matrix
    // cores and the VALU of a wavefront overlap; only the usual 64
    // accumulator registers are live. Pairs past a token's last visible key
    // are computed and masked (at most the block's 8-token spread).
    f32x4 acc[2][2][4];  // [half][n][m]
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[1][n][m] = f32x4{};
    // MFMAs of half h of the pair at pair offset pp in buffer cur into
    // acc[h], interleaved with the reduction of acc[h ^ 1] into part[n].
    auto phase = [&](int h, int cur, int pp, float (&part)[2]) {
        if constexpr (QFP8) {
            // one MFMA per output tile; the reduction of the other half's key
            // tile n follows the four MFMAs of key tile n
            const uint8_t *kp8 = reinterpret_cast<const uint8_t *>(&sm.k[cur][0]) +
                                 (pp * 64 + 32 * h + (lane & 15)) * KROW8 + (lane >> 4) * 32;
            const f32x4 (&r)[2][4] = acc[h ^ 1];
            float s4[2][4] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const uint4 *bp = reinterpret_cast<const uint4 *>(kp8 + 16 * n * KROW8);
                const uint4 lo = bp[0], hi = bp[1];
                const i32x8 bk8 = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                // As in the bf16 path: the key tile's MFMAs interleaved with
                // the reduction, one MFMA to eight VALU instructions, at
                // raised wavefront priority (1.5% on the 64k step).
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    acc[h][n][m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8[m], bk8, f32x4{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s4[n][i] = fmaf(wv[m][i], relu(r[n][m][i]), s4[n][i]);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                }
                asm volatile("" : "+v"(s4[n][0]), "+v"(s4[n][1]), "+v"(s4[n][2]), "+v"(s4[n][3]));
                __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int n = 0; n < 2; ++n) part[n] = (s4[n][0] + s4[n][1]) + (s4[n][2] + s4[n][3]);
            return;
        }
        const int swz = lane & 15;
        const uint16_t *kp = &sm.k[cur][(pp * 64 + 32 * h + (lane & 15)) * KROW + ((lane >> 4) ^ (swz & 3)) * 8];
        const f32x4 (&r)[2][4] = acc[h ^ 1];
        float s4[2][4] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
        bf16x8 bk[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) bk[n] = *reinterpret_cast<const bf16x8 *>(kp + 16 * n * KROW + 32 * (swz >> 2));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 nb[2] = {bk[0], bk[1]};
            if (ks < 3) {
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    nb[n] = *reinterpret_cast<const bf16x8 *>(kp + 16 * n * KROW + ((ks + 1) ^ (swz >> 2)) * 32);
            }
            // A k-step issues its 8 MFMAs interleaved with the 16 VALU
            // instructions of the other half's reduction, one MFMA to two
            // (scheduling group barriers), at raised wavefront priority: the
            // wavefront feeds the matrix pipe first, and the other wavefront
            // of the SIMD fills the gaps that remain. (The priority alone
            // gave 2.5% on the 64k step, the interleave a further 1.1%.)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    acc[h][n][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m][ks], bk[n],
                                                                          ks ? acc[h][n][m] : f32x4{}, 0, 0, 0);
            const int n = ks >> 1;  // 8 of the 32 elements of the half being reduced
#pragma unroll
            for (int mm = 0; mm < 2; ++mm) {
                const int m = 2 * (ks & 1) + mm;
#pragma unroll
                for (int i = 0; i < 4; ++i) s4[n][i] = fmaf(wv[m][i], relu(r[n][m][i]), s4[n][i]);
            }
            // Pin this step's reduction here (value-only code would otherwise
            // sink below the fence, to its use after the last step).
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
            }
            asm volatile("" : "+v"(s4[n][0]), "+v"(s4[n][1]), "+v"(s4[n][2]), "+v"(s4[n][3]));
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
            bk[0] = nb[0];
            bk[1] = nb[1];
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) part[n] = (s4[n][0] + s4[n][1]) + (s4[n][2] + s4[n][3]);
    };
    // Scale, mask and insert (or store) the pair at pbase from its halves'
    // partial head sums and its keys' scales (lane l: key l of the pair):
    // after the 32- and 16-lane swaps lane l holds the score of key l.
    auto finish_pair = [&](const float (&p0)[2], const float (&p1)[2], long long pbase, float kscale) {
        float hsum[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const auto w32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0[n]), __float_as_uint(p1[n]),
                                                              false, false);
            hsum[n] = __uint_as_float(w32[0]) + __uint_as_float(w32[1]);
        }
        const auto w16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(hsum[0]), __float_as_uint(hsum[1]),
                                                          false, false);
        float sc = __uint_as_float(w16[0]) + __uint_as_float(w16[1]);
        if (KFP8) sc *= kscale;
        sc = canon(sc);
        const long long key = pbase + lane;
        const bool vis = key <= lim;
        if (SCORE) {
            if (tok_ok && key < Sb) scores[(q0 + tok) * Sb + key] = vis ? sc : -INFINITY;
        } else {
            const bool pass = vis && sc >= thr;
            const uint64_t m = wave_ballot(pass);
            if (m) {
                const int pos = cnt + (int)lanes_below(m);
                if (pass) {
                    cs[pos] = sc;
                    ci[pos] = (int)key;
                }
                cnt += __builtin_popcountll(m);  // at most RAISE_HI + 128 <= CAP (see the tile loop)
            }
        }
    };
    // Raise this token's threshold (cnt > RAISE_LO > topk entries).
    auto raise_now = [&]() {
        wave_lds_sync();
        uint32_t edge = 0;
        const int kept = wave_raise_threshold(cs, ci, cnt, topk, sm.hist[wid], lane, edge);
        if (kept < cnt && kept <= CAP - 256) {
            cnt = kept;
            thr = key_float(edge);
        } else {  // too little freed (or all entries equal): exact k-th, admit strictly above it
            const float kth = wave_keep_topk(cs, ci, kept, topk, sm.hist[wid], lane);
            cnt = topk;
            thr = key_float(ord_key(kth) + 1u);
        }
    };

    float prev0[2] = {0.0f, 0.0f};  // first half's partial sums of the pair in flight
    // Scales of the tile's last pair, whose finish runs in the next tile's
    // first phase. They are read into a register before the end-of-tile
    // barrier: by that finish, other wavefronts may already be staging the
    // tile after next into the same scale buffer.
    float pend_scale = 1.0f;
    bool raise_pending = false;
    for (int it = 0; it < ntiles; ++it) {
        const int tile = tlo + it;
        const int cur = it & 1;
        if (it + 1 < ntiles) load_tile<KFP8>(tr, tsc, Kb, Ksb, Sb, tile + 1, tid);
        const long long kbase = (long long)tile * KT;
#pragma unroll
        for (int pp = 0; pp < KT / 64; ++pp) {
            float h1[2], h0[2];
            phase(0, cur, pp, h1);  // MFMAs of this pair's first half; previous pair's second half reduced
            if (!SCORE && pp == 0 && raise_pending) raise_now();
            if (pp > 0)
                finish_pair(prev0, h1, kbase + pp * 64 - 64, KFP8 ? sm.scale[cur][(pp - 1) * 64 + lane] : 1.0f);
            else if (it > 0)
                finish_pair(prev0, h1, kbase - 64, pend_scale);
            phase(1, cur, pp, h0);  // MFMAs of the second half; this pair's first half reduced
            prev0[0] = h0[0];
            prev0[1] = h0[1];
        }
        if (KFP8) pend_scale = sm.scale[cur][KT - 64 + lane];
        if (it + 1 < ntiles) {
            if constexpr (QFP8) store_tile_raw(sm, cur ^ 1, tr, tsc, tid);
            else store_tile<KFP8>(sm, cur ^ 1, tr, tsc, tid);
        }
        if (!SCORE && lane == 0) sm.rneed[cur][wid] = cnt > RAISE_HI ? 1 : 0;
        __syncthreads();
        // Raises are taken together: when some buffer is above RAISE_HI, every
        // buffer above RAISE_LO is raised in the next tile, after its first
        // MFMAs are issued and before its first insert. Until the next tile's
        // end, at most 128 more entries arrive (this tile's last pair and the
        // next tile's first); after the last tile only its last pair, so a
        // raise asked for there is not needed. The flags alternate between two
        // rows, so a wavefront already writing the next tile's cannot
        // overwrite these.
        if constexpr (!SCORE)
            raise_pending = *reinterpret_cast<const uint64_t *>(sm.rneed[cur]) != 0 && cnt > RAISE_LO;
    }
    if (ntiles > 0) {  // the last pair's second half
        float h1[2];
        const f32x4 (&r)[2][4] = acc[1];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) s4[i] = fmaf(wv[m][i], relu(r[n][m][i]), s4[i]);
            h1[n] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
        finish_pair(prev0, h1, (long long)thi * KT - 64, pend_scale);
    }

    if constexpr (SPLITK) {
        if (nparts > 1) {
            parts_finish(sm, cs, ci, cnt, topk, tok_ok, q0, tok, t0, part, nparts, pp_ws, idx, vals);
            return;
        }
    }

    if (!SCORE && tok_ok) {
        wave_lds_sync();
        if (cnt > topk) {
            wave_keep_topk(cs, ci, cnt, topk, sm.hist[wid], lane);
            cnt = topk;
        }
        const long long orow = (q0 + tok) * topk;
        for (int i = lane; i < topk; i += 64) {
            const bool have = i < cnt;
            idx[orow + i] = have ? ci[i] : -1;
            if (vals) vals[orow + i] = have ? cs[i] : -INFINITY;
        }
    }
}

template <bool KFP8, bool SCORE>
hipError_t launch(const Problem &p, const void *Q, const void *K, const float *Ks, const float *W,
                  int k, int *idx, float *vals, float *scores, hipStream_t st)
{
    const int nblk = (p.T + TQ - 1) / TQ;
    hipLaunchKernelGGL((mfma_indexer_kernel<KFP8, SCORE, false, false>), dim3(nblk, p.B), dim3(THREADS), 0, st,
                       static_cast<const uint16_t *>(Q), static_cast<const uint8_t *>(K), Ks, W, p.T,
                       p.S, p.offset, k, idx, vals, scores, nullptr, Ragged{});
    return hipGetLastError();
}

}  // namespace

bool mfma_shape_ok(const Problem &p)
{
    return p.H == H && p.D == D && p.q_dtype == BF16 && (p.k_dtype == BF16 || p.k_dtype == FP8);
}

hipError_t launch_mfma_score(const Problem &p, const void *Q, const void *K, const float *Ks,
                             const float *W, float *scores, hipStream_t st)
{
    if (p.k_dtype == FP8) return launch<true, true>(p, Q, K, Ks, W, 0, nullptr, nullptr, scores, st);
    return launch<false, true>(p, Q, K, Ks, W, 0, nullptr, nullptr, scores, st);
}

hipError_t launch_mfma_select(const Problem &p, const void *Q, const void *K, const float *Ks,
                              const float *W, int k, int *idx, float *vals, hipStream_t st)
{
    if (p.k_dtype == FP8) return launch<true, false>(p, Q, K, Ks, W, k, idx, vals, nullptr, st);
    return launch<false, false>(p, Q, K, Ks, W, k, idx, vals, nullptr, st);
}

hipError_t launch_mfma_select_qfp8(const Problem &p, const void *Q8, const float *QS, const void *K, const float *Ks,
                                   const float *W, int k, int *idx, float *vals, hipStream_t st)
{
    const int nblk = (p.T + TQ - 1) / TQ;
    hipLaunchKernelGGL((mfma_indexer_kernel<true, false, false, true>), dim3(nblk, p.B), dim3(THREADS), 0, st,
                       static_cast<const uint16_t *>(Q8), static_cast<const uint8_t *>(K), Ks, W, p.T, p.S, p.offset,
                       k, idx, vals, nullptr, QS, Ragged{});
    return hipGetLastError();
}

long long mfma_varlen_blocks(int B, int total_q) { return ((long long)total_q + TQ - 1) / TQ + B; }

namespace {

std::atomic<int> g_prefill_split{-2};  // -2: not read from the environment yet

int prefill_split_now()
{
    int v = g_prefill_split.load(std::memory_order_relaxed);
    if (v != -2) return v;
    int init = 0;
    if (const char *e = std::getenv("DS4IDX_PREFILL_SPLIT")) {
        const int x = std::atoi(e);
        init = x < 0 ? -1 : x;
    }
    int expected = -2;
    g_prefill_split.compare_exchange_strong(expected, init);
    return g_prefill_split.load(std::memory_order_relaxed);
}

constexpr int kPrefillPartKeys = 8192;  // automatic part length

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

int set_prefill_split(int keys)
{
    const int prev = prefill_split_now();
    g_prefill_split.store(keys < 0 ? -1 : keys, std::memory_order_relaxed);
    return prev;
}

int get_prefill_split() { return prefill_split_now(); }

// A small ragged prefill batch whose longest rows set the pace: 8-token
// blocks over long caches are split into key parts of 8192 (at most
// kPrefillMaxParts, so longer caches get longer parts). Batches with more
// blocks than two rounds of the 256 CUs balance well without parts.
int prefill_kpart(const VarlenProblem &p)
{
    const int o = prefill_split_now();
    if (o < 0 || p.total_q == 0) return 0;
    const long long per4 = ((long long)p.max_k + kPrefillMaxParts - 1) / kPrefillMaxParts;
    long long kp;
    if (o > 0) {
        kp = o > per4 ? o : per4;
    } else {
        if (p.max_k <= kPrefillPartKeys || mfma_varlen_blocks(p.B, p.total_q) > 2 * kSplitCUs) return 0;
        kp = kPrefillPartKeys > per4 ? kPrefillPartKeys : per4;
    }
    kp = (kp + KT - 1) / KT * KT;
    if (kp >= p.max_k) return 0;  // one part
    return kp > 0x7fffffffLL ? 0 : (int)kp;
}

size_t prefill_parts_workspace_bytes(const VarlenProblem &p, int k)
{
    if (prefill_kpart(p) == 0) return 0;
    const size_t rows = (size_t)p.total_q;
    return align256(rows * 4) + align256(rows * kPrefillMaxParts * 4) + align256(rows * kPrefillMaxParts * (size_t)k * 8);
}

hipError_t launch_mfma_select_varlen(const VarlenProblem &p, const int *cu_q, const long long *cu_k,
                                     const void *Q, const void *K, const float *Ks, const float *W,
                                     int k, int *idx, float *vals, void *ws, hipStream_t st)
{
    const Ragged rg{cu_q, cu_k, p.B, p.total_q, p.total_k};
    const uint16_t *q = static_cast<const uint16_t *>(Q);
    const uint8_t *kk = static_cast<const uint8_t *>(K);
    const int kpart = prefill_kpart(p);
    if (kpart > 0) {
        // Every stream's blocks fit in (ceil(total_q / 8) + B) x parts.
        const dim3 grid((unsigned)(mfma_varlen_blocks(p.B, p.total_q) * kPrefillMaxParts));
        const size_t rows = (size_t)p.total_q;
        char *c = static_cast<char *>(ws);
        PrefillParts pw;
        pw.kpart = kpart;
        pw.ctr = reinterpret_cast<uint32_t *>(c);
        c += align256(rows * 4);
        pw.cnt = reinterpret_cast<uint32_t *>(c);
        c += align256(rows * kPrefillMaxParts * 4);
        pw.list = reinterpret_cast<uint64_t *>(c);
        if (p.k_dtype == FP8)
            hipLaunchKernelGGL((mfma_indexer_kernel<true, false, true, false, true>), grid, dim3(THREADS), 0, st, q, kk,
                               Ks, W, 0, 0, 0LL, k, idx, vals, nullptr, nullptr, rg, pw);
        else
            hipLaunchKernelGGL((mfma_indexer_kernel<false, false, true, false, true>), grid, dim3(THREADS), 0, st, q,
                               kk, Ks, W, 0, 0, 0LL, k, idx, vals, nullptr, nullptr, rg, pw);
        return hipGetLastError();
    }
    // Every stream's blocks fit in ceil(total_q / 8) + B.
    const dim3 grid((unsigned)mfma_varlen_blocks(p.B, p.total_q));
    if (p.k_dtype == FP8)
        hipLaunchKernelGGL((mfma_indexer_kernel<true, false, true, false>), grid, dim3(THREADS), 0, st, q, kk, Ks, W, 0,
                           0, 0LL, k, idx, vals, nullptr, nullptr, rg, PrefillParts{});
    else
        hipLaunchKernelGGL((mfma_indexer_kernel<false, false, true, false>), grid, dim3(THREADS), 0, st, q, kk, Ks, W,
                           0, 0, 0LL, k, idx, vals, nullptr, nullptr, rg, PrefillParts{});
    return hipGetLastError();
}

}  // namespace ds4idx
