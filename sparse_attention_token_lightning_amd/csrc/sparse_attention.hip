// Sparse attention over the indexer's selected positions, on gfx950 matrix
// cores. Each query token attends only to its selected cache rows (first
// page, "DeepSeek V4 Flash 추론을 1.6초로 줄인 ds4 최적화", glossary entry on
// sparse attention). The MI300X write-up ("DeepSeek V4 Flash는 단일 AMD
// MI300X에서 실행됩니다") keeps an MLA cache (deployment checklist, hybrid KV
// strategy: fp8_ds_mla) and tiles the sparse prefill 64 heads at a time
// (production tuning table, BLOCK_H=64). Here one latent row c[s] of 576 values
// is the key of every head and its first 512 values the value:
//
//   out[t,h] = sum_j softmax_j(scale * q[t,h] . c[idx_j]) c[idx_j, 0:512]
//
// over the valid entries of idx[t] (0 <= idx < S), plus lse[t,h].
//
// Layout on CDNA4. The work items are (query token, tile of 64 heads); one
// 512-thread workgroup per CU takes a contiguous run of them, and each item's
// selected rows stream through LDS in chunks of 32:
//  * Gather. The rows of a chunk go straight from global memory into LDS
//    (global_load_lds_dwordx4: each wavefront instruction moves 64 x 16 bytes
//    of one 1 KB row head, or in 32 lanes the 128-byte tails of 4 rows), into
//    a ring of four chunk buffers, two to three chunks ahead of the one being
//    computed, so a CU keeps ~75-110 KB of gathers in flight without holding
//    them in registers. The ring runs on from one item into the next: the
//    next item's first chunks, its Q and its successor's row indices are
//    loaded while the current item finishes. The 16-byte pieces of a row are
//    XOR-swizzled by the row number so the MFMA fragment reads below are
//    bank-conflict free.
//  * Scores transposed, S^T = C Q^T (v_mfma_f32_16x16x32_bf16, keys on M,
//    heads on N): wavefront w computes the 16-key x 16-head tile (w & 1,
//    w >> 1) over 18 k-steps of the 576 dims, with its 16 heads of Q resident
//    as B operands and the fragment reads three k-steps ahead.
//  * Online softmax in the log2 domain against a running max per head that
//    every wavefront holds alike; the chunk maxima are exchanged, and the
//    outputs rescaled, only when some head's max rises by more than a factor
//    2^8. Each wavefront sums its own keys' probabilities; the two key tiles'
//    sums are added once per item.
//  * Values, O^T = V^T P^T. The S^T accumulator already has the layout of a
//    B operand (lane = head, 4 consecutive keys per lane group) under a fixed
//    permutation of the chunk's 32 keys, two runs of 4 consecutive keys per
//    lane group; the V^T fragments come from the raw rows in that key order
//    with two transposed LDS reads (ds_read_b64_tr_b16) each, instead of
//    eight 2-byte reads (707 -> 648 us on the 4096-query bench, identical
//    output), one value tile ahead. Wavefront w owns value tiles 4w .. 4w+3
//    of all four head tiles: 16 accumulators.
//  * One barrier per chunk (see the main loop).
#include "device_common.h"
#include "kernels.h"

namespace ds4idx {
namespace {

constexpr int AH = kAttnHeadTile;  // heads per workgroup
constexpr int DQK = kAttnDqk, DV = kAttnDv;
constexpr int CK = 32;             // selected rows per chunk
constexpr int NBUF = 4;            // chunk buffers: three in flight, one in use
constexpr int ATHREADS = 512;
constexpr int MAIN16 = DV / 8;     // 16-byte pieces of a row's first 512 values (64)
constexpr int TAIL16 = (DQK - DV) / 8;  // pieces of the rest (8)
constexpr int NQK = DQK / 32;      // k-steps of the score contraction
constexpr float RESCALE_LOG2 = 8.0f;  // largest log2 probability before O is rescaled

static_assert(MAIN16 == 64 && TAIL16 == 8, "one wavefront instruction per row head, per 8 row tails");
static_assert(kAttnMaxK / CK <= 64, "one chunk per lane in the row-index registers");

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

struct AttnSmem {
    uint4 head[NBUF][CK * MAIN16];  // row r, piece p at [r * 64 + (p ^ (r & 15))]
    uint4 tail[NBUF][CK * TAIL16];  // row r, piece q at [r * 8 + (q ^ (r & 7))]
    uint16_t p[2][4][64][8];        // P^T B fragments per head tile and lane, chunk parity
    float pmax[2][AH];              // chunk maxima per key tile and head
    float psum[2][AH];              // an item's sums per key tile and head
    uint8_t validb[2][kAttnMaxK / CK][8];  // item parity, chunk c, byte w, bit j: row 4w + j is valid
    alignas(8) uint8_t jump[2][8];  // per chunk parity and wavefront: a head's max rose by more than 2^RESCALE_LOG2
};

// The chunk's keys in the order shared by the score tiles and the value
// fragments: lane group g (lanes 16g..16g+15) of a score tile holds keys
// 4g..4g+3 of each 16-key tile, so element e of its value-fragment operand is
// key 4g + e for e < 4 and key 16 + 4g + (e - 4) otherwise.

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to bf16, round to nearest even, in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// 2^x with one v_exp_f32: the probabilities here lie in (0, 2^8], and any
// below 2^-126 (flushed to 0 by the instruction) weigh nothing beside the
// row's largest, which is at least 2^-8.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// One 16-byte gather per lane straight into LDS (global_load_lds_dwordx4):
// lane i's bytes land at LDS address lds + 16 i. Issued as inline assembly
// so that the compiler does not treat it as an LDS store it must drain
// (vmcnt(0)) before every later LDS read; completion is awaited explicitly
// with wait_vm, and no other vector-memory instruction runs in the main
// loop. M0 carries the (wavefront-uniform) LDS address; this kernel uses M0
// for nothing else.
__device__ __forceinline__ void gather16(const void *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}

// gather16_at (shared device helpers) does the same from a wavefront-uniform
// base plus a 32-bit per-lane offset: no per-lane 64-bit address arithmetic.

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one head of a
// 16 x 16 accumulator tile) with the permlane swaps, VALU only.
__device__ __forceinline__ float quad_max(float x)
{
    auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(w[0]), __uint_as_float(w[1]));
    w = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(w[0]), __uint_as_float(w[1]));
}

__device__ __forceinline__ float quad_sum(float x)
{
    auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(w[0]) + __uint_as_float(w[1]);
    w = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(w[0]) + __uint_as_float(w[1]);
}

// Where an item (query row, head tile) is: uniform values that step from
// one item to the next without a division.
struct ItemPos {
    long long row;      // b * T + t
    int tile;           // head tile
    int t;              // the row's position in its stream
    const char *cache;  // the stream's latent cache
};

__global__ __launch_bounds__(ATHREADS, 1) void sparse_attention_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ C, const int *__restrict__ idx, int T, int S,
    int H, int topk, long long items, float scale_log2, uint16_t *__restrict__ O, float *__restrict__ lse)
{
    __shared__ AttnSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kt = wid & 1, ht = wid >> 1;
    const int ntile = H / AH;
    const int nchunk = (topk + CK - 1) / CK;
    const int last = topk - 1;

    // Items (query row i / ntile, head tile i % ntile) are dealt out in
    // contiguous runs, one per workgroup, and taken in order.
    const long long first = blockIdx.x * items / gridDim.x, end = (blockIdx.x + 1) * items / gridDim.x;
    if (first >= end) return;
    ItemPos cp;
    cp.row = first / ntile;
    cp.tile = (int)(first % ntile);
    cp.t = (int)(cp.row % T);
    cp.cache = reinterpret_cast<const char *>(C + (cp.row / T) * (long long)S * DQK);
    auto advance = [&](ItemPos q) {
        if (++q.tile == ntile) {
            q.tile = 0;
            ++q.row;
            if (++q.t == T) {
                q.t = 0;
                q.cache += (long long)S * DQK * 2;
            }
        }
        return q;
    };
    ItemPos np = advance(cp);

    // The rows this wavefront gathers for an item, in registers: lane l
    // holds entries 32 l + 4 w + j (j < 4) of chunk l. Every load is issued,
    // at a clamped entry, so that they fly together.
    // (The lane number is made opaque at each call, so that the offsets are
    // computed there instead of being hoisted and held across the loop.)
    auto load_sel = [&](long long row, int (&s)[4]) {
        const int *ir = idx + row * topk;
        int l = lane;
        asm volatile("" : "+v"(l));
#pragma unroll
        for (int j = 0; j < 4; ++j) s[j] = ir[min(l * CK + 4 * wid + j, last)];
    };
    // An entry is valid if it lies within topk and 0 <= idx < S. Its bit
    // goes to the score mask of item parity `par` (chunk c, byte w, bit j =
    // row 4w + j); a row that is not valid is gathered from row 0, so every
    // gathered value is finite, and its score is masked.
    auto validate = [&](int (&s)[4], int par) {
        uint32_t vbits = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool ok = lane * CK + 4 * wid + j <= last && s[j] >= 0 && s[j] < S;
            vbits |= (ok ? 1u : 0u) << j;
            s[j] = ok ? s[j] : 0;
        }
        if (lane < nchunk) sm.validb[par][lane][wid] = (uint8_t)vbits;
    };
    // Q^T fragments of head tile ht: head h0 + 16 ht + lane % 16, dims 32 ks + 8 (lane / 16) ..
    bf16x8 qf[NQK];
    auto q_ptr = [&](const ItemPos &q) {
        const uint16_t *qb = Q + (q.row * H + q.tile * AH + ht * 16) * DQK;
        int l = lane;
        asm volatile("" : "+v"(l));
        return reinterpret_cast<const bf16x8 *>(qb + ((l & 15) * DQK + (l >> 4) * 8));
    };
    auto load_q = [&](const ItemPos &q) {
        const bf16x8 *qp = q_ptr(q);
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks) qf[ks] = qp[ks * 4];
    };
    // Gather of chunk c of an item into buffer b: wavefront w loads the
    // heads of rows 4w..4w+3 (lane i takes piece i ^ (r & 15) of row r into
    // slot i) and, in lanes 0..31, their tails: five instructions per
    // wavefront and chunk.
    // e[j]: the row of entry 4w + j (uniform).
    auto issue = [&](const char *Cb, const int (&e)[4], int b) {
        int l = lane;
        asm volatile("" : "+v"(l));
        int e4 = e[0];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * wid + j;
            e4 = ((l >> 3) & 3) == j ? e[j] : e4;
            gather16_at(Cb + (long long)e[j] * (DQK * 2), (uint32_t)((lane ^ (r & 15)) * 16),
                        __builtin_amdgcn_readfirstlane(lds_addr(&sm.head[b][r * MAIN16])));
        }
        const int r = 4 * wid + ((l >> 3) & 3);
        const char *src = Cb + (long long)e4 * (DQK * 2) + DV * 2 + (((l & 7) ^ (r & 7)) * 16);
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(&sm.tail[b][4 * wid * TAIL16]));
        if (l < 32) gather16(src, dst);
    };
    auto rows_of = [&](const int (&s)[4], int c, int (&e)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = __builtin_amdgcn_readlane(s[j], c);
    };

    int cur[4], nxt[4];
    load_sel(cp.row, cur);
    load_sel(first + 1 < end ? np.row : cp.row, nxt);
    load_q(cp);
    // Finish these loads here, so that no wait for them is left to the main
    // loop (where vmcnt counts only the gathers and, after an item, its
    // output stores).
    wait_vm<0>();
#pragma unroll
    for (int ks = 0; ks < NQK; ++ks) asm volatile("" : "+v"(qf[ks]));
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(cur[j]), "+v"(nxt[j]));
    validate(cur, 0);
    validate(nxt, 1);

    // The chunks of this workgroup's items form one sequence, g = 0, 1, ...:
    // chunk g goes to buffer g % NBUF, and its P and flags to parity g & 1.
    // One barrier per chunk. Before the barrier of chunk g each wavefront has
    // written its share of P(g) and waited for its own gathers of chunk g + 1;
    // after it, chunk g + 1 is visible to all and every wavefront is past the
    // values of chunk g - 1, so chunk g + 3 (of this item or the next) is
    // gathered into that chunk's buffer. P and the flags alternate between two
    // buffers, so a wavefront writing those of chunk g + 1 cannot overwrite
    // what a slower one still reads of chunk g. At the end of an item the
    // next item's Q, taken after the last score phase, and its successor's
    // row indices are waited for, once: the next item's first three chunks
    // have landed by then, so its first two waits are skipped (they would
    // wait for the output stores issued after). Waits count gathers, five
    // per chunk.
    for (int c = 0; c < NBUF - 1 && c < nchunk; ++c) {
        int e[4];
        rows_of(cur, c, e);
        issue(cp.cache, e, c);
    }
    if (nchunk >= 3) wait_vm<10>();
    else if (nchunk == 2) wait_vm<5>();
    else wait_vm<0>();
    __syncthreads();  // chunk 0 and the validity bits visible

    int g = 0;
    int par = 0;  // item parity of the validity bits
    bool fresh = false;
    for (long long n = first;;) {
        const bool more = n + 1 < end;
        const bool carry = more && nchunk >= NBUF - 1;  // the ring runs on into the next item
        f32x4 o[4][4];  // [head tile][value tile 4 wid + j]
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j) o[a][j] = f32x4{};
        float m_run[4];  // running max of heads 16 a + lane % 16, log2 domain
#pragma unroll
        for (int a = 0; a < 4; ++a) m_run[a] = -INFINITY;
        float l_part = 0.0f;  // sum of P over this wavefront's keys (tile kt), head 16 ht + lane % 16

        for (int c = 0; c < nchunk; ++c, ++g) {
            const int b = g & (NBUF - 1), pb = g & 1;

            // scores of key tile kt x head tile ht
            f32x4 s = f32x4{};
            {
                const int r = kt * 16 + (lane & 15);
                const uint4 *hr = &sm.head[b][r * MAIN16];
                const uint4 *tr = &sm.tail[b][r * TAIL16];
                // Each MFMA group runs at raised wavefront priority, so the other
                // wavefront of the SIMD fills the matrix pipe's gaps with its
                // VALU work instead of delaying the next MFMA (2% on the bench).
                __builtin_amdgcn_s_setprio(1);
                // The fragment reads run three ahead of the MFMAs, so their
                // LDS latency stays hidden behind the chain; scheduling
                // barriers keep that order under register pressure.
                // Piece 4 ks + lane / 16 of the row, swizzled: for k-step
                // 4a + c (a, c < 4) that is piece 16a + ((4c + lane / 16) ^
                // (r & 15)), so the four k-steps of each c share one address
                // and differ by an immediate offset.
                auto frag = [&](int ks) {
                    const int q = lane >> 4;
                    return ks < 16 ? hr[((4 * (ks & 3) + q) ^ (r & 15)) + 16 * (ks >> 2)]
                                   : tr[(4 * (ks - 16) + q) ^ (r & 7)];
                };
                uint4 v0 = frag(0), v1 = frag(1), v2 = frag(2);
                // In an item's last chunk, when the ring runs on, each Q
                // fragment of the next item is loaded as soon as the MFMA that
                // used this item's has been issued.
                const bool nextq = c == nchunk - 1 && carry;
                const bf16x8 *qn = q_ptr(np);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < NQK; ++ks) {
                    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v0), qf[ks], s, 0, 0, 0);
                    if (nextq) qf[ks] = qn[ks * 4];
                    v0 = v1;
                    v1 = v2;
                    if (ks + 3 < NQK) v2 = frag(ks + 3);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_s_setprio(0);
            const uint32_t vb = sm.validb[par][c][4 * kt + (lane >> 4)];  // keys kt * 16 + 4 (lane / 16) + i
            float z[4], mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[i] = (vb >> i) & 1u ? s[i] * scale_log2 : -INFINITY;
                mx = fmaxf(mx, z[i]);
            }
            mx = quad_max(mx);
            if (lane < 16) sm.pmax[kt][ht * 16 + lane] = mx;

            // Lazy rescaling: a head keeps its running max until a chunk's max
            // exceeds it by more than RESCALE_LOG2, so the probabilities stay
            // below 2^RESCALE_LOG2 (exact in fp32; bf16 keeps its relative
            // precision) and O is rescaled only when some head's max jumps, in
            // practice after the first chunk only. So P is first formed against
            // the running max, which every wavefront holds alike, with no
            // exchange; a wavefront that sees one of its heads jump raises a
            // flag, and only then do all wavefronts exchange the chunk maxima,
            // form P again and rescale.
            float m_ht = m_run[0];
#pragma unroll
            for (int a = 1; a < 4; ++a) m_ht = ht == a ? m_run[a] : m_ht;
            if (lane == 0) sm.jump[pb][wid] = wave_ballot(mx > m_ht + RESCALE_LOG2) != 0 ? 1 : 0;
            float pr[4], ps = 0.0f;
            {
                const float mu = m_ht == -INFINITY ? 0.0f : m_ht;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i] = exp2_fast(z[i] - mu);
                    ps += pr[i];
                }
            }
            *reinterpret_cast<uint2 *>(&sm.p[pb][ht][lane][kt * 4]) =
                make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
            if (c == nchunk - 1 && carry) {
                wait_vm<5 + NQK>();  // the next item's Q loads were issued after chunk g + 2's gathers
            } else if (!fresh || c >= 2) {
                if (c + 2 < nchunk || carry) wait_vm<5>();
                else wait_vm<0>();
            }
            __syncthreads();
            {
                const bool own = c + NBUF - 1 < nchunk;
                if (own || carry) {
                    int e[4], en[4];
                    rows_of(cur, c + NBUF - 1, e);
                    rows_of(nxt, c + NBUF - 1 - nchunk, en);
#pragma unroll
                    for (int j = 0; j < 4; ++j) e[j] = own ? e[j] : en[j];
                    issue(own ? cp.cache : np.cache, e, (g + NBUF - 1) & (NBUF - 1));
                }
            }
            if (c == nchunk - 1 && carry) {
                // The row indices of the item after next are loaded now, and
                // they and the next item's Q (loaded during the scores) are
                // waited for at the end of the item.
#pragma unroll
                for (int j = 0; j < 4; ++j) cur[j] = nxt[j];
                load_sel(n + 2 < end ? advance(np).row : np.row, nxt);
            }

            if (*reinterpret_cast<const uint64_t *>(sm.jump[pb]) != 0) {  // the same answer in every wavefront
                float m_new[4], m_use[4], alpha[4];
                bool moved = false;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int hh = a * 16 + (lane & 15);
                    const float cm = fmaxf(sm.pmax[0][hh], sm.pmax[1][hh]);
                    const bool up = cm > m_run[a] + RESCALE_LOG2;  // always, from -inf, once a key is valid
                    m_new[a] = up ? cm : m_run[a];
                    m_use[a] = m_new[a] == -INFINITY ? 0.0f : m_new[a];
                    alpha[a] = up ? exp2_fast(m_run[a] - m_use[a]) : 1.0f;
                    moved = moved || up;
                }
                float mu = m_use[0], al = alpha[0];
#pragma unroll
                for (int a = 1; a < 4; ++a) {
                    mu = ht == a ? m_use[a] : mu;
                    al = ht == a ? alpha[a] : al;
                }
                ps = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i] = exp2_fast(z[i] - mu);
                    ps += pr[i];
                }
                l_part *= al;
                *reinterpret_cast<uint2 *>(&sm.p[pb][ht][lane][kt * 4]) =
                    make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
#pragma unroll
                for (int a = 0; a < 4; ++a) m_run[a] = m_new[a];
                if (wave_ballot(moved)) {  // a head's running max rose: rescale
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int i = 0; i < 4; ++i) o[a][j][i] *= alpha[a];
                }
                __syncthreads();  // P formed again; maxima and flags read
            }
            l_part += quad_sum(ps);
            // Value fragments (each 8 keys of one dim column, read from the raw
            // rows) one tile ahead of the MFMAs that use them; the four P
            // fragments are read once per chunk and kept in registers (reading
            // them for each value tile was 96 KB of LDS reads per chunk more:
            // 605 -> 585 us). Nothing spills, so no vector-memory instruction
            // but the gathers runs in this loop.
            const int ln = lane, g = lane >> 4, i16 = lane & 15;
            const int kr0 = 4 * g + (i16 >> 2), kr1 = kr0 + 16;  // the two key runs of lane group g
            // Transposed LDS reads: lane 4q + c of a 16-lane group points at 4
            // values (dims dv0 + 4c ..) of key 4g + q (then 16 + 4g + q), and
            // lane i of the group receives dim dv0 + i of those 4 keys.
            auto vfrag = [&](int j) {
                const int col = (4 * wid + j) * 16 + 4 * (i16 & 3);
                auto trv = [&](int key) {
                    const char *p = reinterpret_cast<const char *>(&sm.head[b][key * MAIN16 + ((col >> 3) ^ (key & 15))]) +
                                    (col & 7) * 2;
                    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p);
                };
                const v4s lo = trv(kr0), hi = trv(kr1);
                return bf16x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            };
            bf16x8 pf[4];  // the chunk's P fragments, read once for the four value tiles
#pragma unroll
            for (int a = 0; a < 4; ++a) pf[a] = *reinterpret_cast<const bf16x8 *>(&sm.p[pb][a][ln][0]);
            bf16x8 va = vfrag(0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 vn = j + 1 < 4 ? vfrag(j + 1) : va;
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    o[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[a], o[a][j], 0, 0, 0);
                __builtin_amdgcn_s_setprio(0);
                va = vn;
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // The two key tiles' sums of each head, added once.
        if (lane < 16) sm.psum[kt][ht * 16 + lane] = l_part;
        __syncthreads();
        float l_run[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) l_run[a] = sm.psum[0][a * 16 + (lane & 15)] + sm.psum[1][a * 16 + (lane & 15)];
        if (carry) {
            wait_vm<0>();
#pragma unroll
            for (int ks = 0; ks < NQK; ++ks) asm volatile("" : "+v"(qf[ks]));
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(nxt[j]));
            validate(nxt, par);  // the item after next; this item's bits are no longer read
        }

        // O^T tile (value tile 4 wid + j, head tile a): lane holds head 16 a +
        // lane % 16 and value dims 16 (4 wid + j) + 4 (lane / 16) .. +3.
        const long long row = cp.row;
        const int h0 = cp.tile * AH;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const float inv = l_run[a] > 0.0f ? 1.0f / l_run[a] : 0.0f;
            const long long orow = (row * H + h0 + a * 16 + (lane & 15)) * DV;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int dv = (4 * wid + j) * 16 + 4 * (lane >> 4);
                *reinterpret_cast<uint2 *>(&O[orow + dv]) = make_uint2(pack_bf16x2(o[a][j][0] * inv, o[a][j][1] * inv),
                                                                        pack_bf16x2(o[a][j][2] * inv, o[a][j][3] * inv));
            }
            if (lse && wid == 0 && lane < 16)
                lse[row * H + h0 + a * 16 + lane] =
                    l_run[a] > 0.0f ? (m_run[a] + log2f(l_run[a])) * 0.69314718055994530942f : -INFINITY;
        }
        if (!more) break;
        if (!carry) {
            // Items of fewer than NBUF - 1 chunks: the next one starts as the
            // first did (its bits go to the other parity, whose item is done).
            load_sel(np.row, cur);
            load_q(np);
            wait_vm<0>();
#pragma unroll
            for (int ks = 0; ks < NQK; ++ks) asm volatile("" : "+v"(qf[ks]));
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(cur[j]));
            validate(cur, par ^ 1);
            for (int c = 0; c < nchunk; ++c) {
                int e[4];
                rows_of(cur, c, e);
                issue(np.cache, e, (g + c) & (NBUF - 1));
            }
            if (nchunk == 2) wait_vm<5>();
            else wait_vm<0>();
            __syncthreads();  // its chunk 0 and validity bits visible
        }
        ++n;
        cp = np;
        np = advance(np);
        par ^= 1;
        fresh = carry;
    }
}

}  // namespace

hipError_t launch_sparse_attention(const AttnProblem &p, const void *Q, const void *KV, const int *idx, void *O,
                                   float *lse, hipStream_t st)
{
    const float scale_log2 = (float)((double)p.softmax_scale * 1.4426950408889634);
    const long long items = (long long)p.B * p.T * (p.H / AH);
    // One workgroup per CU (the LDS ring allows no more), each walking its
    // items, with the gather ring carried from one item into the next.
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const long long grid = cus > 0 && cus < items ? cus : items;
    hipLaunchKernelGGL(sparse_attention_kernel, dim3((unsigned)grid), dim3(ATHREADS), 0, st,
                       static_cast<const uint16_t *>(Q), static_cast<const uint16_t *>(KV), idx, p.T, p.S, p.H, p.topk,
                       items, scale_log2, static_cast<uint16_t *>(O), lse);
    return hipGetLastError();
}

}  // namespace ds4idx
