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
// Layout on CDNA4. A 512-thread workgroup owns one query token and one tile of
// 64 heads; the selected rows stream through LDS in chunks of 32:
//  * Rows are gathered global -> registers (issued one chunk ahead) -> LDS,
//    twice: row-major for the scores and transposed (value dims x keys) for the
//    weighted sum, so that both contractions read 16-byte MFMA fragments.
//  * Scores transposed, S^T = C Q^T (v_mfma_f32_16x16x32_bf16, keys on M,
//    heads on N): wavefront w computes the 16-key x 16-head tile (w & 1,
//    w >> 1) over 18 k-steps of the 576 dims, with its 16 heads of Q resident
//    as B operands.
//  * Online softmax in the log2 domain: per-head chunk maxima and sums go
//    through LDS; every wavefront keeps the running max and sum of the heads
//    its outputs cover.
//  * The S^T accumulator already has the layout of a B operand of the value
//    contraction O^T = V^T P^T (lane = head, 4 consecutive keys per lane group)
//    under a fixed permutation of the 32 keys of a chunk; the transposed value
//    copy is stored in that permuted key order, so P needs no transpose.
//    Wavefront w owns value tiles 4w .. 4w+3 of all four head tiles: 16
//    accumulator tiles.
#include "device_common.h"
#include "kernels.h"

namespace ds4idx {
namespace {

constexpr int AH = kAttnHeadTile;  // heads per workgroup
constexpr int DQK = kAttnDqk, DV = kAttnDv;
constexpr int CK = 32;             // selected rows per chunk
constexpr int ATHREADS = 512;
constexpr int KSTR = DQK + 8;      // bf16 per LDS key row (16-byte aligned rows)
constexpr int VSTR = CK + 8;       // bf16 per LDS transposed value row
constexpr int NPIECE = DQK / 8;    // 16-byte pieces per cache row
constexpr int NQK = DQK / 32;      // k-steps of the score contraction

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

struct AttnSmem {
    uint16_t k[CK * KSTR];   // chunk rows, row-major
    uint16_t vt[DV * VSTR];  // value dims x keys (permuted order)
    uint16_t p[4][64][8];    // P^T B fragments per head tile and lane
    float pmax[2][AH];       // chunk maxima per key tile and head
    float psum[2][AH];
    int valid[CK];
};

// Key s of a chunk sits at position pos(s) of the permuted order: lane group
// g = (s % 16) / 4 of the score tile holds keys 4g..4g+3 of each 16-key tile,
// and a value-contraction fragment of group g takes those 8 keys.
__device__ __forceinline__ int perm_pos(int s) { return 8 * ((s & 15) >> 2) + 4 * (s >> 4) + (s & 3); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    // round to nearest even (inputs are finite probabilities in [0, 1])
    auto rne = [](float x) {
        const uint32_t u = __float_as_uint(x);
        return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    };
    return rne(a) | (rne(b) << 16);
}

__global__ __launch_bounds__(ATHREADS, 1) void sparse_attention_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ C, const int *__restrict__ idx, int T, int S,
    int H, int topk, float scale_log2, uint16_t *__restrict__ O, float *__restrict__ lse)
{
    __shared__ AttnSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const long long row = blockIdx.x;  // b * T + t
    const int h0 = blockIdx.y * AH;
    const uint16_t *Cb = C + (row / T) * (long long)S * DQK;
    const int *ir = idx + row * topk;
    const int kt = wid & 1, ht = wid >> 1;

    // Q^T fragments of head tile ht: head h0 + 16 ht + lane % 16, dims 32 ks + 8 (lane / 16) ..
    bf16x8 qf[NQK];
    {
        const bf16x8 *qp = reinterpret_cast<const bf16x8 *>(
            Q + ((row * H + h0 + ht * 16 + (lane & 15)) * DQK + (lane >> 4) * 8));
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks) qf[ks] = qp[ks * 4];
    }

    f32x4 o[4][4];  // [head tile][value tile 4 wid + j]
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[a][j] = f32x4{};
    float m_run[4], l_run[4];  // heads 16 a + lane % 16 of the tile, log2 domain
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        m_run[a] = -INFINITY;
        l_run[a] = 0.0f;
    }

    // Staging: lanes 0..31 and 32..63 of wavefront w take pieces 2w and 2w+1
    // (+16 j) of chunk row lane % 32.
    const int skey = lane & 31;
    uint4 stg[5];
    bool sok = false;
    auto prefetch = [&](int c) {
        const int j0 = c * CK + skey;
        const int s = j0 < topk ? ir[j0] : -1;
        sok = s >= 0 && s < S;
        const uint4 *src = reinterpret_cast<const uint4 *>(Cb + (long long)(sok ? s : 0) * DQK);
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int p = 2 * wid + (lane >> 5) + 16 * j;
            stg[j] = (sok && p < NPIECE) ? src[p] : make_uint4(0, 0, 0, 0);
        }
    };
    auto stage = [&]() {
        const int pos = perm_pos(skey);
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int p = 2 * wid + (lane >> 5) + 16 * j;
            if (p < NPIECE) {
                *reinterpret_cast<uint4 *>(&sm.k[skey * KSTR + p * 8]) = stg[j];
                if (p < DV / 8) {
                    const uint32_t w[4] = {stg[j].x, stg[j].y, stg[j].z, stg[j].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        sm.vt[(p * 8 + e) * VSTR + pos] = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : w[e >> 1]);
                }
            }
        }
        if (wid == 0 && lane < 32) sm.valid[lane] = sok ? 1 : 0;
    };

    const int nchunk = (topk + CK - 1) / CK;
    prefetch(0);
    for (int c = 0; c < nchunk; ++c) {
        stage();
        __syncthreads();
        if (c + 1 < nchunk) prefetch(c + 1);

        // scores of key tile kt x head tile ht
        f32x4 s = f32x4{};
        const uint16_t *kp = &sm.k[(kt * 16 + (lane & 15)) * KSTR + (lane >> 4) * 8];
#pragma unroll
        for (int ks = 0; ks < NQK; ++ks)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8 *>(kp + ks * 32), qf[ks],
                                                        s, 0, 0, 0);
        float z[4], mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kt * 16 + 4 * (lane >> 4) + i;
            z[i] = sm.valid[key] ? s[i] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, z[i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (lane < 16) sm.pmax[kt][ht * 16 + lane] = mx;
        __syncthreads();

        float m_new[4], m_use[4], alpha[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int hh = a * 16 + (lane & 15);
            m_new[a] = fmaxf(m_run[a], fmaxf(sm.pmax[0][hh], sm.pmax[1][hh]));
            m_use[a] = m_new[a] == -INFINITY ? 0.0f : m_new[a];
            alpha[a] = exp2f(m_run[a] - m_use[a]);
        }
        float pr[4], ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[i] = exp2f(z[i] - m_use[ht]);
            ps += pr[i];
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        if (lane < 16) sm.psum[kt][ht * 16 + lane] = ps;
        *reinterpret_cast<uint2 *>(&sm.p[ht][lane][kt * 4]) =
            make_uint2(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]));
        __syncthreads();

#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int hh = a * 16 + (lane & 15);
            l_run[a] = l_run[a] * alpha[a] + (sm.psum[0][hh] + sm.psum[1][hh]);
            m_run[a] = m_new[a];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[a][j][i] *= alpha[a];
        }
        bf16x8 pb[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) pb[a] = *reinterpret_cast<const bf16x8 *>(&sm.p[a][lane][0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 va =
                *reinterpret_cast<const bf16x8 *>(&sm.vt[((4 * wid + j) * 16 + (lane & 15)) * VSTR + (lane >> 4) * 8]);
#pragma unroll
            for (int a = 0; a < 4; ++a) o[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[a], o[a][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // O^T tile (value tile 4 wid + j, head tile a): lane holds head 16 a +
    // lane % 16 and value dims 16 (4 wid + j) + 4 (lane / 16) .. +3.
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const float inv = l_run[a] > 0.0f ? 1.0f / l_run[a] : 0.0f;
        const long long orow = (row * H + h0 + a * 16 + (lane & 15)) * DV;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int dv = (4 * wid + j) * 16 + 4 * (lane >> 4);
            *reinterpret_cast<uint2 *>(&O[orow + dv]) =
                make_uint2(pack_bf16x2(o[a][j][0] * inv, o[a][j][1] * inv), pack_bf16x2(o[a][j][2] * inv, o[a][j][3] * inv));
        }
        if (lse && wid == 0 && lane < 16)
            lse[row * H + h0 + a * 16 + lane] =
                l_run[a] > 0.0f ? (m_run[a] + log2f(l_run[a])) * 0.69314718055994530942f : -INFINITY;
    }
}

}  // namespace

hipError_t launch_sparse_attention(const AttnProblem &p, const void *Q, const void *KV, const int *idx, void *O,
                                   float *lse, hipStream_t st)
{
    const float scale_log2 = (float)((double)p.softmax_scale * 1.4426950408889634);
    hipLaunchKernelGGL(sparse_attention_kernel, dim3((unsigned)((long long)p.B * p.T), (unsigned)(p.H / AH)),
                       dim3(ATHREADS), 0, st, static_cast<const uint16_t *>(Q), static_cast<const uint16_t *>(KV), idx,
                       p.T, p.S, p.H, p.topk, scale_log2, static_cast<uint16_t *>(O), lse);
    return hipGetLastError();
}

}  // namespace ds4idx
