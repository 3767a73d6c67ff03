// Plain HIP kernels for any shape and dtype: the rollback path kept next to
// the MFMA kernels so that the two can be compared on the same inputs (the
// pages put every new indexer kernel behind such a switch: first page,
// practical advice, third paragraph).
//
//  * score_ref: one thread per (query, key); the query's H x D block and head
//    weights are staged in LDS; fp32 FMA accumulation over d, then
//    score = scale[s] * sum_h w[h] * max(0, dot_h).
//  * topk_ref: one 1024-thread workgroup per query row; exact radix selection
//    of the k-th largest score key over the row's visible prefix (four 8-bit
//    digit passes over an order-preserving 32-bit key), then one ordered pass
//    that keeps every score above the k-th and the lowest-index ties at it.
//    Output is ascending by index, so no sort is ever done.
#include "device_common.h"
#include "kernels.h"

namespace ds4idx {
namespace {

template <int DT>
__device__ __forceinline__ float load_elem(const void *p, long long i)
{
    if (DT == F32) return static_cast<const float *>(p)[i];
    if (DT == BF16) return bf16_value(static_cast<const uint16_t *>(p)[i]);
    return e4m3_value(static_cast<const uint8_t *>(p)[i]);
}

constexpr int kScoreThreads = 256;
constexpr int kKeysPerThread = 4;
constexpr int kKeysPerBlock = kScoreThreads * kKeysPerThread;
constexpr int kHeadGroup = 8;

template <int QT, int KT>
__global__ __launch_bounds__(kScoreThreads) void score_ref_kernel(Problem p, const void *Q,
                                                                   const void *K, const float *Ks,
                                                                   const float *W, float *scores,
                                                                   int key_blocks)
{
    extern __shared__ float smem[];
    const int H = p.H, D = p.D;
    float *qs = smem;
    float *ws = smem + H * D;
    const long long row = blockIdx.x / key_blocks;  // b * T + t
    const int kb = blockIdx.x % key_blocks;
    const int b = (int)(row / p.T), t = (int)(row % p.T);
    for (int i = threadIdx.x; i < H * D; i += kScoreThreads)
        qs[i] = load_elem<QT>(Q, row * H * D + i);
    for (int i = threadIdx.x; i < H; i += kScoreThreads)
        ws[i] = W[row * H + i];
    __syncthreads();
    const long long lim = p.offset + t;
    float *out = scores + row * p.S;
    for (int j = 0; j < kKeysPerThread; ++j) {
        const long long s = (long long)kb * kKeysPerBlock + j * kScoreThreads + threadIdx.x;
        if (s >= p.S) break;
        if (s > lim) {
            out[s] = -INFINITY;
            continue;
        }
        const long long kbase = ((long long)b * p.S + s) * D;
        float score = 0.0f;
        for (int h0 = 0; h0 < H; h0 += kHeadGroup) {
            float acc[kHeadGroup];
#pragma unroll
            for (int g = 0; g < kHeadGroup; ++g) acc[g] = 0.0f;
            for (int d = 0; d < D; ++d) {
                const float kv = load_elem<KT>(K, kbase + d);
#pragma unroll
                for (int g = 0; g < kHeadGroup; ++g)
                    if (h0 + g < H) acc[g] = fmaf(qs[(h0 + g) * D + d], kv, acc[g]);
            }
#pragma unroll
            for (int g = 0; g < kHeadGroup; ++g)
                if (h0 + g < H) score = fmaf(ws[h0 + g], fmaxf(acc[g], 0.0f), score);
        }
        if (KT == FP8) score *= Ks[(long long)b * p.S + s];
        out[s] = canon(score);
    }
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Block-wide exclusive prefix count of `flag`; `total` gets the block sum.
__device__ __forceinline__ uint32_t block_excl_count(bool flag, uint32_t *wave_counts,
                                                     uint32_t &total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const uint64_t m = wave_ballot(flag);
    if (lane == 0) wave_counts[wid] = (uint32_t)__builtin_popcountll(m);
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
        const uint32_t c = wave_counts[w];
        before += (w < wid) ? c : 0u;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + lanes_below(m);
}

__global__ __launch_bounds__(kTopkThreads) void topk_ref_kernel(Problem p, const float *scores,
                                                                int k, int *idx, float *vals)
{
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wave_counts[kTopkWaves];
    __shared__ uint32_t pick[2];
    const long long row = blockIdx.x;
    const int t = (int)(row % p.T);
    const long long L = p.offset + t + 1;
    const float *sr = scores + row * p.S;
    int *io = idx + row * k;
    float *vo = vals ? vals + row * k : nullptr;
    const int tid = threadIdx.x, lane = tid & 63;

    const bool keep_all = L <= k;
    uint32_t tau = 0, ties_wanted = 0;
    if (!keep_all) {
        uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)k;
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            for (long long i = tid; i < L; i += kTopkThreads) {
                const uint32_t u = ord_key(canon(sr[i]));
                if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid < 64) {
                // Lane l owns bins 4l..4l+3; find the bin, scanning from the
                // top, where the count of larger keys reaches `remaining`.
                uint32_t c[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) c[q] = hist[4 * lane + q];
                const uint32_t tot = c[0] + c[1] + c[2] + c[3];
                uint32_t suf = tot;
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t y = __shfl_down(suf, off);
                    if (lane + off < 64) suf += y;
                }
                uint32_t above = suf - tot;
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
                const uint64_t fm = wave_ballot(found >= 0);
                const int src = __builtin_ctzll(fm);
                if (lane == src) {
                    pick[0] = (uint32_t)(4 * lane + found);
                    pick[1] = rem;
                }
            }
            __syncthreads();
            prefix |= pick[0] << shift;
            pmask |= 0xffu << shift;
            remaining = pick[1];
            __syncthreads();
        }
        tau = prefix;
        ties_wanted = remaining;
    }

    uint32_t out_base = 0, tie_base = 0;
    for (long long base = 0; base < L; base += kTopkThreads) {
        const long long i = base + tid;
        const bool in = i < L;
        const float sv = in ? canon(sr[i]) : 0.0f;
        const uint32_t u = ord_key(sv);
        const bool eq = in && !keep_all && u == tau;
        uint32_t eq_total;
        const uint32_t eq_rank = block_excl_count(eq, wave_counts, eq_total);
        const bool keep = in && (keep_all || u > tau || (eq && tie_base + eq_rank < ties_wanted));
        uint32_t keep_total;
        const uint32_t pos = out_base + block_excl_count(keep, wave_counts, keep_total);
        if (keep && pos < (uint32_t)k) {
            io[pos] = (int)i;
            if (vo) vo[pos] = sv;
        }
        out_base += keep_total;
        tie_base += eq_total;
    }
    for (int j = (int)out_base + tid; j < k; j += kTopkThreads) {
        io[j] = -1;
        if (vo) vo[j] = -INFINITY;
    }
}

template <int QT, int KT>
hipError_t launch_score_ref_t(const Problem &p, const void *Q, const void *K, const float *Ks,
                              const float *W, float *scores, hipStream_t st)
{
    const int key_blocks = (p.S + kKeysPerBlock - 1) / kKeysPerBlock;
    const long long blocks = (long long)p.B * p.T * key_blocks;
    const size_t lds = (size_t)(p.H * p.D + p.H) * sizeof(float);
    hipLaunchKernelGGL((score_ref_kernel<QT, KT>), dim3((unsigned)blocks), dim3(kScoreThreads), lds,
                       st, p, Q, K, Ks, W, scores, key_blocks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_score_ref(const Problem &p, const void *Q, const void *K, const float *Ks,
                            const float *W, float *scores, hipStream_t st)
{
    if (p.q_dtype == F32) {
        if (p.k_dtype == F32) return launch_score_ref_t<F32, F32>(p, Q, K, Ks, W, scores, st);
        if (p.k_dtype == BF16) return launch_score_ref_t<F32, BF16>(p, Q, K, Ks, W, scores, st);
        return launch_score_ref_t<F32, FP8>(p, Q, K, Ks, W, scores, st);
    }
    if (p.k_dtype == F32) return launch_score_ref_t<BF16, F32>(p, Q, K, Ks, W, scores, st);
    if (p.k_dtype == BF16) return launch_score_ref_t<BF16, BF16>(p, Q, K, Ks, W, scores, st);
    return launch_score_ref_t<BF16, FP8>(p, Q, K, Ks, W, scores, st);
}

hipError_t launch_topk_ref(const Problem &p, const float *scores, int k, int *idx, float *vals,
                           hipStream_t st)
{
    const long long rows = (long long)p.B * p.T;
    hipLaunchKernelGGL(topk_ref_kernel, dim3((unsigned)rows), dim3(kTopkThreads), 0, st, p,
                       scores, k, idx, vals);
    return hipGetLastError();
}

}  // namespace ds4idx
