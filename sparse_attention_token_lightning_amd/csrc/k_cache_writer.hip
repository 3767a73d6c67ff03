// Indexer key-cache writer: per-token OCP E4M3FN quantisation of new key
// vectors, one fp32 scale per token, stored into rows of the key cache that the
// scorer reads. The indexer's cache holds E4M3 codes, and the MI300X write-up
// ("DeepSeek V4 Flash는 단일 AMD MI300X에서 실행됩니다", FP8 format mismatch
// section) shows what reading one E4M3 variant as the other costs: a factor 2
// on every key. gfx950's conversion instructions produce the OCP variant.
//
//   scale = max(amax, 2^-126) / 448           (fp32, correctly rounded division)
//   code  = E4M3 RNE of clamp(k / scale, -448, 448)
//
// HBM-bound: a token of D values is spread over the lanes of one wavefront, 16
// (or 8) values per lane, so loads and code stores are 16-byte (8-byte) vectors
// contiguous across the wavefront.
#include "device_common.h"
#include "kernels.h"

namespace ds4idx {
namespace {

constexpr int kWriterThreads = 256;

template <int V>
__device__ __forceinline__ void load_vals(const float *p, float (&x)[V])
{
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
        const float4 a = reinterpret_cast<const float4 *>(p)[j];
        x[4 * j] = a.x; x[4 * j + 1] = a.y; x[4 * j + 2] = a.z; x[4 * j + 3] = a.w;
    }
}

template <int V>
__device__ __forceinline__ void load_vals(const uint16_t *p, float (&x)[V])
{
#pragma unroll
    for (int j = 0; j < V / 8; ++j) {
        const uint4 v = reinterpret_cast<const uint4 *>(p)[j];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[8 * j + 2 * i] = __uint_as_float(w[i] << 16);
            x[8 * j + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

// q[i] = x[i] / sc, correctly rounded. A division per element is the largest
// cost of this kernel, so for sc >= 2^-80 it takes one correctly rounded
// reciprocal y per lane and two residual corrections per element, r = x - sc*q
// (exact in an fma) and q + r*y: Markstein's final steps (P. Markstein, IBM J.
// Res. Dev. 34(1), 1990), which give the correctly rounded quotient when no
// intermediate underflows. With sc >= 2^-80 a quotient that can round to a
// nonzero E4M3 code (|q| >= 2^-10) has |x| >= 2^-90, so the residuals stay
// normal; smaller quotients encode to a signed zero either way, and the sign is
// taken from x. Tokens with a smaller scale divide directly.
template <int V>
__device__ __forceinline__ void quotients(const float (&x)[V], float sc, float (&q)[V])
{
    if (sc >= 0x1p-80f) {
        const float y = 1.0f / sc;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const float q0 = x[i] * y;
            const float r0 = __builtin_fmaf(-sc, q0, x[i]);
            const float q1 = __builtin_fmaf(r0, y, q0);
            const float r1 = __builtin_fmaf(-sc, q1, x[i]);
            q[i] = __builtin_copysignf(__builtin_fmaf(r1, y, q1), x[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) q[i] = x[i] / sc;
    }
}

// V values per lane, G lanes per token (G divides 64, so a token's lanes share
// a wavefront). V = 16 (16-byte code stores) when D is a multiple of 16 and the
// cache rows are 16-byte aligned, else V = 8.
template <class In, int V>
__global__ __launch_bounds__(kWriterThreads) void k_cache_write_kernel(
    const In *__restrict__ kin, long long n, int D, int G, const long long *__restrict__ slots,
    uint8_t *__restrict__ cache, float *__restrict__ cache_scale, long long rows)
{
    const long long gt = (long long)blockIdx.x * kWriterThreads + threadIdx.x;
    const long long tok = gt / G;
    const int d0 = (int)(gt % G) * V;
    const bool live = tok < n && d0 < D;
    float x[V];
    if (live) {
        load_vals<V>(kin + tok * D + d0, x);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) x[i] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) m = fmaxf(m, fabsf(x[i]));
    for (int o = 1; o < G; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (!live) return;
    const long long slot = slots ? slots[tok] : tok;
    if (slot < 0 || slot >= rows) return;

    const float sc = fmaxf(m, 0x1p-126f) / 448.0f;
    float q[V];
    quotients<V>(x, sc, q);
#pragma unroll
    for (int i = 0; i < V; ++i) q[i] = fminf(fmaxf(q[i], -448.0f), 448.0f);
    // Round to nearest even into OCP E4M3; src0 goes to the lower byte of the
    // selected 16-bit half, src1 to the upper byte.
    uint32_t w[V / 4];
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * j], q[4 * j + 1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * j + 2], q[4 * j + 3], v, true);
        w[j] = (uint32_t)v;
    }
    uint8_t *dst = cache + slot * D + d0;
    if constexpr (V == 16)
        *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    else
        *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
    if (d0 == 0) cache_scale[slot] = sc;
}

template <class In, int V>
void launch_v(const In *kin, long long n, int D, const long long *slots, uint8_t *cache,
              float *cache_scale, long long rows, hipStream_t st)
{
    const int G = k_cache_lanes(D, V);
    const long long blocks = (n * G + kWriterThreads - 1) / kWriterThreads;
    hipLaunchKernelGGL((k_cache_write_kernel<In, V>), dim3((unsigned)blocks), dim3(kWriterThreads), 0, st,
                       kin, n, D, G, slots, cache, cache_scale, rows);
}

}  // namespace

int k_cache_lanes(int D, int V)
{
    int g = 1;
    while (g * V < D) g <<= 1;
    return g;
}

int k_cache_vals_per_lane(int D, const void *cache)
{
    return (D % 16 == 0 && reinterpret_cast<uintptr_t>(cache) % 16 == 0) ? 16 : 8;
}

hipError_t launch_k_cache_write(const void *kin, int k_dtype, long long n, int D,
                                const long long *slots, uint8_t *cache, float *cache_scale,
                                long long rows, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    const bool v16 = k_cache_vals_per_lane(D, cache) == 16;
    if (k_dtype == F32) {
        const float *k = static_cast<const float *>(kin);
        if (v16) launch_v<float, 16>(k, n, D, slots, cache, cache_scale, rows, st);
        else launch_v<float, 8>(k, n, D, slots, cache, cache_scale, rows, st);
    } else {
        const uint16_t *k = static_cast<const uint16_t *>(kin);
        if (v16) launch_v<uint16_t, 16>(k, n, D, slots, cache, cache_scale, rows, st);
        else launch_v<uint16_t, 8>(k, n, D, slots, cache, cache_scale, rows, st);
    }
    return hipGetLastError();
}

}  // namespace ds4idx
