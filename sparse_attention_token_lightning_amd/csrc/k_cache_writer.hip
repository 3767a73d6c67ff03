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
// HBM-bound: a token of D values is spread over G = D/8 (rounded up to a power
// of two) lanes of one wavefront, 8 values per lane, so loads are 16-byte
// vectors and stores 8-byte vectors, contiguous across a wavefront.
#include "device_common.h"
#include "kernels.h"

namespace ds4idx {
namespace {

constexpr int kWriterThreads = 256;

__device__ __forceinline__ void load8(const float *p, float (&x)[8])
{
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void load8(const uint16_t *p, float (&x)[8])
{
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

template <class In>
__global__ __launch_bounds__(kWriterThreads) void k_cache_write_kernel(
    const In *__restrict__ kin, long long n, int D, int G, const long long *__restrict__ slots,
    uint8_t *__restrict__ cache, float *__restrict__ cache_scale, long long rows)
{
    // G divides 64, so the G lanes of a token sit in one wavefront.
    const long long gt = (long long)blockIdx.x * kWriterThreads + threadIdx.x;
    const long long tok = gt / G;
    const int d0 = (int)(gt % G) * 8;
    const bool live = tok < n && d0 < D;
    float x[8];
    if (live) {
        load8(kin + tok * D + d0, x);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
    for (int o = 1; o < G; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (!live) return;
    const long long slot = slots ? slots[tok] : tok;
    if (slot < 0 || slot >= rows) return;

    const float sc = fmaxf(m, 0x1p-126f) / 448.0f;
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(x[i] / sc, -448.0f), 448.0f);
    // Round to nearest even into OCP E4M3; src0 goes to the lower byte of the
    // selected 16-bit half, src1 to the upper byte.
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
    *reinterpret_cast<uint2 *>(cache + slot * D + d0) = make_uint2((uint32_t)w0, (uint32_t)w1);
    if (d0 == 0) cache_scale[slot] = sc;
}

}  // namespace

int k_cache_lanes(int D)
{
    int g = 1;
    while (g * 8 < D) g <<= 1;
    return g;
}

hipError_t launch_k_cache_write(const void *kin, int k_dtype, long long n, int D,
                                const long long *slots, uint8_t *cache, float *cache_scale,
                                long long rows, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    const int G = k_cache_lanes(D);
    const long long blocks = (n * G + kWriterThreads - 1) / kWriterThreads;
    if (k_dtype == F32)
        hipLaunchKernelGGL(k_cache_write_kernel<float>, dim3((unsigned)blocks), dim3(kWriterThreads), 0, st,
                           static_cast<const float *>(kin), n, D, G, slots, cache, cache_scale, rows);
    else
        hipLaunchKernelGGL(k_cache_write_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kWriterThreads), 0,
                           st, static_cast<const uint16_t *>(kin), n, D, G, slots, cache, cache_scale, rows);
    return hipGetLastError();
}

}  // namespace ds4idx
