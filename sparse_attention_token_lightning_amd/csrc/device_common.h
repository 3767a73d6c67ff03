// Device helpers shared by the HIP kernels: the order-preserving score key and
// wavefront (64-lane) mask arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ds4idx {

// Scores are compared through a 32-bit key that orders like the float. The
// score is first canonicalised with +0.0f so that -0.0 and +0.0 (both arise:
// a negative head weight times a zero ReLU gives -0.0) map to the same key and
// therefore tie, leaving the decision to the index rule.
__device__ __forceinline__ float canon(float x) { return x + 0.0f; }

__device__ __forceinline__ uint32_t ord_key(float x)
{
    uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t o)
{
    uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of m in lanes below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int wave_readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Inclusive scan across the 64 lanes with DPP moves (row shifts by 1, 2, 4, 8
// within each 16-lane row, then row broadcasts of lanes 15 and 31): a few
// VALU operations instead of a chain of LDS-crossbar permutes. `id` is the
// identity of `op`; lane 63 ends with the reduction of the whole wavefront.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v, uint32_t id, Op op)
{
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xf, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xa, 0xf, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xc, 0xf, false));
    return v;
}

struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpAnd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a & b; } };
struct OpOr { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };

__device__ __forceinline__ uint32_t wave_total(uint32_t incl) { return (uint32_t)__builtin_amdgcn_readlane((int)incl, 63); }
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return wave_total(wave_scan_incl(v, 0u, OpAdd{})); }
__device__ __forceinline__ uint32_t wave_and(uint32_t v) { return wave_total(wave_scan_incl(v, ~0u, OpAnd{})); }
__device__ __forceinline__ uint32_t wave_or(uint32_t v) { return wave_total(wave_scan_incl(v, 0u, OpOr{})); }
__device__ __forceinline__ uint32_t wave_min(uint32_t v) { return wave_total(wave_scan_incl(v, ~0u, OpMin{})); }
__device__ __forceinline__ uint32_t wave_max(uint32_t v) { return wave_total(wave_scan_incl(v, 0u, OpMax{})); }

// Orders this wavefront's LDS accesses before and after the call.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Exact OCP E4M3FN decode by bit fields (sign, exponent bias 7, 3-bit
// mantissa, exponent 0 subnormal, S.1111.111 NaN). Used by the plain kernels.
__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v;
    if (e == 15u && m == 7u)
        v = __uint_as_float(0x7fc00000u);
    else if (e == 0u)
        v = ldexpf((float)m, -9);
    else
        v = ldexpf((float)(8u + m), (int)e - 10);
    return (c & 0x80u) ? -v : v;
}

__device__ __forceinline__ float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace ds4idx
