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

// Device-scope (agent) relaxed stores and loads: the candidate lists that one
// workgroup publishes and another, on any XCD, merges after an arrival
// counter (global_store / global_load with sc1 on gfx950).
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

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) void *)p;
}

// One 16-byte load per lane straight into LDS (global_load_lds_dwordx4) from
// a wavefront-uniform base in scalar registers plus a 32-bit per-lane byte
// offset: lane i's bytes land at LDS address lds + 16 i (lds wavefront-
// uniform, carried in M0). Issued as inline assembly so that the compiler
// does not treat it as an LDS store that it must drain (vmcnt(0)) before every
// later LDS read; the caller awaits completion with wait_vm, counting these
// loads itself.
__device__ __forceinline__ void gather16_at(const void *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

// A pointer that is the same in every lane, moved to scalar registers (the
// base operand of gather16_at).
template <class T>
__device__ __forceinline__ const T *uniform_ptr(const T *p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return reinterpret_cast<const T *>(((uint64_t)hi << 32) | lo);
}

// Wait until at most N of this wavefront's vector-memory operations are
// outstanding (expcnt and lgkmcnt left free).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
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

// Ragged batches: stream b owns query rows cu_q[b] .. cu_q[b+1]-1 and key rows
// cu_k[b] .. cu_k[b+1]-1 (prefix arrays in device memory). Query t of the
// stream sees its keys s <= S - T + t: the new tokens are the last T cached.
// The bounds are clamped to [0, total] and made non-decreasing, so malformed
// arrays give wrong rows but no access outside the caller's buffers.
struct Ragged {
    const int *cu_q;        // [B + 1]
    const long long *cu_k;  // [B + 1]
    int B, total_q;
    long long total_k;
};

struct StreamGeo {
    long long q0;  // first query row
    long long k0;  // first key row
    int T;         // query rows
    long long S;   // cached keys
};

__device__ __forceinline__ StreamGeo stream_geo(const int *cu_q, const long long *cu_k, int b,
                                                int total_q, long long total_k)
{
    auto clampq = [&](int v) { return v < 0 ? 0 : (v > total_q ? total_q : v); };
    auto clampk = [&](long long v) { return v < 0 ? 0 : (v > total_k ? total_k : v); };
    const int qa = clampq(cu_q[b]), qb = clampq(cu_q[b + 1]);
    const long long ka = clampk(cu_k[b]), kb = clampk(cu_k[b + 1]);
    StreamGeo g;
    g.q0 = qa;
    g.T = qb > qa ? qb - qa : 0;
    g.k0 = ka;
    g.S = kb > ka ? kb - ka : 0;
    return g;
}

// The stream holding query row r (the first whose clamped range holds it), by
// a wavefront scan of 64 streams per step; -1 if none. Wave-uniform result.
__device__ __forceinline__ int wave_row_stream(const int *cu_q, const long long *cu_k, int B,
                                               int total_q, long long total_k, long long r, int lane)
{
    for (int c = 0; c < B; c += 64) {
        const int s = c + lane;
        bool hit = false;
        if (s < B) {
            const StreamGeo g = stream_geo(cu_q, cu_k, s, total_q, total_k);
            hit = r >= g.q0 && r < g.q0 + g.T;
        }
        const uint64_t m = wave_ballot(hit);
        if (m) return c + __builtin_ctzll(m);
    }
    return -1;
}

// Parts a stream's key range is split into when blocks take at most kpart
// keys each (kpart = 0: one part). At most `maxp`.
__device__ __forceinline__ int stream_parts(long long S, int kpart, int maxp)
{
    if (kpart <= 0 || S <= kpart) return 1;
    const long long n = (S + kpart - 1) / kpart;
    return (int)(n < maxp ? n : maxp);
}

// Block x of a grid giving each stream ceil(min(T, S) / tq) * parts blocks
// (parts from stream_parts(S, kpart, maxp)), streams in order: returns the
// stream (-1 past the last block) and sets j, the block's index within the
// stream. Wave-uniform result.
__device__ __forceinline__ int wave_block_stream(const int *cu_q, const long long *cu_k, int B,
                                                 int total_q, long long total_k, int tq, long long x,
                                                 int lane, int &j, int kpart = 0, int maxp = 1)
{
    long long base = 0;
    for (int c = 0; c < B; c += 64) {
        const int s = c + lane;
        uint32_t nb = 0;
        if (s < B) {
            const StreamGeo g = stream_geo(cu_q, cu_k, s, total_q, total_k);
            const long long t = (long long)g.T < g.S ? (long long)g.T : g.S;
            nb = (uint32_t)((t + tq - 1) / tq) * (uint32_t)stream_parts(g.S, kpart, maxp);
        }
        const uint32_t incl = wave_scan_incl(nb, 0u, OpAdd{});
        const long long lo = base + (long long)(incl - nb), hi = base + (long long)incl;
        const uint64_t m = wave_ballot(s < B && x >= lo && x < hi);
        if (m) {
            const int src = __builtin_ctzll(m);
            j = (int)(x - base - (long long)(uint32_t)wave_readlane((int)(incl - nb), src));
            return c + src;
        }
        base += wave_total(incl);
    }
    return -1;
}

}  // namespace ds4idx
