// Wavefront-level exact selection over order-preserving 32-bit score keys
// held in registers (C keys per lane; key 0 = no key, below every finite
// score's key). Shared by the prefill and split-key kernels.
#pragma once

#include "device_common.h"

namespace ds4idx {

// Histogram of the digit (u >> lo) & dmask over keys matching (prefix, pmask)
// in the 256-bin LDS array `hist`, then the bin holding the `want`-th largest
// matching key. Returns the bin; `above_cnt` = matching keys in higher bins.
template <int C>
__device__ __forceinline__ uint32_t wave_digit(const uint32_t (&u)[C], uint32_t prefix,
                                               uint32_t pmask, int lo, uint32_t dmask,
                                               uint32_t want, uint32_t *hist, int lane,
                                               uint32_t &above_cnt)
{
    for (int b = lane; b < 256; b += 64) hist[b] = 0;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < C; ++j)
        if (u[j] != 0u && (u[j] & pmask) == prefix) atomicAdd(&hist[(u[j] >> lo) & dmask], 1u);
    wave_lds_sync();
    uint32_t c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) c[q] = hist[4 * lane + q];
    const uint32_t tot = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_scan_incl(tot, 0u, OpAdd{});
    uint32_t abv = wave_total(incl) - incl, mine = 0;  // keys in the bins of higher lanes
    int found = -1;
#pragma unroll
    for (int q = 3; q >= 0; --q) {
        if (found < 0 && abv < want && want <= abv + c[q]) {
            found = q;
            mine = abv;
        }
        abv += c[q];
    }
    const int src = __builtin_ctzll(wave_ballot(found >= 0));
    above_cnt = (uint32_t)wave_readlane((int)mine, src);
    const uint32_t bin = (uint32_t)(4 * src + wave_readlane(found, src));
    wave_lds_sync();
    return bin;
}

// The exact k-th largest key among the wavefront's keys (more than k keys
// present). Digit by digit: each pass takes the AND and OR of the keys still
// in play and starts its 8-bit window at their highest differing bit, so
// shared high bits cost no pass. `ties` = how many keys equal to the result
// belong to the top k (the lowest-index ones, by the caller's order).
template <int C>
__device__ uint32_t wave_kth_key(const uint32_t (&u)[C], uint32_t k, uint32_t *hist, int lane,
                                 uint32_t &ties)
{
    uint32_t prefix = 0, pmask = 0, remaining = k;
    while (pmask != ~0u) {
        uint32_t a = ~0u, o = 0u;
#pragma unroll
        for (int j = 0; j < C; ++j)
            if (u[j] != 0u && (u[j] & pmask) == prefix) {
                a &= u[j];
                o |= u[j];
            }
        a = wave_and(a);
        o = wave_or(o);
        const uint32_t diff = (a ^ o) & ~pmask;
        if (diff == 0u) {  // every key still in play is equal: that is the k-th
            prefix = a;
            break;
        }
        const int hb = 31 - __builtin_clz(diff);
        const uint32_t above = hb == 31 ? 0u : (~0u << (hb + 1));
        prefix = (prefix & pmask) | (a & above & ~pmask);
        pmask |= above;
        const int lo = hb >= 7 ? hb - 7 : 0;
        const uint32_t dmask = (2u << (hb - lo)) - 1u;
        uint32_t higher;
        const uint32_t bin = wave_digit<C>(u, prefix, pmask, lo, dmask, remaining, hist, lane, higher);
        remaining -= higher;
        prefix |= bin << lo;
        pmask |= dmask << lo;
    }
    ties = remaining;
    return prefix;
}

}  // namespace ds4idx
