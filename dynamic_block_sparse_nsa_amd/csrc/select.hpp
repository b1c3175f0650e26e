// Group-shared top-n block selection, shared by the prefill and decode kernels.
//
// Rule (zjai.club notes, section 8: one top-k over group-summed scores; forced blocks
// and the lowest-index tie-break as documented in nsa.h): with jc the query's own block,
// blocks 0..n_init-1 and jc-n_local+1..jc are always kept; the remaining slots up to
// min(top_n, jc+1) go to the other blocks 0..jc by descending score, ties to the lower
// index.  Output ascending, padded with -1.
#pragma once

#include "common.hpp"

namespace nsa {

__device__ __forceinline__ int visible_count(int t, int l, int s, int N) {
    if (t < l - 1) return 0;
    const int n = (t - l + 1) / s + 1;
    return n < N ? n : N;
}

// Order-preserving map of a float to uint32 (larger float -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t f2key(float x) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, off);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// One wave selects the blocks of one (token, group) from scores sc[0..jc] and writes
// top_n entries (ascending, -1 padded) to out.  All 64 lanes must call it.
__device__ inline void select_blocks_wave(const float* sc, int jc, int top_n, int n_init, int n_local,
                                   int32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int n_elig = jc + 1;
    const int f_init = min(n_init, n_elig);
    const int f_loc_lo = max(0, jc - n_local + 1);
    const int n_forced = f_init + (jc - f_loc_lo + 1) - max(0, f_init - f_loc_lo);
    const int m = min(top_n, n_elig);
    const int k = m - n_forced;
    const int nu = (n_elig + 63) >> 6;
    uint32_t picked = 0;  // bit u: candidate lane + 64u already taken

    auto is_forced = [&](int j) { return j < f_init || j >= f_loc_lo; };
    auto local_best = [&]() -> uint64_t {
        uint64_t best = 0;
        for (int u = 0; u < nu; ++u) {
            const int j = lane + 64 * u;
            if (j < n_elig && !is_forced(j) && !((picked >> u) & 1u)) {
                const uint64_t key = ((uint64_t)f2key(sc[j]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)j);
                best = key > best ? key : best;
            }
        }
        return best;
    };
    uint64_t mine = local_best();
    for (int r = 0; r < k; ++r) {
        const uint64_t win = wave_max_u64(mine);
        if (win == 0) break;  // no candidate left (cannot happen for a valid configuration)
        const int jw = (int)(0xFFFFFFFFu - (uint32_t)win);
        if ((jw & 63) == lane) {
            picked |= 1u << (jw >> 6);
            mine = local_best();
        }
    }
    // compaction in ascending block order
    int base = 0;
    for (int u = 0; u < nu; ++u) {
        const int j = lane + 64 * u;
        const bool take = j < n_elig && (is_forced(j) || ((picked >> u) & 1u));
        const uint64_t mask = __ballot(take);
        const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
        if (take) out[pos] = j;
        base += __popcll(mask);
    }
    for (int c = base + lane; c < top_n; c += 64) out[c] = -1;
}


}  // namespace nsa
