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

template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > v ? o : v;
}

// Maximum over the 64 lanes (all lanes active): DPP moves inside each 16-lane row, then
// two cross-row lane shuffles.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_dpp_u64<kDppQuadXor1>(v);
    v = max_dpp_u64<kDppQuadXor2>(v);
    v = max_dpp_u64<kDppRowHalfMirror>(v);
    v = max_dpp_u64<kDppRowMirror>(v);
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, off);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// One wave selects the blocks of one (token, group) from scores sc[0..jc] and writes
// top_n entries (ascending, -1 padded) to out (and to out2 when it is not null).  All 64
// lanes must call it; NU * 64 must cover jc + 1.  Each lane keeps its candidates
// (blocks lane, lane + 64, ...) in registers as 64-bit keys score:~index, so one wave
// maximum per pick yields the best score and, among equal scores, the lowest index.
template <int NU>
__device__ inline void select_blocks_wave(const float* sc, int jc, int top_n, int n_init, int n_local,
                                          int32_t* __restrict__ out, int32_t* __restrict__ out2 = nullptr) {
    const int lane = threadIdx.x & 63;
    const int n_elig = jc + 1;
    const int f_init = min(n_init, n_elig);
    const int f_loc_lo = max(0, jc - n_local + 1);
    const int n_forced = f_init + (jc - f_loc_lo + 1) - max(0, f_init - f_loc_lo);
    const int m = min(top_n, n_elig);
    const int k = m - n_forced;
    auto is_forced = [&](int j) { return j < f_init || j >= f_loc_lo; };

    uint64_t key[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int j = lane + 64 * u;
        const bool cand = j < n_elig && !is_forced(j);
        key[u] = cand ? (((uint64_t)f2key(sc[j]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)j)) : 0ull;
    }
    uint32_t picked = 0;  // bit u: candidate lane + 64u taken
    for (int r = 0; r < k; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int u = 0; u < NU; ++u) best = key[u] > best ? key[u] : best;
        const uint64_t win = wave_max_u64(best);
        if (win == 0) break;  // no candidate left (cannot happen for a valid configuration)
        const int jw = (int)(0xFFFFFFFFu - (uint32_t)win);
        if ((jw & 63) == lane) {
#pragma unroll
            for (int u = 0; u < NU; ++u)
                if (u == (jw >> 6)) key[u] = 0ull;
            picked |= 1u << (jw >> 6);
        }
    }
    // compaction in ascending block order
    int base = 0;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int j = lane + 64 * u;
        const bool take = j < n_elig && (is_forced(j) || ((picked >> u) & 1u));
        const uint64_t mask = __ballot(take);
        const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
        if (take) {
            out[pos] = j;
            if (out2) out2[pos] = j;
        }
        base += __popcll(mask);
    }
    for (int c = base + lane; c < top_n; c += 64) {
        out[c] = -1;
        if (out2) out2[c] = -1;
    }
}

// Candidates per lane for n_slc selection blocks (a power of two, at most 32).
__host__ __device__ constexpr int select_nu(int n_slc) {
    return n_slc <= 64 ? 1 : n_slc <= 128 ? 2 : n_slc <= 256 ? 4 : n_slc <= 512 ? 8 : n_slc <= 1024 ? 16 : 32;
}

#define NSA_NU_SWITCH(NSLC, ...)                                        \
    switch (select_nu(NSLC)) {                                          \
        case 1: { constexpr int NU = 1; __VA_ARGS__; } break;           \
        case 2: { constexpr int NU = 2; __VA_ARGS__; } break;           \
        case 4: { constexpr int NU = 4; __VA_ARGS__; } break;           \
        case 8: { constexpr int NU = 8; __VA_ARGS__; } break;           \
        case 16: { constexpr int NU = 16; __VA_ARGS__; } break;         \
        default: { constexpr int NU = 32; __VA_ARGS__; } break;         \
    }

}  // namespace nsa
