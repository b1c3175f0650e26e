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
__device__ __forceinline__ uint32_t max_dpp_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
    return o > v ? o : v;
}

template <int CTRL>
__device__ __forceinline__ uint32_t min_dpp_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, CTRL, 0xF, 0xF, false);
    return o < v ? o : v;
}

// Minimum over the 64 lanes (all lanes active), wave-uniform.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min_dpp_u32<kDppQuadXor1>(v);
    v = min_dpp_u32<kDppQuadXor2>(v);
    v = min_dpp_u32<kDppRowHalfMirror>(v);
    v = min_dpp_u32<kDppRowMirror>(v);
    u32x2 r = swap16(v);
    v = r[0] < r[1] ? r[0] : r[1];
    r = swap32(v);
    v = r[0] < r[1] ? r[0] : r[1];
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Maximum over the 64 lanes (all lanes active): DPP moves inside each 16-lane row, then
// the two row-swapping permutes; returned as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max_dpp_u32<kDppQuadXor1>(v);
    v = max_dpp_u32<kDppQuadXor2>(v);
    v = max_dpp_u32<kDppRowHalfMirror>(v);
    v = max_dpp_u32<kDppRowMirror>(v);
    u32x2 r = swap16(v);
    v = r[0] > r[1] ? r[0] : r[1];
    r = swap32(v);
    v = r[0] > r[1] ? r[0] : r[1];
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Forced blocks of the query's own block jc: blocks 0..f_init-1 and f_loc_lo..jc.
struct ForcedBlocks {
    int n_elig, f_init, f_loc_lo, k;
    __device__ ForcedBlocks(int jc, int top_n, int n_init, int n_local) {
        n_elig = jc + 1;
        f_init = min(n_init, n_elig);
        f_loc_lo = max(0, jc - n_local + 1);
        const int n_forced = f_init + (jc - f_loc_lo + 1) - max(0, f_init - f_loc_lo);
        k = min(top_n, n_elig) - n_forced;   // picks left for the scores
    }
    __device__ bool forced(int j) const { return j < f_init || j >= f_loc_lo; }
    __device__ bool candidate(int j) const { return j < n_elig && !forced(j); }
};

// Writes the forced blocks and the blocks flagged by taken(u) (slot u of this lane, block
// lane + 64u) to out (and out2) in ascending order, padded with -1 to top_n.
template <int NU, typename Taken>
__device__ __forceinline__ void emit_selection(const ForcedBlocks& fb, int top_n, Taken taken,
                                               int32_t* __restrict__ out, int32_t* __restrict__ out2) {
    const int lane = threadIdx.x & 63;
    int base = 0;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int j = lane + 64 * u;
        const bool take = j < fb.n_elig && (fb.forced(j) || taken(u));
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

// One wave selects the blocks of one (token, group) from scores sc[0..jc] and writes
// top_n entries (ascending, -1 padded) to out (and to out2 when it is not null).  All 64
// lanes must call it; NU * 64 must cover jc + 1.  Lane l holds the candidates l, l + 64,
// ... as 64-bit entries key:slot (key: order-preserving 32-bit image of the score; slot u
// stored as NU-1-u, so a larger entry is a better score or, for equal scores, the lower
// block index).  For more than 4 picks each lane sorts its entries once (bitonic network,
// best first) and a pick is a wave maximum over the lanes' heads, the winning lane shifting
// its list; for up to 4 picks each pick rescans the lane's entries instead.
template <int NU>
__device__ inline void select_blocks_wave(const float* sc, int jc, int top_n, int n_init, int n_local,
                                          int32_t* __restrict__ out, int32_t* __restrict__ out2 = nullptr) {
    const int lane = threadIdx.x & 63;
    const ForcedBlocks fb(jc, top_n, n_init, n_local);
    uint64_t e[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int j = lane + 64 * u;
        e[u] = fb.candidate(j) ? (((uint64_t)f2key(sc[j]) << 32) | (uint32_t)(NU - 1 - u)) : 0ull;
    }
    uint32_t picked = 0;  // bit u: candidate lane + 64u taken
    if (fb.k <= 4) {
        // few picks: rescan the lane's entries per pick instead of sorting them
        for (int r = 0; r < fb.k; ++r) {
            uint64_t t = e[0];
#pragma unroll
            for (int u = 1; u < NU; ++u) t = e[u] > t ? e[u] : t;
            const uint32_t hk = (uint32_t)(t >> 32);
            const uint32_t m = wave_max_u32(hk);
            if (m == 0) break;
            const int hu = NU - 1 - (int)(uint32_t)t;
            const uint32_t jl = hk == m ? (uint32_t)(lane + 64 * hu) : 0xFFFFFFFFu;
            const uint64_t holders = __ballot(hk == m);
            const uint32_t jw = __popcll(holders) == 1
                                    ? (uint32_t)__builtin_amdgcn_readlane((int)jl, (int)__builtin_ctzll(holders))
                                    : wave_min_u32(jl);
            if (jl == jw) {
                picked |= 1u << hu;
#pragma unroll
                for (int u = 0; u < NU; ++u) e[u] = u == hu ? 0ull : e[u];
            }
        }
        emit_selection<NU>(fb, top_n, [&](int u) { return ((picked >> u) & 1u) != 0; }, out, out2);
        return;
    }
    // bitonic sort, descending
#pragma unroll
    for (int kk = 2; kk <= NU; kk <<= 1)
#pragma unroll
        for (int jj = kk >> 1; jj > 0; jj >>= 1)
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                const int l = i ^ jj;
                if (l > i) {
                    const bool desc = (i & kk) == 0;
                    const uint64_t a = e[i], b = e[l];
                    const bool sw = desc ? (b > a) : (a > b);
                    e[i] = sw ? b : a;
                    e[l] = sw ? a : b;
                }
            }
    for (int r = 0; r < fb.k; ++r) {
        const uint32_t hk = (uint32_t)(e[0] >> 32);
        const uint32_t m = wave_max_u32(hk);
        if (m == 0) break;  // no candidate left (cannot happen for a valid configuration)
        // the lowest block index among the heads scoring m
        const int hu = NU - 1 - (int)(uint32_t)e[0];
        const uint32_t jl = hk == m ? (uint32_t)(lane + 64 * hu) : 0xFFFFFFFFu;
        const uint64_t holders = __ballot(hk == m);
        const uint32_t jw = __popcll(holders) == 1
                                ? (uint32_t)__builtin_amdgcn_readlane((int)jl, (int)__builtin_ctzll(holders))
                                : wave_min_u32(jl);
        if (jl == jw) {
            picked |= 1u << hu;
#pragma unroll
            for (int u = 0; u + 1 < NU; ++u) e[u] = e[u + 1];
            e[NU - 1] = 0ull;
        }
    }
    emit_selection<NU>(fb, top_n, [&](int u) { return ((picked >> u) & 1u) != 0; }, out, out2);
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
