// Compressed attention, block scores and group-shared top-n selection.
//
// Method (zjai.club notes, sections 5 and 8; sunshychen.top comparison): a query attends
// to the compressed blocks whose tokens are all at or before it; those attention
// probabilities, summed over the heads of the GQA group and over the compressed blocks
// that overlap a selection block, are that block's score; the group then keeps the
// forced blocks plus the best-scoring others.  MoBA mode scores a block by the inner
// product of the query with the block's mean key instead.
//
// Kernels (per KV group):
//   cmp_attn_kernel    compressed attention and block scores (the body is cmp_attn_tile in
//                      cmp_attn.hpp, shared with the fused prefill kernel).
//   mean_scores_kernel mode 1: head-summed raw dot products with the mean keys.
//   select_kernel      one wave per (token, group): the shared top-n from the scores.
#include <climits>

#include "cmp_attn.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace nsa {

namespace {

using cmpk::kWaves;
using cmpk::kKeysPerTile;
using cmpk::kRing;
constexpr int kVmaxParts = 64;           // partial maxima of |V_cmp| per unit

// Rows [k0, k0+64) of a [N][D] bf16 matrix (rows clamped to N-1) into LDS rows of
// stride LSTR.  All global loads are issued before the first LDS store.
template <int D, int LSTR>
__device__ __forceinline__ void stage_rows(const u16* __restrict__ src, int k0, int N, u16* dst) {
    constexpr int PER_ROW = D / 8;
    constexpr int TOTAL = kKeysPerTile * PER_ROW;
    constexpr int ITERS = (TOTAL + 255) / 256;
    u32x4 v[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int row = idx / PER_ROW, col = (idx % PER_ROW) * 8;
        if (TOTAL % 256 == 0 || idx < TOTAL)
            v[i] = *reinterpret_cast<const u32x4*>(src + (size_t)min(k0 + row, N - 1) * D + col);
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int row = idx / PER_ROW, col = (idx % PER_ROW) * 8;
        if (TOTAL % 256 == 0 || idx < TOTAL) *reinterpret_cast<u32x4*>(&dst[row * LSTR + col]) = v[i];
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Largest |V_cmp| per unit, in 64 partial maxima (bf16 magnitudes compare as integers).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void cmp_vmax_kernel(const u16* __restrict__ V, uint32_t* __restrict__ part,
                                                       int N, int DV) {
    __shared__ uint32_t red[256];
    const size_t unit = blockIdx.y;
    // 16-byte loads: n and each part's bounds are multiples of 8 elements (DV is)
    const size_t n = (size_t)N * DV, per = ((n + kVmaxParts - 1) / kVmaxParts + 7) / 8 * 8;
    const size_t lo = min(blockIdx.x * per, n), hi = min(lo + per, n);
    const u16* v = V + unit * n;
    // eight 16-byte loads in flight per thread (one at a time left the pass latency-bound:
    // 0.31 ms for the 67 MB of V at 64K)
    constexpr int UNR = 8;
    uint32_t mx = 0;
    for (size_t i0 = lo + 8 * threadIdx.x; i0 < hi; i0 += (size_t)8 * 256 * UNR) {
        u32x4 w[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const size_t i = i0 + (size_t)8 * 256 * u;
            w[u] = i < hi ? *reinterpret_cast<const u32x4*>(v + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u)
#pragma unroll
            for (int k = 0; k < 4; ++k) mx = max(mx, max(w[u][k] & 0x7FFFu, (w[u][k] >> 16) & 0x7FFFu));
    }
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + off]);
        __syncthreads();
    }
    if (threadIdx.x == 0) part[unit * kVmaxParts + blockIdx.x] = red[0];
}

// Power-of-two exponent e that brings the unit's largest |V_cmp| into (2^13, 2^14]: the
// fp16 copy holds V_cmp * 2^-e (exact unless a value falls below fp16's normal range
// relative to the largest one) and o_cmp is rescaled by 2^e in fp32.
__device__ __forceinline__ int cmp_v_exponent(const uint32_t* part) {
    uint32_t mx = 0;
    for (int i = 0; i < kVmaxParts; ++i) mx = max(mx, part[i]);
    const float m = bf2f((u16)mx);
    if (!(m > 0.f) || !(m < INFINITY)) return 0;
    int k;
    (void)frexpf(m, &k);   // m <= 2^k
    return min(max(k - 14, -100), 100);
}

// ---------------------------------------------------------------------------
// Fragment order of the compressed keys / values (the layout of the attention kernel's
// K and V copies): for 16-key group kt and contraction step ds, lane (li, lq) of the A
// operand holds K[16kt + li][32ds + 8lq .. +7], the 64 lanes' pieces contiguous; for
// 32-key chunk c and value slice dt, lane (li, lq) holds V^T[16dt + li] at keys
// 32c + {4lq..4lq+3, 16+4lq..16+4lq+3}, as fp16 scaled by 2^-e (cmp_v_exponent; e is
// written to vexp[unit]).  Keys >= N are zero.  With Kf null only the values are copied
// (the block-major kernel gathers its K tiles from the row-major keys itself).
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void tile_cmp_kernel(const u16* __restrict__ K, const u16* __restrict__ V,
                                                       const uint32_t* __restrict__ vmax_part,
                                                       int* __restrict__ vexp, u16* __restrict__ Kf,
                                                       u16* __restrict__ Vf, int N, int Npad) {
    constexpr int NDS = DK / 32, NDT = DV / 16;
    constexpr int KSTR = DK + 8, VSTR = DV + 16;
    __shared__ __attribute__((aligned(16))) u16 ks[32 * KSTR];
    __shared__ __attribute__((aligned(16))) u16 vs[32 * VSTR];
    const int c = blockIdx.x;
    const size_t bg = blockIdx.y;
    const u16* kg = K + bg * (size_t)N * DK;
    for (int idx = threadIdx.x; Kf && idx < 32 * DK / 8; idx += 256) {
        const int r = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
        const int key = 32 * c + r;
        const u32x4 v = key < N ? *reinterpret_cast<const u32x4*>(kg + (size_t)key * DK + col) : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(&ks[r * KSTR + col]) = v;
    }
    if (V) {
        const int e = cmp_v_exponent(vmax_part + bg * kVmaxParts);
        if (c == 0 && threadIdx.x == 0) vexp[bg] = e;
        const float sc = ldexpf(1.0f, -e);
        const u16* vg = V + bg * (size_t)N * DV;
        for (int idx = threadIdx.x; idx < 32 * DV / 8; idx += 256) {
            const int r = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            const int key = 32 * c + r;
            const u32x4 v =
                key < N ? *reinterpret_cast<const u32x4*>(vg + (size_t)key * DV + col) : u32x4{0u, 0u, 0u, 0u};
            u16 h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u16 bits = (u16)(v[i >> 1] >> (16 * (i & 1)));
                h[i] = __builtin_bit_cast(u16, static_cast<_Float16>(bf2f(bits) * sc));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) vs[r * VSTR + col + i] = h[i];
        }
    }
    __syncthreads();
    u16* kout = Kf + bg * (size_t)Npad * DK + (size_t)(2 * c) * NDS * 512;
    for (int idx = threadIdx.x; Kf && idx < 2 * NDS * 64; idx += 256) {
        const int kk = idx / (NDS * 64), ds = (idx / 64) % NDS, ln = idx % 64;
        const int li = ln & 15, lq = ln >> 4;
        *reinterpret_cast<u32x4*>(kout + (size_t)idx * 8) =
            *reinterpret_cast<const u32x4*>(&ks[(16 * kk + li) * KSTR + 32 * ds + 8 * lq]);
    }
    if (V) {
        u16* vout = Vf + bg * (size_t)Npad * DV + (size_t)c * NDT * 512;
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        for (int dt = wave; dt < NDT; dt += 4)
            *reinterpret_cast<bf16x8*>(vout + (size_t)(dt * 64 + lane) * 8) = ld_vt_tr(vs, VSTR, 0, 16 * dt);
    }
}

// ---------------------------------------------------------------------------
// mode 0: compressed attention (log-sum-exp, o_cmp) and block scores, one kernel
// ---------------------------------------------------------------------------
template <int DK, int DV, int G, int NQ, bool WITH_O>
__global__ __launch_bounds__(64 * cmp_waves(G), 2) void cmp_attn_kernel(SelParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    constexpr int TQ = cmp_waves(G) * NQ * 16 / G;
    const int n_tiles = (p.T + TQ - 1) / TQ;
    int unit, it;
    if (!xcd_map_tile(blockIdx.x, p.B * p.Hkv, n_tiles, unit, it)) return;
    cmp_attn_tile<DK, DV, G, NQ, WITH_O>(p, unit, (n_tiles - 1 - it) * TQ, smem);   // longest rows first
}

// ---------------------------------------------------------------------------
// mode 1: block score = sum over the group's heads of q . (mean key of the block), for
// the complete blocks before the query's own block (requires l == s == l')
// ---------------------------------------------------------------------------
template <int DK, int G, int NQ>
__global__ __launch_bounds__(256, 2) void mean_scores_kernel(SelParams p) {
    constexpr int TQ = kWaves * NQ * 16 / G;
    constexpr int KSTR = DK + 8;
    constexpr int NDS = DK / 32;
    __shared__ __attribute__((aligned(16))) u16 ks[kKeysPerTile * KSTR];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int T = p.T, N = p.N;
    const int n_tiles = (T + TQ - 1) / TQ;
    int unit, it;
    if (!xcd_map_tile(blockIdx.x, p.B * p.Hkv, n_tiles, unit, it)) return;
    const int b = unit / p.Hkv, g = unit % p.Hkv;
    const int H = p.Hkv * G;
    const int tok0 = (n_tiles - 1 - it) * TQ;

    using M = QMap<G, NQ>;
    bf16x8 qf[NQ][NDS];
    int tok[NQ], hl[NQ], nv[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        tok[c] = tok0 + wave * M::TPW + M::token(c, li);
        hl[c] = M::head(c, li);
        const int tt = min(tok[c], T - 1);
        const u16* qp = p.Q + (((size_t)b * T + tt) * H + g * G + hl[c]) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[c][ds] = ld8(qp + 32 * ds);
        nv[c] = tok[c] < T ? min(tok[c] / p.lp, N) : 0;
    }
    const int t_last = min(tok0 + TQ - 1, T - 1);
    const int nv_max = min(t_last / p.lp, N);
    const u16* kbase = p.Kc + (size_t)unit * N * DK;

    for (int k0 = 0; k0 < nv_max; k0 += kKeysPerTile) {
        __syncthreads();
        stage_rows<DK, KSTR>(kbase, k0, N, ks);
        __syncthreads();
        f32x4 s[4][NQ];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int c = 0; c < NQ; ++c) s[kt][c] = zero4();
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const bf16x8 a = ld8(&ks[(16 * kt + li) * KSTR + 32 * ds + lq * 8]);
#pragma unroll
                for (int c = 0; c < NQ; ++c) s[kt][c] = mfma16(a, qf[c][ds], s[kt][c]);
            }
#pragma unroll
        for (int cg = 0; cg < NQ / M::CL; ++cg) {
            const int tl = wave * M::TPW + M::token(cg * M::CL, li);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float hs = 0.f;
#pragma unroll
                    for (int c = cg * M::CL; c < (cg + 1) * M::CL; ++c) hs += s[kt][c][r];
                    hs = lane_group_sum<M::GL>(hs);
                    const int key = k0 + 16 * kt + 4 * lq + r;
                    if ((li % M::GL) == 0 && key < nv[cg * M::CL])
                        p.scores[(((size_t)b * T + tok0 + tl) * p.Hkv + g) * p.n_slc + key] = hs;
                }
        }
    }
}

// mode 1 with the selection fused, for one query head per KV head (G = 1) and at most
// kFusedMaxPicks picks besides the forced blocks (the MoBA configuration: top-3 with the
// own block forced, two picks).  A workgroup owns 64 tokens (a wave's 16 MFMA columns are
// 16 tokens); each lane keeps, for its column, the best K candidates (K = the picks rounded
// up to 1, 2 or 4) among the keys it holds, as fp32 scores with their block indices, so no
// score row is ever stored.  A lane meets its keys in ascending index order, so a candidate
// enters the list only on a strictly larger score (equal scores keep the lower index), and
// the entries it displaces move down unconditionally; every candidate goes through the
// branch-free insertion (an invalid one as -inf).  The four lanes of a
// column then merge their lists as 64-bit entries score-key:~index (larger = better score,
// then lower index): bitonic top-K of two sorted lists, then a sort, across the 16- and
// 32-lane swaps.
template <int DK, int K>
__global__ __launch_bounds__(256, 2) void mean_select_kernel(SelParams p) {
    constexpr int TQ = kWaves * 16;
    constexpr int KSTR = DK + 8;
    constexpr int NDS = DK / 32;
    __shared__ __attribute__((aligned(16))) u16 ks[kKeysPerTile * KSTR];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int T = p.T, N = p.N;
    const int n_tiles = (T + TQ - 1) / TQ;
    int unit, it;
    if (!xcd_map_tile(blockIdx.x, p.B * p.Hkv, n_tiles, unit, it)) return;
    const int b = unit / p.Hkv, g = unit % p.Hkv;
    const int tok0 = (n_tiles - 1 - it) * TQ;
    const int tok = tok0 + wave * 16 + li;
    const int tt = min(tok, T - 1);
    bf16x8 qf[NDS];
    {
        const u16* qp = p.Q + (((size_t)b * T + tt) * p.Hkv + g) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[ds] = ld8(qp + 32 * ds);
    }
    const ForcedBlocks fb(tt / p.lp, p.top_n, p.n_init, p.n_local);
    const bool live = tok < T;
    const int t_last = min(tok0 + TQ - 1, T - 1);
    const int nv_max = min(t_last / p.lp, N);
    const u16* kbase = p.Kc + (size_t)unit * N * DK;

    // this lane's candidates: blocks f_init <= j < f_loc_lo (the initial and local blocks are
    // forced; f_loc_lo <= jc, so every candidate is a complete earlier block)
    const int clo = live ? fb.f_init : 0, chi = live ? fb.f_loc_lo : 0;
    // tiles whose 64 keys are candidates of every lane of the wave skip the range test
    const int wclo = (int)wave_max_u32((uint32_t)clo), wchi = (int)wave_min_u32((uint32_t)chi);
    const uint32_t span = chi > clo ? (uint32_t)(chi - clo) : 0u;   // j is a candidate iff j - clo < span
    float bs[K];
    int bi[K];
#pragma unroll
    for (int i = 0; i < K; ++i) { bs[i] = -INFINITY; bi[i] = -1; }
    for (int k0 = 0; k0 < nv_max; k0 += kKeysPerTile) {
        __syncthreads();
        stage_rows<DK, KSTR>(kbase, k0, N, ks);
        __syncthreads();
        f32x4 s[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) s[kt] = zero4();
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) s[kt] = mfma16(ld8(&ks[(16 * kt + li) * KSTR + 32 * ds + lq * 8]), qf[ds], s[kt]);
        // insert into the descending list: the candidate takes the first slot it beats (the
        // tests x > bs[q] are monotone in q and independent of each other); every later slot
        // takes the entry above it (ranked higher by the list's order even on an equal score,
        // being of a lower index)
        auto insert = [&](float x, int jx) {
            bool cp = false;   // the slot above was taken by the candidate or shifted
            int ip = 0;
            float bp = 0.f;
#pragma unroll
            for (int q = 0; q < K; ++q) {
                const bool c = x > bs[q];
                const float tb = bs[q];
                const int ti = bi[q];
                // the new value of slot q is the middle one of (bs[q], x, bs[q-1]) as
                // bs[q] <= bs[q-1]: the one above if x beat it, else x if x beats bs[q]
                bs[q] = q == 0 ? (c ? x : tb) : __builtin_amdgcn_fmed3f(tb, x, bp);
                bi[q] = cp ? ip : (c ? jx : ti);
                cp = c;
                bp = tb;
                ip = ti;
            }
        };
        if (k0 >= wclo && k0 + kKeysPerTile <= wchi) {   // wave-uniform: every key a candidate
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) insert(s[kt][r], k0 + 16 * kt + 4 * lq + r);
        } else {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = k0 + 16 * kt + 4 * lq + r;
                    insert((uint32_t)(j - clo) < span ? s[kt][r] : -INFINITY, j);
                }
        }
    }
    uint64_t best[K];
#pragma unroll
    for (int q = 0; q < K; ++q)
        best[q] = bi[q] >= 0 ? (((uint64_t)f2key(bs[q]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)bi[q])) : 0ull;
    // merge the column's four lists: lanes l and l ^ 16, then l and l ^ 32
#pragma unroll
    for (int step = 0; step < 2; ++step) {
        uint64_t other[K];
#pragma unroll
        for (int q = 0; q < K; ++q) {
            const u32x2 lo = step == 0 ? swap16((uint32_t)best[q]) : swap32((uint32_t)best[q]);
            const u32x2 hi = step == 0 ? swap16((uint32_t)(best[q] >> 32)) : swap32((uint32_t)(best[q] >> 32));
            const bool upper = step == 0 ? (lane & 16) != 0 : (lane & 32) != 0;
            other[q] = ((uint64_t)(upper ? hi[0] : hi[1]) << 32) | (upper ? lo[0] : lo[1]);
        }
        // the top K of two descending lists is max(a[i], b[K-1-i]) (a bitonic sequence) ...
#pragma unroll
        for (int q = 0; q < K; ++q) best[q] = best[q] > other[K - 1 - q] ? best[q] : other[K - 1 - q];
        // ... sorted descending by a bitonic half-cleaner cascade
#pragma unroll
        for (int w = K / 2; w >= 1; w /= 2)
#pragma unroll
            for (int q = 0; q < K; ++q)
                if ((q & w) == 0) {
                    const uint64_t a = best[q], bb = best[q + w];
                    best[q] = a > bb ? a : bb;
                    best[q + w] = a > bb ? bb : a;
                }
    }
    if (lq != 0 || !live) return;
    // the row: initial blocks, the picks (ascending), the local blocks; -1 padded
    int pk[K];
    int np = 0;
#pragma unroll
    for (int q = 0; q < K; ++q) {
        const bool take = q < fb.k && best[q] != 0ull;
        pk[q] = take ? (int)(0xFFFFFFFFu - (uint32_t)best[q]) : INT_MAX;
        np += take ? 1 : 0;
    }
#pragma unroll
    for (int a = 0; a < K; ++a)
#pragma unroll
        for (int q = 0; q + 1 < K; ++q) {
            const int lo = min(pk[q], pk[q + 1]), hi = max(pk[q], pk[q + 1]);
            pk[q] = lo;
            pk[q + 1] = hi;
        }
    int32_t* out = p.sel + ((size_t)(b * T + tok) * p.Hkv + g) * p.top_n;
    int pos = 0;
    for (int j = 0; j < fb.f_init; ++j) out[pos++] = j;
#pragma unroll
    for (int q = 0; q < K; ++q)
        if (q < np) out[pos++] = pk[q];
    for (int j = max(fb.f_loc_lo, fb.f_init); j <= fb.n_elig - 1; ++j) out[pos++] = j;
    for (; pos < p.top_n; ++pos) out[pos] = -1;
}

// Selection from scores [B,T,Hkv,n_slc]: one wave per (b, t, g).
template <int NU>
__global__ __launch_bounds__(256) void select_from_scores_kernel(const float* __restrict__ scores,
                                                                 int32_t* __restrict__ sel, int T, int Hkv,
                                                                 int n_slc, int lp, int top_n, int n_init,
                                                                 int n_local, long rows) {
    const long row = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int t = (int)((row / Hkv) % T);
    select_blocks_wave<NU>(scores + row * n_slc, t / lp, top_n, n_init, n_local, sel + row * top_n);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {

template <int DK, int DV, int G, int NQ, bool WITH_O>
void cmp_attn_g(const SelParams& p, hipStream_t st) {
    constexpr int TQ = cmp_waves(G) * NQ * 16 / G;
    const int n_tiles = (p.T + TQ - 1) / TQ;
    const size_t lds = cmp_attn_lds_bytes(DK, DV, G, WITH_O);
    const void* fn = reinterpret_cast<const void*>(cmp_attn_kernel<DK, DV, G, NQ, WITH_O>);
    if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    cmp_attn_kernel<DK, DV, G, NQ, WITH_O><<<xcd_grid(p.B * p.Hkv, n_tiles), 64 * cmp_waves(G), lds, st>>>(p);
}

template <int DK, int DV, int G>
void cmp_attn_dk(bool with_o, const SelParams& p, hipStream_t st) {
    constexpr int NQ = G == 1 ? 1 : 2;
    if (with_o) cmp_attn_g<DK, DV, G, NQ, true>(p, st);
    else cmp_attn_g<DK, DV, G, NQ, false>(p, st);
}

template <int DK, int G>
void mean_scores_g(const SelParams& p, hipStream_t st) {
    constexpr int NQ = G == 1 ? 1 : 2;
    constexpr int TQ = kWaves * NQ * 16 / G;
    const int n_tiles = (p.T + TQ - 1) / TQ;
    mean_scores_kernel<DK, G, NQ><<<xcd_grid(p.B * p.Hkv, n_tiles), 256, 0, st>>>(p);
}

}  // namespace

size_t cmp_attn_lds_bytes(int DK, int DV, int G, bool with_o) {
    const int NQ = G == 1 ? 1 : 2;
    const int TQ = cmp_waves(G) * NQ * 16 / G;
    const size_t k = (size_t)kKeysPerTile * DK * 2, v = with_o ? (size_t)kKeysPerTile * DV * 2 : 0;
    return 2 * k + v + (size_t)TQ * kRing * 4;
}

#define NSA_G_SWITCH(G, ...)                                       \
    switch (G) {                                                   \
        case 1: { constexpr int GG = 1; __VA_ARGS__; } break;      \
        case 2: { constexpr int GG = 2; __VA_ARGS__; } break;      \
        case 4: { constexpr int GG = 4; __VA_ARGS__; } break;      \
        case 8: { constexpr int GG = 8; __VA_ARGS__; } break;      \
        case 16: { constexpr int GG = 16; __VA_ARGS__; } break;    \
        default: return false;                                     \
    }

int cmp_vmax_parts() { return kVmaxParts; }

bool launch_tile_cmp(int DK, int DV, const u16* K, const u16* V, uint32_t* vmax_part, int* vexp, u16* Kf, u16* Vf,
                     int BG, int N, int Npad, hipStream_t st) {
    if (V) cmp_vmax_kernel<<<dim3(kVmaxParts, BG), 256, 0, st>>>(V, vmax_part, N, DV);
    dim3 grid(Npad / 32, BG);
    if (DK == 192 && DV == 128)
        tile_cmp_kernel<192, 128><<<grid, 256, 0, st>>>(K, V, vmax_part, vexp, Kf, Vf, N, Npad);
    else if (DK == 128 && DV == 128)
        tile_cmp_kernel<128, 128><<<grid, 256, 0, st>>>(K, V, vmax_part, vexp, Kf, Vf, N, Npad);
    else if (DK == 64 && DV == 64)
        tile_cmp_kernel<64, 64><<<grid, 256, 0, st>>>(K, V, vmax_part, vexp, Kf, Vf, N, Npad);
    else return false;
    return true;
}

bool launch_cmp_attn(bool with_o, int DK, int DV, int G, const SelParams& p, hipStream_t st) {
    if (DK == 192 && DV == 128) { NSA_G_SWITCH(G, cmp_attn_dk<192, 128, GG>(with_o, p, st)); }
    else if (DK == 128 && DV == 128) { NSA_G_SWITCH(G, cmp_attn_dk<128, 128, GG>(with_o, p, st)); }
    else if (DK == 64 && DV == 64) { NSA_G_SWITCH(G, cmp_attn_dk<64, 64, GG>(with_o, p, st)); }
    else return false;
    return true;
}

namespace {
// each lane keeps the best K candidates, K the free picks rounded up to a power of two
template <int DK>
void mean_select_k(int picks, int grid, const SelParams& p, hipStream_t st) {
    if (picks <= 1) mean_select_kernel<DK, 1><<<grid, 256, 0, st>>>(p);
    else if (picks <= 2) mean_select_kernel<DK, 2><<<grid, 256, 0, st>>>(p);
    else mean_select_kernel<DK, kFusedMaxPicks><<<grid, 256, 0, st>>>(p);
}
}  // namespace

bool launch_mean_select(int DK, const SelParams& p, hipStream_t st) {
    constexpr int TQ = kWaves * 16;
    const int grid = xcd_grid(p.B * p.Hkv, (p.T + TQ - 1) / TQ);
    const int picks = p.top_n - p.n_local;   // at most this many blocks are picked by score
    if (DK == 192) mean_select_k<192>(picks, grid, p, st);
    else if (DK == 128) mean_select_k<128>(picks, grid, p, st);
    else if (DK == 64) mean_select_k<64>(picks, grid, p, st);
    else return false;
    return true;
}

bool launch_mean_scores(int DK, int G, const SelParams& p, hipStream_t st) {
    if (DK == 192) { NSA_G_SWITCH(G, mean_scores_g<192, GG>(p, st)); }
    else if (DK == 128) { NSA_G_SWITCH(G, mean_scores_g<128, GG>(p, st)); }
    else if (DK == 64) { NSA_G_SWITCH(G, mean_scores_g<64, GG>(p, st)); }
    else return false;
    return true;
}

void launch_select_from_scores(const float* scores, int32_t* sel, int B, int T, int Hkv, int n_slc, int lp,
                               int top_n, int n_init, int n_local, hipStream_t st) {
    const long rows = (long)B * T * Hkv;
    const long blocks = (rows + kWaves - 1) / kWaves;
    NSA_NU_SWITCH(n_slc, select_from_scores_kernel<NU><<<(unsigned)blocks, 256, 0, st>>>(
                             scores, sel, T, Hkv, n_slc, lp, top_n, n_init, n_local, rows));
}

}  // namespace nsa
