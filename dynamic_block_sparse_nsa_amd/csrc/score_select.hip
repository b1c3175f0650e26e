// Compressed attention, block scores and group-shared top-n selection.
//
// Method (zjai.club notes, sections 5 and 8; sunshychen.top comparison): a query attends
// to the compressed blocks whose tokens are all at or before it; those attention
// probabilities, summed over the heads of the GQA group and over the compressed blocks
// that overlap a selection block, are that block's score; the group then keeps the
// forced blocks plus the best-scoring others.  MoBA mode scores a block by the inner
// product of the query with the block's mean key instead.
//
// Kernels (per KV group; a workgroup owns 128 query rows = 128/G tokens, each wave two
// 16-column MFMA tiles laid out by QMap so a token's heads share lanes and tiles):
//   cmp_attn_kernel    sweep 1: S^T = K_cmp . Q^T over 64-key tiles, per-lane running max
//                      and sum, combined into the log-sum-exp b (base 2) of every query row.
//                      Sweep 2: the same S^T again; p = 2^(x - b) are the normalized
//                      probabilities (nothing is rescaled afterwards); o_cmp += V_cmp^T.P^T
//                      on the MFMA; p summed over the group's heads in fp32 (in-lane + DPP)
//                      into a per-token ring in LDS; one tile later, every selection block
//                      whose last compressed key is complete gets its score (sum over its
//                      overlapping compressed blocks, ascending key order) written to the
//                      score workspace.  The compressed keys and values are read in MFMA
//                      fragment order (tile_cmp_kernel), so a tile is one contiguous span
//                      copied to LDS through registers while the previous tile is computed.
//   mean_scores_kernel mode 1: head-summed raw dot products with the mean keys.
//   select_kernel      one wave per (token, group): the shared top-n from the scores.
// Block j of l' tokens takes compressed blocks i with j*R - L + 1 <= i <= j*R + R - 1,
// R = l'/s and L = l/s, i.e. every compressed block whose token span meets block j.
#include <climits>

#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace nsa {

namespace {

constexpr int kWaves = 4;
constexpr int kKeysPerTile = 64;
constexpr int kRing = 4 * kKeysPerTile;  // per-token ring: the tile being written and the two before it
constexpr int kVmaxParts = 64;           // partial maxima of |V_cmp| per unit

// Waves per workgroup of the compressed-attention kernel.  Two workgroups share a CU
// (72 KB of LDS each for G = 16), so the two waves on a SIMD belong to different
// workgroups and drift apart: one's MFMAs overlap the other's VALU work.
__host__ __device__ constexpr int cmp_waves(int) { return 4; }

typedef __attribute__((address_space(3))) void lds_void;

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
    uint32_t mx = 0;
    for (size_t i = lo + 8 * threadIdx.x; i < hi; i += 8 * 256) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(v + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) mx = max(mx, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
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
// written to vexp[unit]).  Keys >= N are zero.
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
    for (int idx = threadIdx.x; idx < 32 * DK / 8; idx += 256) {
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
    for (int idx = threadIdx.x; idx < 2 * NDS * 64; idx += 256) {
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
    constexpr int WAVES = cmp_waves(G);
    constexpr int NT = 64 * WAVES;             // threads
    constexpr int TQ = WAVES * NQ * 16 / G;    // tokens per workgroup
    constexpr int NDS = DK / 32, NDT = DV / 16;
    constexpr int KE = 4 * NDS * 512;          // K elements of a 64-key tile (fragment order)
    constexpr int VE = WITH_O ? 2 * NDT * 512 : 0;
    constexpr int TPT = NT / TQ;               // threads per token when emitting block scores
    // LDS: two K tile slots, one V tile slot, then the ring [TQ][kRing]
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    u16* kslot = reinterpret_cast<u16*>(smem);   // [2][KE]
    u16* vbuf = kslot + 2 * KE;                   // [VE]
    float* ring = reinterpret_cast<float*>(vbuf + VE);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar addressing
    const int li = lane & 15, lq = lane >> 4;
    const int T = p.T, N = p.N;
    const int n_tiles = (T + TQ - 1) / TQ;
    int unit, it;
    if (!xcd_map_tile(blockIdx.x, p.B * p.Hkv, n_tiles, unit, it)) return;
    const int b = unit / p.Hkv, g = unit % p.Hkv;
    const int H = p.Hkv * G;
    const int tok0 = (n_tiles - 1 - it) * TQ;
    const int R = p.lp / p.s, L = p.l / p.s;
    const float sl2 = p.scale_log2;

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
        nv[c] = tok[c] < T ? visible_count(tok[c], p.l, p.s, N) : 0;
    }
    const int t_last = min(tok0 + TQ - 1, T - 1);
    const int nv_max = visible_count(t_last, p.l, p.s, N);
    const int nv_min = visible_count(min(tok0, T - 1), p.l, p.s, N);
    const int ntile = (nv_max + kKeysPerTile - 1) / kKeysPerTile;
    const u16* kg = p.Kf + (size_t)unit * p.Npad * DK;
    const u16* vg = WITH_O ? p.Vf + (size_t)unit * p.Npad * DV : nullptr;

    // Asynchronous copies of a tile's K (KE elements) or V (VE elements), contiguous in
    // fragment order, into LDS: 1 KB per wave instruction, each lane's 16 bytes at lane * 16.
    auto issue_k = [&](int tix, u16* dst) {
        const u16* src = kg + (size_t)tix * KE;
        for (int ch = wave; ch < KE / 512; ch += WAVES)
            __builtin_amdgcn_global_load_lds(src + ch * 512 + lane * 8, (lds_void*)(dst + ch * 512), 16, 0, 0);
    };
    auto issue_v = [&](int tix, u16* dst) {
        if constexpr (WITH_O) {
            const u16* src = vg + (size_t)tix * VE;
            for (int ch = wave; ch < VE / 512; ch += WAVES)
                __builtin_amdgcn_global_load_lds(src + ch * 512 + lane * 8, (lds_void*)(dst + ch * 512), 16, 0, 0);
        }
    };
    // this thread's copies have landed, then every thread's have; every wave is past the
    // reads of whatever the next copies overwrite
    auto copies_done = [&]() {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    // S^T rows of key sub-tiles 2h, 2h+1 (this wave's 16*NQ query columns)
    auto qk_half = [&](const u16* kb, f32x4 (&s)[4][NQ], int h) {
#pragma unroll
        for (int kt = 2 * h; kt < 2 * h + 2; ++kt)
#pragma unroll
            for (int c = 0; c < NQ; ++c) s[kt][c] = zero4();
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
            for (int kt = 2 * h; kt < 2 * h + 2; ++kt) {
                const bf16x8 a = ld8(&kb[((kt * NDS + ds) * 64 + lane) * 8]);
#pragma unroll
                for (int c = 0; c < NQ; ++c) s[kt][c] = mfma16(a, qf[c][ds], s[kt][c]);
            }
    };

    int nb = 0;   // sweep 1: K slot of the current tile

    // ---- sweep 1: per-lane running max and sum over the lane's keys ----
    float m[NQ], lsum[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) { m[c] = -INFINITY; lsum[c] = 0.f; }
    const int nfull = nv_min / kKeysPerTile;   // tiles [0, nfull) are visible to every row
    auto k1buf = [&](int buf) { return kslot + buf * KE; };
    // statistics update from key sub-tiles 2h, 2h+1 of s (all keys visible: mnew is finite,
    // and a first update from m = -inf, lsum = 0 gives 0 * 0)
    auto stats_half = [&](const f32x4 (&s)[4][NQ], int h) {
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            float tmax = fmaxf(s[2 * h][c][0], s[2 * h][c][1]);
#pragma unroll
            for (int e = 2; e < 8; ++e) tmax = fmaxf(tmax, s[2 * h + (e >> 2)][c][e & 3]);
            const float mnew = fmaxf(m[c], tmax * sl2);
            float acc = lsum[c] * fast_exp2(m[c] - mnew);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += fast_exp2(__builtin_fmaf(s[2 * h + (e >> 2)][c][e & 3], sl2, -mnew));
            lsum[c] = acc;
            m[c] = mnew;
        }
    };
    auto tile_start1 = [&](int tix) {   // tile tix landed; copy of tile tix + 1 under way
        copies_done();
        if (tix + 1 < ntile) issue_k(tix + 1, k1buf(nb ^ 1));
        const u16* kb = k1buf(nb);
        nb ^= 1;
        return kb;
    };
    if (ntile > 0) issue_k(0, kslot);
    // Tiles visible to every row, software-pipelined: the statistics of each half tile are
    // updated under the QK products of the next half (across the tile barrier too).
    if (nfull > 0) {
        f32x4 s[4][NQ];
        const u16* kb = tile_start1(0);
        qk_half(kb, s, 0);
        qk_half(kb, s, 1);
        stats_half(s, 0);
        for (int tix = 1; tix < nfull; ++tix) {
            f32x4 prev[4][NQ];
#pragma unroll
            for (int c = 0; c < NQ; ++c) { prev[2][c] = s[2][c]; prev[3][c] = s[3][c]; }
            kb = tile_start1(tix);
            qk_half(kb, s, 0);
            stats_half(prev, 1);
            qk_half(kb, s, 1);
            stats_half(s, 0);
            constexpr int NMQ = 2 * NDS * NQ;   // MFMAs of a QK half
#pragma unroll
            for (int i = 0; i < 2 * NMQ; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
            }
        }
        stats_half(s, 1);
    }
    // tiles with keys invisible to some rows
    for (int tix = nfull; tix < ntile; ++tix) {
        const u16* kb = tile_start1(tix);
        f32x4 s[4][NQ];
        qk_half(kb, s, 0);
        qk_half(kb, s, 1);
        const int k0 = tix * kKeysPerTile;
#pragma unroll
        for (int c = 0; c < NQ; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = k0 + 16 * (e >> 2) + 4 * lq + (e & 3);
                if (key >= nv[c]) s[e >> 2][c][e & 3] = -INFINITY;
            }
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            float tmax = -INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[e >> 2][c][e & 3]);
            const float mnew = fmaxf(m[c], tmax * sl2);
            if (mnew != -INFINITY) {
                float acc = lsum[c] * fast_exp2(m[c] - mnew);
#pragma unroll
                for (int e = 0; e < 16; ++e) acc += fast_exp2(__builtin_fmaf(s[e >> 2][c][e & 3], sl2, -mnew));
                lsum[c] = acc;
                m[c] = mnew;
            }
        }
    }
    // log-sum-exp (base 2) of each query row from the four lanes that share its column
    float bias[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const float Mx = col_max(m[c]);
        const float part = m[c] == -INFINITY ? 0.f : lsum[c] * fast_exp2(m[c] - Mx);
        const float Ls = col_sum(part);
        bias[c] = Ls > 0.f ? Mx + __log2f(Ls) : INFINITY;
        if (p.lse && lq == 0 && tok[c] < T)
            p.lse[((size_t)b * T + tok[c]) * H + g * G + hl[c]] = Ls > 0.f ? bias[c] * kLn2 : -INFINITY;
    }

    // ---- sweep 2: probabilities, o_cmp, head sums, block scores ----
    const int tl_e = threadIdx.x / TPT, je = threadIdx.x % TPT;   // emitter role
    const int t_e = tok0 + tl_e;
    const int jc_e = min(t_e, T - 1) / p.lp;
    float* score_row = p.scores + (((size_t)b * T + min(t_e, T - 1)) * p.Hkv + g) * p.n_slc;
    const float* ring_e = ring + tl_e * kRing;
    // score of block j from the ring (keys at or after kend count as 0)
    auto block_score = [&](int j, int kend) {
        const int ilo = max(0, j * R - L + 1), ihi = min(j * R + R - 1, kend - 1);
        float acc = 0.f;
        if (ihi - ilo < 8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = (ilo + q <= ihi) ? ring_e[(ilo + q) & (kRing - 1)] : 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) acc += v[q];
        } else {
            for (int i = ilo; i <= ihi; ++i) acc += ring_e[i & (kRing - 1)];
        }
        return acc;
    };
    // blocks whose last compressed key lies in tile e (keys of tile e and e-1 are in the ring)
    auto emit_tile = [&](int e) {
        const int kend = (e + 1) * kKeysPerTile;
        for (int j = e * kKeysPerTile / R + je; j < kend / R; j += TPT)
            if (t_e < T && j <= jc_e) score_row[j] = block_score(j, kend);
    };

    f32x4 oacc[WITH_O ? NDT : 1][NQ];
    if constexpr (WITH_O) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int c = 0; c < NQ; ++c) oacc[dt][c] = zero4();
    }
    auto probs_half = [&](f32x4 (&s)[4][NQ], int h, bool full, int k0) {   // p = 2^(x - lse), 0 if invisible
#pragma unroll
        for (int c = 0; c < NQ; ++c)
#pragma unroll
            for (int kt = 2 * h; kt < 2 * h + 2; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = fast_exp2(__builtin_fmaf(s[kt][c][r], sl2, -bias[c]));
                    s[kt][c][r] = (full || k0 + 16 * kt + 4 * lq + r < nv[c]) ? v : 0.f;
                }
    };
    auto pv_half = [&](const u16* vb, const f32x4 (&s)[4][NQ], int u) {   // fp16 P against fp16 V_cmp
        if constexpr (WITH_O) {
            f16x8 pb[NQ];
#pragma unroll
            for (int c = 0; c < NQ; ++c) pb[c] = pack_p_h(s[2 * u][c], s[2 * u + 1][c]);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const f16x8 a = ld8h(&vb[((u * NDT + dt) * 64 + lane) * 8]);
#pragma unroll
                for (int c = 0; c < NQ; ++c) oacc[dt][c] = mfma16h(a, pb[c], oacc[dt][c]);
            }
        }
    };
    // sums over the group's heads (in-lane over the token's tiles, then DPP over its lanes)
    // into the ring; every lane of a head group writes the same value to the same slot
    auto head_sums = [&](const f32x4 (&s)[4][NQ], int k0) {
#pragma unroll
        for (int cg = 0; cg < NQ / M::CL; ++cg) {
            // k0 is a multiple of 64, so a tile's 64 slots never wrap around the ring
            float* rt = ring + (wave * M::TPW + M::token(cg * M::CL, li)) * kRing + (k0 & (kRing - 1)) + 4 * lq;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float hs = 0.f;
#pragma unroll
                    for (int c = cg * M::CL; c < (cg + 1) * M::CL; ++c) hs += s[kt][c][r];
                    rt[16 * kt + r] = lane_group_sum<M::GL>(hs);
                }
        }
    };

    // Sweep 2 tile t: K(t) in K slot t & 1, V(t) in the V slot.  K(t+1) is copied at the
    // start of tile t, V(t+1) as soon as every wave has finished its PV products of tile t.
    auto step2 = [&](int tix, bool full) {
        copies_done();
        if (tix + 1 < ntile) issue_k(tix + 1, kslot + ((tix + 1) & 1) * KE);
        // scores of the blocks tile tix-1 completed; stored now, so they are long done by
        // the next wait on this thread's memory counter
        if (tix > 0) emit_tile(tix - 1);
        const u16* kb = kslot + (tix & 1) * KE;
        const u16* vb = vbuf;
        const int k0 = tix * kKeysPerTile;
        f32x4 s[4][NQ];
        if (full) {
            // Every key visible to every row.  The VALU work of one half rides in the shadow
            // of the other half's MFMAs: exponentials of keys 0-31 under the QK products of
            // keys 32-63, those of keys 32-63 under the PV products of keys 0-31, head sums
            // under the PV products of keys 32-63.
            qk_half(kb, s, 0);
            qk_half(kb, s, 1);
            probs_half(s, 0, true, k0);
            pv_half(vb, s, 0);
            probs_half(s, 1, true, k0);
            pv_half(vb, s, 1);
            head_sums(s, k0);
            constexpr int NMQ = 2 * NDS * NQ;           // MFMAs of a QK half
            constexpr int NMP = WITH_O ? NDT * NQ : 0;  // MFMAs of a PV half
#pragma unroll
            for (int i = 0; i < NMQ; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
#pragma unroll
            for (int i = 0; i < NMQ; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // VALU
            }
#pragma unroll
            for (int i = 0; i < NMP; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
#pragma unroll
            for (int i = 0; i < NMP; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
        } else {
            qk_half(kb, s, 0);
            qk_half(kb, s, 1);
            probs_half(s, 0, false, k0);
            probs_half(s, 1, false, k0);
            pv_half(vb, s, 0);
            pv_half(vb, s, 1);
            head_sums(s, k0);
        }
        if constexpr (WITH_O) {
            // Every wave has issued its PV products of this tile, so its reads of the V slot
            // have returned.  A bare barrier: no wait for this thread's copies and stores.
            asm volatile("s_barrier" ::: "memory");
            if (tix + 1 < ntile) issue_v(tix + 1, vbuf);
        }
    };
    // sweep 2's first tiles: every wave is done with sweep 1's buffers
    __syncthreads();
    if (ntile > 0) {
        issue_k(0, kslot);
        issue_v(0, vbuf);
    }
    for (int tix = 0; tix < nfull; ++tix) step2(tix, true);
    for (int tix = nfull; tix < ntile; ++tix) step2(tix, false);
    __syncthreads();
    if (ntile > 0) emit_tile(ntile - 1);
    // remaining blocks up to the token's own block (their later keys are invisible)
    for (int j = ntile * kKeysPerTile / R + je; j <= jc_e; j += TPT)
        if (t_e < T) score_row[j] = block_score(j, ntile * kKeysPerTile);

    if constexpr (WITH_O) {
        const float vs = ldexpf(1.0f, p.vexp[unit]);   // undo the fp16 copy's scaling
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            if (tok[c] < T) {
                float* op = p.o_cmp + (((size_t)b * T + tok[c]) * H + g * G + hl[c]) * DV + 4 * lq;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    *reinterpret_cast<float4*>(op + 16 * dt) = make_float4(
                        oacc[dt][c][0] * vs, oacc[dt][c][1] * vs, oacc[dt][c][2] * vs, oacc[dt][c][3] * vs);
            }
        }
    }
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
// own block forced).  A workgroup owns 64 tokens (a wave's 16 MFMA columns are 16 tokens);
// each lane keeps, for its column, the best kFusedMaxPicks candidates among the keys it
// holds as 64-bit entries score-key:~index (larger = better score, then lower index), so no
// score row is ever stored.  A tile is skipped when no lane of the wave has a candidate
// above its current fourth best.  The four lanes of a column merge their lists (bitonic
// top-K of two sorted lists, then a sort) across the 16- and 32-lane swaps.
template <int DK>
__global__ __launch_bounds__(256, 2) void mean_select_kernel(SelParams p) {
    constexpr int K = kFusedMaxPicks;
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

    uint64_t best[K];
#pragma unroll
    for (int i = 0; i < K; ++i) best[i] = 0ull;
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
        uint64_t c[16];
        bool improves = false;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = k0 + 16 * kt + 4 * lq + r;
                // candidates are complete earlier blocks: the own block is forced (n_local >= 1)
                const bool ok = live && fb.candidate(j);
                const uint64_t e = ok ? (((uint64_t)f2key(s[kt][r]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)j)) : 0ull;
                c[4 * kt + r] = e;
                improves |= e > best[K - 1];
            }
        if (__any(improves)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint64_t e = c[i];
#pragma unroll
                for (int q = 0; q < K; ++q) {   // insert into the descending list
                    const uint64_t hi = e > best[q] ? e : best[q];
                    e = e > best[q] ? best[q] : e;
                    best[q] = hi;
                }
            }
        }
    }
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

bool launch_mean_select(int DK, const SelParams& p, hipStream_t st) {
    constexpr int TQ = kWaves * 16;
    const int grid = xcd_grid(p.B * p.Hkv, (p.T + TQ - 1) / TQ);
    if (DK == 192) mean_select_kernel<192><<<grid, 256, 0, st>>>(p);
    else if (DK == 128) mean_select_kernel<128><<<grid, 256, 0, st>>>(p);
    else if (DK == 64) mean_select_kernel<64><<<grid, 256, 0, st>>>(p);
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
