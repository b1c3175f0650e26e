// Compressed attention + block scores of one workgroup tile: the device body shared by
// cmp_attn_kernel (score_select.hip) and the fused prefill kernel (prefill.hip).
//
// Method (zjai.club notes, sections 5 and 8; sunshychen.top comparison): a query attends
// to the compressed blocks whose tokens are all at or before it; those attention
// probabilities, summed over the heads of the GQA group and over the compressed blocks
// that overlap a selection block, are that block's score.
//
// A workgroup owns 128 query rows = 128/G tokens of one KV group, each wave two 16-column
// MFMA tiles laid out by QMap so a token's heads share lanes and tiles.
//   sweep 1: S^T = K_cmp . Q^T over 64-key tiles, a per-lane lazily moved reference and sum, combined
//            into the log-sum-exp b (base 2) of every query row.
//   sweep 2: the same S^T again; p = 2^(x - b) are the normalized probabilities (nothing is
//            rescaled afterwards); o_cmp += V_cmp^T.P^T on the MFMA; p summed over the
//            group's heads in fp32 (in-lane + DPP) into a per-token ring in LDS; one tile
//            later, every selection block whose last compressed key is complete gets its
//            score (sum over its overlapping compressed blocks, ascending key order) written
//            to the score workspace.  The compressed keys and values are read in MFMA
//            fragment order (tile_cmp_kernel), so a tile is one contiguous span copied to
//            LDS while the previous tile is computed.
// Block j of l' tokens takes compressed blocks i with j*R - L + 1 <= i <= j*R + R - 1,
// R = l'/s and L = l/s, i.e. every compressed block whose token span meets block j.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace nsa {

namespace cmpk {
constexpr int kWaves = 4;
constexpr int kKeysPerTile = 64;
constexpr int kRing = 4 * kKeysPerTile;  // per-token ring: the tile being written and the two before it
}  // namespace cmpk

// Waves per workgroup of the compressed-attention kernel.  Two workgroups share a CU
// (72 KB of LDS each for G = 16), so the two waves on a SIMD belong to different
// workgroups and drift apart: one's MFMAs overlap the other's VALU work.
__host__ __device__ constexpr int cmp_waves(int) { return 4; }

// Tokens per workgroup tile of the compressed-attention body.
__host__ __device__ constexpr int cmp_tile_tokens(int G) { return cmp_waves(G) * (G == 1 ? 1 : 2) * 16 / G; }

// ---------------------------------------------------------------------------
// Compressed attention (log-sum-exp, o_cmp) and block scores of one workgroup's tile of
// TQ = WAVES * NQ * 16 / G tokens starting at tok0 (a multiple of TQ) of KV group `unit`.  Every wave of the workgroup must call it.  Ends with the workgroup's
// score rows written to p.scores and o_cmp / lse to p.o_cmp / p.lse; the last step is a
// barrier followed by each thread's own stores only, so a caller that reads those rows back
// must place a barrier first.
// ---------------------------------------------------------------------------
template <int DK, int DV, int G, int NQ, bool WITH_O>
__device__ __forceinline__ void cmp_attn_tile(const SelParams& p, int unit, int tok0, unsigned char* smem) {
    constexpr int WAVES = cmp_waves(G);
    constexpr int NT = 64 * WAVES;             // threads
    constexpr int TQ = WAVES * NQ * 16 / G;    // tokens per workgroup
    constexpr int NDS = DK / 32, NDT = DV / 16;
    constexpr int KE = 4 * NDS * 512;          // K elements of a 64-key tile (fragment order)
    constexpr int VE = WITH_O ? 2 * NDT * 512 : 0;
    constexpr int TPT = NT / TQ;               // threads per token when emitting block scores
    // LDS (smem, cmp_attn_lds_bytes): two K tile slots, one V tile slot, then the ring [TQ][cmpk::kRing]
    u16* kslot = reinterpret_cast<u16*>(smem);   // [2][KE]
    u16* vbuf = kslot + 2 * KE;                   // [VE]
    float* ring = reinterpret_cast<float*>(vbuf + VE);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar addressing
    const int li = lane & 15, lq = lane >> 4;
    const int T = p.T, N = p.N;
    const int b = unit / p.Hkv, g = unit % p.Hkv;
    const int H = p.Hkv * G;
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
    const int ntile = (nv_max + cmpk::kKeysPerTile - 1) / cmpk::kKeysPerTile;
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

    // ---- sweep 1: per-lane reference and sum over the lane's keys ----
    // m is a lazily moved reference (log2 units) and lsum the lane's sum of 2^(x - m).  The
    // common path only adds 2^(x - m) (no maximum, no rescale); a lane's reference moves
    // when the sum of the values just added leaves [0, 2^32] (the first keys, where
    // m = -inf, or a value about 2^28 above m), which is rare after the first tile.  fp32
    // keeps the sum's relative precision at any such scale.
    float m[NQ], lsum[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) { m[c] = -INFINITY; lsum[c] = 0.f; }
    const int nfull = nv_min / cmpk::kKeysPerTile;   // tiles [0, nfull) are visible to every row
    auto k1buf = [&](int buf) { return kslot + buf * KE; };
    constexpr float kOver = 0x1p32f;
    // sum of 2^(x - m) over the lane's 8 values of key sub-tiles 2h, 2h+1, column c
    auto half_sum = [&](const f32x4 (&s)[4][NQ], int h, int c) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += fast_exp2(__builtin_fmaf(s[2 * h + (e >> 2)][c][e & 3], sl2, -m[c]));
        return acc;
    };
    // acc holds the sums of half (sa, ha) and, if two, of half (sb, hb) against m: fold them
    // into lsum, first moving the reference of the columns whose sum left the range and
    // summing those halves again against it
    auto settle = [&](const f32x4 (&sa)[4][NQ], int ha, const f32x4 (&sb)[4][NQ], int hb, bool two,
                      float (&acc)[NQ]) {
        bool over = false;
#pragma unroll
        for (int c = 0; c < NQ; ++c) over |= !(acc[c] <= kOver);
        if (__any(over)) {   // wave-uniform branch
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                if (acc[c] <= kOver) continue;
                float tmax = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    tmax = fmaxf(tmax, sa[2 * ha + (e >> 2)][c][e & 3]);
                    if (two) tmax = fmaxf(tmax, sb[2 * hb + (e >> 2)][c][e & 3]);
                }
                const float mnew = fmaxf(m[c], tmax * sl2);
                float a = 0.f;
                if (mnew != -INFINITY) {
                    lsum[c] = m[c] == -INFINITY ? 0.f : lsum[c] * fast_exp2(m[c] - mnew);
                    m[c] = mnew;
                    a = half_sum(sa, ha, c);
                    if (two) a += half_sum(sb, hb, c);
                }
                acc[c] = a;
            }
        }
#pragma unroll
        for (int c = 0; c < NQ; ++c) lsum[c] += acc[c];
    };
    auto tile_start1 = [&](int tix) {   // tile tix landed; copy of tile tix + 1 under way
        copies_done();
        if (tix + 1 < ntile) issue_k(tix + 1, k1buf(nb ^ 1));
        const u16* kb = k1buf(nb);
        nb ^= 1;
        return kb;
    };
    if (ntile > 0) issue_k(0, kslot);
    // Tiles visible to every row, software-pipelined: the sums of each half tile are taken
    // under the QK products of the next half (across the tile barrier too).
    if (nfull > 0) {
        f32x4 s[4][NQ];
        const u16* kb = tile_start1(0);
        qk_half(kb, s, 0);
        qk_half(kb, s, 1);
        {
            float acc[NQ];
#pragma unroll
            for (int c = 0; c < NQ; ++c) acc[c] = half_sum(s, 0, c);
            settle(s, 0, s, 0, false, acc);
        }
        for (int tix = 1; tix < nfull; ++tix) {
            f32x4 prev[4][NQ];
#pragma unroll
            for (int c = 0; c < NQ; ++c) { prev[2][c] = s[2][c]; prev[3][c] = s[3][c]; }
            kb = tile_start1(tix);
            float acc[NQ];
            qk_half(kb, s, 0);
#pragma unroll
            for (int c = 0; c < NQ; ++c) acc[c] = half_sum(prev, 1, c);
            qk_half(kb, s, 1);
#pragma unroll
            for (int c = 0; c < NQ; ++c) acc[c] += half_sum(s, 0, c);
            constexpr int NMQ = 2 * NDS * NQ;   // MFMAs of a QK half
#pragma unroll
            for (int i = 0; i < 2 * NMQ; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // VALU
            }
            settle(prev, 1, s, 0, true, acc);
        }
        float acc[NQ];
#pragma unroll
        for (int c = 0; c < NQ; ++c) acc[c] = half_sum(s, 1, c);
        settle(s, 1, s, 1, false, acc);
    }
    // tiles with keys invisible to some rows
    for (int tix = nfull; tix < ntile; ++tix) {
        const u16* kb = tile_start1(tix);
        f32x4 s[4][NQ];
        qk_half(kb, s, 0);
        qk_half(kb, s, 1);
        const int k0 = tix * cmpk::kKeysPerTile;
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
    const float* ring_e = ring + tl_e * cmpk::kRing;
    // score of block j from the ring (keys at or after kend count as 0)
    auto block_score = [&](int j, int kend) {
        const int ilo = max(0, j * R - L + 1), ihi = min(j * R + R - 1, kend - 1);
        float acc = 0.f;
        if (ihi - ilo < 8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = (ilo + q <= ihi) ? ring_e[(ilo + q) & (cmpk::kRing - 1)] : 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) acc += v[q];
        } else {
            for (int i = ilo; i <= ihi; ++i) acc += ring_e[i & (cmpk::kRing - 1)];
        }
        return acc;
    };
    // blocks whose last compressed key lies in tile e (keys of tile e and e-1 are in the ring)
    auto emit_tile = [&](int e) {
        const int kend = (e + 1) * cmpk::kKeysPerTile;
        for (int j = e * cmpk::kKeysPerTile / R + je; j < kend / R; j += TPT)
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
            float* rt = ring + (wave * M::TPW + M::token(cg * M::CL, li)) * cmpk::kRing + (k0 & (cmpk::kRing - 1)) + 4 * lq;
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

    // The quad geometry (l' = 4s and l = 2s, as in the 64 / 32 / 16 workloads): block j covers
    // compressed keys 4j-1 .. 4j+3, and keys 4j .. 4j+3 are exactly the four C-fragment rows a
    // lane holds in one 16-key group (lane quarter lq = j mod 4).  Per 16-key group a lane adds
    // its own four probabilities (of its heads' columns) and that of key 4j-1 - held by the
    // same column one quarter below, or for lq = 0 by quarter 3 of the previous 16-key group
    // or of the previous tile - and one reduction over the group's lanes gives the block
    // score: no ring, no LDS, no one-tile delay, one cross-lane sum per block instead of one
    // per key.
    float carry[NQ / M::CL];   // lanes lq = 0: the previous tile's last key (this lane's heads)
#pragma unroll
    for (int cg = 0; cg < NQ / M::CL; ++cg) carry[cg] = 0.f;
    auto quad_scores = [&](const f32x4 (&s)[4][NQ], int k0) {
#pragma unroll
        for (int cg = 0; cg < NQ / M::CL; ++cg) {
            float own[4], sh[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] = 0.f;
#pragma unroll
                    for (int c = cg * M::CL; c < (cg + 1) * M::CL; ++c) v[r] += s[kt][c][r];
                }
                own[kt] = (v[0] + v[1]) + (v[2] + v[3]);
                sh[kt] = __shfl(v[3], (lane + 48) & 63);   // key 4j-1 from quarter lq-1 (mod 4)
            }
            const int tl = wave * M::TPW + M::token(cg * M::CL, li);
            const int t = tok0 + tl;
            const int jc = min(t, T - 1) / p.lp;
            float* row = p.scores + (((size_t)b * T + min(t, T - 1)) * p.Hkv + g) * p.n_slc;
            const bool writer = (li % M::GL) == 0 && t < T;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const float prev = lq > 0 ? sh[kt] : (kt > 0 ? sh[kt - 1] : carry[cg]);
                const float sc = lane_group_sum<M::GL>(prev + own[kt]);
                const int j = k0 / 4 + 4 * kt + lq;
                if (writer && j <= jc && j < p.n_slc) row[j] = sc;
            }
            carry[cg] = sh[3];
        }
    };
    // blocks past the last tile up to the own block: block 16 * ntile takes the last tile's
    // last key, later ones no visible key
    auto quad_tail = [&]() {
#pragma unroll
        for (int cg = 0; cg < NQ / M::CL; ++cg) {
            const float last = lane_group_sum<M::GL>(carry[cg]);   // all lanes take part
            const int t = tok0 + wave * M::TPW + M::token(cg * M::CL, li);
            if ((li % M::GL) != 0 || lq != 0 || t >= T) continue;
            const int jc = t / p.lp;
            float* row = p.scores + (((size_t)b * T + t) * p.Hkv + g) * p.n_slc;
            for (int j = ntile * cmpk::kKeysPerTile / 4; j <= jc; ++j)
                row[j] = j == ntile * cmpk::kKeysPerTile / 4 ? last : 0.f;
        }
    };
    const bool quad = R == 4 && L == 2;

    // Sweep 2 tile t: K(t) in K slot t & 1, V(t) in the V slot.  K(t+1) is copied at the
    // start of tile t, V(t+1) as soon as every wave has finished its PV products of tile t.
    auto step2 = [&](int tix, bool full, auto quad_tag) {
        constexpr bool QUAD = decltype(quad_tag)::value;
        copies_done();
        if (tix + 1 < ntile) issue_k(tix + 1, kslot + ((tix + 1) & 1) * KE);
        // scores of the blocks tile tix-1 completed; stored now, so they are long done by
        // the next wait on this thread's memory counter
        if (!QUAD && tix > 0) emit_tile(tix - 1);
        const u16* kb = kslot + (tix & 1) * KE;
        const u16* vb = vbuf;
        const int k0 = tix * cmpk::kKeysPerTile;
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
            if constexpr (QUAD) quad_scores(s, k0);
            else head_sums(s, k0);
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
            if constexpr (QUAD) quad_scores(s, k0);
            else head_sums(s, k0);
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
    if (quad) {
        using Q = std::integral_constant<bool, true>;
        for (int tix = 0; tix < nfull; ++tix) step2(tix, true, Q{});
        for (int tix = nfull; tix < ntile; ++tix) step2(tix, false, Q{});
        __syncthreads();
        quad_tail();
    } else {
        using Q = std::integral_constant<bool, false>;
        for (int tix = 0; tix < nfull; ++tix) step2(tix, true, Q{});
        for (int tix = nfull; tix < ntile; ++tix) step2(tix, false, Q{});
        __syncthreads();
        if (ntile > 0) emit_tile(ntile - 1);
        // remaining blocks up to the token's own block (their later keys are invisible)
        for (int j = ntile * cmpk::kKeysPerTile / R + je; j <= jc_e; j += TPT)
            if (t_e < T) score_row[j] = block_score(j, ntile * cmpk::kKeysPerTile);
    }

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

}  // namespace nsa
