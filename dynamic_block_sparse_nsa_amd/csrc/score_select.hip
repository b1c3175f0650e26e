// Compressed attention, block scores and group-shared top-n selection.
//
// Method (zjai.club notes, sections 5 and 8; sunshychen.top comparison): a query attends
// to the compressed blocks whose tokens are all at or before it; those attention
// probabilities, summed over the heads of the GQA group and over the compressed blocks
// that overlap a selection block, are that block's score; the group then keeps the
// forced blocks plus the best-scoring others.  MoBA mode scores a block by the inner
// product of the query with the block's mean key instead.
//
// Kernel structure (per KV group; a workgroup owns 128 query rows = 128/G tokens, each
// wave 32 rows = two 16-row MFMA column tiles):
//   cmp_stats_kernel     pass 1: S^T = K_cmp . Q^T tile by tile (64 keys staged in LDS);
//                        running max m and sum l per query row (base-2 exponentials).
//   score_select_kernel  pass 2: recompute S^T; p = 2^(x - m) / l (exact normalized
//                        probabilities, so no rescaling); o_cmp += V_cmp^T . P^T on the
//                        MFMA; head sums in fp32 via lane shuffles, accumulated per
//                        (token, block) in LDS in a fixed order; then one wave per token
//                        selects the blocks (tournament argmax over 64 lanes, 64-bit keys
//                        = score bits : ~index, so ties go to the lower index).
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace nsa {

namespace {

constexpr int kWaves = 4;
constexpr int kKeysPerTile = 64;

}  // namespace

// ---------------------------------------------------------------------------
// pass 1: per query row, m = max_i x_i and l = sum_i 2^(x_i - m), x = scale*log2(e)*q.k
// ---------------------------------------------------------------------------
template <int DK, int G>
__global__ __launch_bounds__(256) void cmp_stats_kernel(const u16* __restrict__ Q, const u16* __restrict__ Kc,
                                                        float* __restrict__ stat_m, float* __restrict__ stat_il,
                                                        float* __restrict__ lse_out, int T, int Hkv, int N, int l,
                                                        int s, float scale_log2) {
    constexpr int NQ = 2;
    constexpr int TQ = kWaves * NQ * 16 / G;
    constexpr int KSTR = DK + 8;
    constexpr int NDS = DK / 32;
    __shared__ __attribute__((aligned(16))) u16 ks[kKeysPerTile * KSTR];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int b = blockIdx.z, g = blockIdx.y;
    const int H = Hkv * G;
    const int tok0 = (gridDim.x - 1 - blockIdx.x) * TQ;

    bf16x8 qf[NQ][NDS];
    int tok[NQ], hl[NQ], nv[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const int r = (wave * NQ + c) * 16 + li;
        tok[c] = tok0 + r / G;
        hl[c] = r % G;
        const int tt = min(tok[c], T - 1);
        nv[c] = tok[c] < T ? visible_count(tok[c], l, s, N) : 0;
        const u16* qp = Q + (((size_t)b * T + tt) * H + g * G + hl[c]) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[c][ds] = ld8(qp + 32 * ds);
    }
    const int nv_max = visible_count(min(tok0 + TQ - 1, T - 1), l, s, N);
    const u16* kbase = Kc + ((size_t)b * Hkv + g) * (size_t)N * DK;

    float m[NQ], lsum[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) { m[c] = -INFINITY; lsum[c] = 0.f; }

    for (int k0 = 0; k0 < nv_max; k0 += kKeysPerTile) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < kKeysPerTile * (DK / 8); idx += 256) {
            const int row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const int kr = min(k0 + row, N - 1);
            *reinterpret_cast<uint4*>(&ks[row * KSTR + col]) =
                *reinterpret_cast<const uint4*>(kbase + (size_t)kr * DK + col);
        }
        __syncthreads();
        f32x4 sacc[4][NQ];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int c = 0; c < NQ; ++c) sacc[kt][c] = zero4();
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const bf16x8 a = ld8(&ks[(16 * kt + li) * KSTR + 32 * ds + lq * 8]);
#pragma unroll
                for (int c = 0; c < NQ; ++c) sacc[kt][c] = mfma16(a, qf[c][ds], sacc[kt][c]);
            }
        }
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            float x[16];
            float tmax = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + 16 * kt + 4 * lq + r;
                    const float v = key < nv[c] ? sacc[kt][c][r] * scale_log2 : -INFINITY;
                    x[kt * 4 + r] = v;
                    tmax = fmaxf(tmax, v);
                }
            tmax = col_max(tmax);
            const float mnew = fmaxf(m[c], tmax);
            if (mnew != -INFINITY) {
                float acc = lsum[c] * fast_exp2(m[c] - mnew);
#pragma unroll
                for (int e = 0; e < 16; ++e) acc += fast_exp2(x[e] - mnew);
                lsum[c] = acc;
                m[c] = mnew;
            }
        }
    }
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const float L = col_sum(lsum[c]);
        if (lq == 0 && tok[c] < T) {
            const size_t o = ((size_t)b * T + tok[c]) * H + g * G + hl[c];
            stat_m[o] = m[c];
            stat_il[o] = L > 0.f ? 1.0f / L : 0.f;
            if (lse_out) lse_out[o] = L > 0.f ? (m[c] + __log2f(L)) * kLn2 : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// pass 2 (MODE 0: compressed-overlap scores, optional o_cmp) and MoBA mean-key scores
// (MODE 1), followed by the selection.
// ---------------------------------------------------------------------------

template <int DK, int DV, int G, int MODE, int NQ, bool WITH_O>
__global__ __launch_bounds__(256) void score_select_kernel(SelParams p) {
    constexpr int TQ = kWaves * NQ * 16 / G;
    constexpr int KSTR = DK + 8;
    constexpr int VSTR = kKeysPerTile + 8;
    constexpr int NDS = DK / 32;
    constexpr int NDT = DV / 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    u16* ks = reinterpret_cast<u16*>(smem);
    u16* vs = ks + kKeysPerTile * KSTR;                                       // WITH_O only
    float* psum = reinterpret_cast<float*>(vs + (WITH_O ? DV * VSTR : 0));    // [TQ][64]
    float* sc = psum + TQ * kKeysPerTile;                                     // [TQ][n_slc]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int b = blockIdx.z, g = blockIdx.y;
    const int T = p.T, N = p.N;
    const int H = p.Hkv * G;
    const int tok0 = (gridDim.x - 1 - blockIdx.x) * TQ;

    bf16x8 qf[NQ][NDS];
    int tok[NQ], hl[NQ], nv[NQ];
    float rm[NQ], ril[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const int r = (wave * NQ + c) * 16 + li;
        tok[c] = tok0 + r / G;
        hl[c] = r % G;
        const int tt = min(tok[c], T - 1);
        const size_t row = ((size_t)b * T + tt) * H + g * G + hl[c];
        const u16* qp = p.Q + row * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[c][ds] = ld8(qp + 32 * ds);
        if constexpr (MODE == 0) {
            nv[c] = tok[c] < T ? visible_count(tok[c], p.l, p.s, N) : 0;
            rm[c] = p.stat_m[row];
            ril[c] = p.stat_il[row];
        } else {
            // complete blocks before the query's own block (requires l == s == lp)
            nv[c] = tok[c] < T ? min(tok[c] / p.lp, N) : 0;
            rm[c] = 0.f;
            ril[c] = 0.f;
        }
    }
    const int t_last = min(tok0 + TQ - 1, T - 1);
    const int nv_max = MODE == 0 ? visible_count(t_last, p.l, p.s, N) : min(t_last / p.lp, N);

    for (int idx = threadIdx.x; idx < TQ * p.n_slc; idx += 256) sc[idx] = 0.f;

    f32x4 oacc[WITH_O ? NDT : 1][NQ];
    if constexpr (WITH_O) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int c = 0; c < NQ; ++c) oacc[dt][c] = zero4();
    }
    const u16* kbase = p.Kc + ((size_t)b * p.Hkv + g) * (size_t)N * DK;
    const u16* vbase = WITH_O ? p.Vct + ((size_t)b * p.Hkv + g) * (size_t)DV * p.Npad : nullptr;

    for (int k0 = 0; k0 < nv_max; k0 += kKeysPerTile) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < kKeysPerTile * (DK / 8); idx += 256) {
            const int row = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const int kr = min(k0 + row, N - 1);
            *reinterpret_cast<uint4*>(&ks[row * KSTR + col]) =
                *reinterpret_cast<const uint4*>(kbase + (size_t)kr * DK + col);
        }
        if constexpr (WITH_O) {
            for (int idx = threadIdx.x; idx < DV * (kKeysPerTile / 8); idx += 256) {
                const int row = idx / (kKeysPerTile / 8), col = (idx % (kKeysPerTile / 8)) * 8;
                *reinterpret_cast<uint4*>(&vs[row * VSTR + col]) =
                    *reinterpret_cast<const uint4*>(vbase + (size_t)row * p.Npad + k0 + col);
            }
        }
        __syncthreads();

        f32x4 sacc[4][NQ];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int c = 0; c < NQ; ++c) sacc[kt][c] = zero4();
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const bf16x8 a = ld8(&ks[(16 * kt + li) * KSTR + 32 * ds + lq * 8]);
#pragma unroll
                for (int c = 0; c < NQ; ++c) sacc[kt][c] = mfma16(a, qf[c][ds], sacc[kt][c]);
            }
        }
        // probabilities (MODE 0) or raw scores (MODE 1), zero outside the visible set
#pragma unroll
        for (int c = 0; c < NQ; ++c)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + 16 * kt + 4 * lq + r;
                    float v = 0.f;
                    if (key < nv[c]) {
                        if constexpr (MODE == 0) v = fast_exp2(sacc[kt][c][r] * p.scale_log2 - rm[c]) * ril[c];
                        else v = sacc[kt][c][r];
                    }
                    sacc[kt][c][r] = v;
                }
        if constexpr (WITH_O) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                bf16x8 bh[NQ], bl[NQ];
#pragma unroll
                for (int c = 0; c < NQ; ++c) pack_p_split(sacc[2 * u][c], sacc[2 * u + 1][c], bh[c], bl[c]);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const bf16x8 a = ld8(&vs[(16 * dt + li) * VSTR + 32 * u + lq * 8]);
#pragma unroll
                    for (int c = 0; c < NQ; ++c) {
                        oacc[dt][c] = mfma16(a, bh[c], oacc[dt][c]);
                        oacc[dt][c] = mfma16(a, bl[c], oacc[dt][c]);
                    }
                }
            }
        }
        // head sums: every lane of a token's G-lane group ends with the group total
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const int tl = ((wave * NQ + c) * 16 + li) / G;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float hs = head_sum<G>(sacc[kt][c][r]);
                    if constexpr (MODE == 0) {
                        if ((li % G) == 0) psum[tl * kKeysPerTile + 16 * kt + 4 * lq + r] = hs;
                    } else {
                        const int key = k0 + 16 * kt + 4 * lq + r;
                        if ((li % G) == 0 && key < nv[c]) sc[tl * p.n_slc + key] = hs;
                    }
                }
        }
        if constexpr (MODE == 0) {
            __syncthreads();
            // blocks touched by keys k0 .. k0+63: block j gets keys i with
            // i*s <= (j+1)*lp - 1 and i*s + l - 1 >= j*lp, added in ascending i
            const int jlo = (k0 * p.s) / p.lp;
            const int jhi = min(((k0 + kKeysPerTile - 1) * p.s + p.l - 1) / p.lp, p.n_slc - 1);
            const int nj = jhi - jlo + 1;
            for (int idx = threadIdx.x; idx < TQ * nj; idx += 256) {
                const int tl = idx / nj, j = jlo + idx % nj;
                const int ilo = max(k0, (j * p.lp - p.l + 1 + p.s - 1 >= 0) ? (j * p.lp - p.l + 1 + p.s - 1) / p.s : 0);
                const int ihi = min(k0 + kKeysPerTile - 1, (j * p.lp + p.lp - 1) / p.s);
                float acc = 0.f;
                for (int i = ilo; i <= ihi; ++i) acc += psum[tl * kKeysPerTile + (i - k0)];
                sc[tl * p.n_slc + j] += acc;
            }
        }
    }
    __syncthreads();

    if constexpr (WITH_O) {
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            if (tok[c] < T) {
                float* op = p.o_cmp + (((size_t)b * T + tok[c]) * H + g * G + hl[c]) * DV + 4 * lq;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    *reinterpret_cast<float4*>(op + 16 * dt) =
                        make_float4(oacc[dt][c][0], oacc[dt][c][1], oacc[dt][c][2], oacc[dt][c][3]);
            }
        }
    }
    for (int tl = wave; tl < TQ; tl += kWaves) {
        const int t = tok0 + tl;
        if (t >= T) break;
        select_blocks_wave(sc + tl * p.n_slc, t / p.lp, p.top_n, p.n_init, p.n_local,
                           p.sel + (((size_t)b * T + t) * p.Hkv + g) * p.top_n);
    }
}

// Selection from caller scores [B,T,Hkv,n_slc]: one wave per (b, t, g).
__global__ __launch_bounds__(256) void select_from_scores_kernel(const float* __restrict__ scores,
                                                                 int32_t* __restrict__ sel, int T, int Hkv,
                                                                 int n_slc, int lp, int top_n, int n_init,
                                                                 int n_local, long rows) {
    const long row = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int t = (int)((row / Hkv) % T);
    select_blocks_wave(scores + row * n_slc, t / lp, top_n, n_init, n_local, sel + row * top_n);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {
template <int DK, int G>
void stats_g(const u16* Q, const u16* Kc, float* m, float* il, float* lse, int B, int T, int Hkv, int N, int l,
             int s, float sl2, hipStream_t st) {
    constexpr int TQ = kWaves * 2 * 16 / G;
    dim3 grid((T + TQ - 1) / TQ, Hkv, B);
    cmp_stats_kernel<DK, G><<<grid, 256, 0, st>>>(Q, Kc, m, il, lse, T, Hkv, N, l, s, sl2);
}

template <int DK, int DV, int G, int MODE, int NQ, bool WITH_O>
void select_g(const SelParams& p, int B, hipStream_t st) {
    constexpr int TQ = kWaves * NQ * 16 / G;
    dim3 grid((p.T + TQ - 1) / TQ, p.Hkv, B);
    const size_t lds = score_select_lds_bytes(DK, DV, G, MODE, NQ, WITH_O, p.n_slc);
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(score_select_kernel<DK, DV, G, MODE, NQ, WITH_O>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    score_select_kernel<DK, DV, G, MODE, NQ, WITH_O><<<grid, 256, lds, st>>>(p);
}

template <int DK, int DV, int G>
bool select_dk(int mode, bool with_o, const SelParams& p, int B, hipStream_t st) {
    if (mode == 0) {
        if (with_o) select_g<DK, DV, G, 0, 2, true>(p, B, st);
        else select_g<DK, DV, G, 0, 2, false>(p, B, st);
    } else {
        select_g<DK, DV, G, 1, (G == 1 ? 1 : 2), false>(p, B, st);
    }
    return true;
}
}  // namespace

size_t score_select_lds_bytes(int DK, int DV, int G, int mode, int NQ, bool with_o, int n_slc) {
    const int TQ = kWaves * NQ * 16 / G;
    size_t bytes = (size_t)kKeysPerTile * (DK + 8) * 2;
    if (with_o) bytes += (size_t)DV * (kKeysPerTile + 8) * 2;
    bytes += (size_t)TQ * kKeysPerTile * 4;
    bytes += (size_t)TQ * n_slc * 4;
    (void)mode;
    return bytes;
}

int score_select_nq(int G, int mode) { return (mode == 1 && G == 1) ? 1 : 2; }

#define NSA_G_SWITCH(G, ...)                                       \
    switch (G) {                                                   \
        case 1: { constexpr int GG = 1; __VA_ARGS__; } break;      \
        case 2: { constexpr int GG = 2; __VA_ARGS__; } break;      \
        case 4: { constexpr int GG = 4; __VA_ARGS__; } break;      \
        case 8: { constexpr int GG = 8; __VA_ARGS__; } break;      \
        case 16: { constexpr int GG = 16; __VA_ARGS__; } break;    \
        default: return false;                                     \
    }

bool launch_cmp_stats(const u16* Q, const u16* Kc, float* m, float* il, float* lse, int B, int T, int Hkv, int G,
                      int DK, int N, int l, int s, float sl2, hipStream_t st) {
    if (DK == 192) { NSA_G_SWITCH(G, stats_g<192, GG>(Q, Kc, m, il, lse, B, T, Hkv, N, l, s, sl2, st)); }
    else if (DK == 128) { NSA_G_SWITCH(G, stats_g<128, GG>(Q, Kc, m, il, lse, B, T, Hkv, N, l, s, sl2, st)); }
    else if (DK == 64) { NSA_G_SWITCH(G, stats_g<64, GG>(Q, Kc, m, il, lse, B, T, Hkv, N, l, s, sl2, st)); }
    else return false;
    return true;
}

bool launch_score_select(int mode, bool with_o, int DK, int DV, int G, const SelParams& p, int B, hipStream_t st) {
    if (DK == 192 && DV == 128) { NSA_G_SWITCH(G, return select_dk<192, 128, GG>(mode, with_o, p, B, st)); }
    if (DK == 128 && DV == 128) { NSA_G_SWITCH(G, return select_dk<128, 128, GG>(mode, with_o, p, B, st)); }
    if (DK == 64 && DV == 64) { NSA_G_SWITCH(G, return select_dk<64, 64, GG>(mode, with_o, p, B, st)); }
    return false;
}

void launch_select_from_scores(const float* scores, int32_t* sel, int B, int T, int Hkv, int n_slc, int lp,
                               int top_n, int n_init, int n_local, hipStream_t st) {
    const long rows = (long)B * T * Hkv;
    const long blocks = (rows + kWaves - 1) / kWaves;
    select_from_scores_kernel<<<(unsigned)blocks, 256, 0, st>>>(scores, sel, T, Hkv, n_slc, lp, top_n, n_init,
                                                                n_local, rows);
}

}  // namespace nsa
