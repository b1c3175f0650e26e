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
//   cmp_stats_kernel   pass 1: S^T = K_cmp . Q^T, 64 compressed keys per LDS tile; running
//                      max m and sum l per query row (base-2 exponentials).
//   cmp_scores_kernel  pass 2: recompute S^T; p = 2^(x - m) / l (the exact normalized
//                      probabilities, so nothing is rescaled); o_cmp += V_cmp^T . P^T on
//                      the MFMA (P split into bf16 high and low parts); sums over the
//                      group's heads in fp32 (in-lane + DPP) into a per-key ring in LDS;
//                      each block's score (sum over its overlapping compressed blocks,
//                      ascending key order) is written to the score workspace once the
//                      tile holding its last key is done.  Mode 1 writes the head-summed
//                      raw dot products with the mean keys directly.
//   select_kernel      one wave per (token, group): the shared top-n from the scores.
// Block j of l' tokens takes compressed blocks i with j*R - L + 1 <= i <= j*R + R - 1,
// R = l'/s and L = l/s, i.e. every compressed block whose token span meets block j.
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace nsa {

namespace {

constexpr int kWaves = 4;
constexpr int kKeysPerTile = 64;
constexpr int kRing = 2 * kKeysPerTile;  // per-token head-sum ring: this tile and the previous one

// Copy rows [k0, k0+64) of a [N][D] bf16 matrix (rows clamped to N-1) into LDS rows of
// stride LSTR.  All global loads are issued before the first LDS store.
template <int D, int LSTR>
__device__ __forceinline__ void stage_rows(const u16* __restrict__ src, int k0, int N, u16* dst) {
    constexpr int PER_ROW = D / 8;
    constexpr int TOTAL = kKeysPerTile * PER_ROW;
    constexpr int ITERS = (TOTAL + 255) / 256;
    uint4 v[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int row = idx / PER_ROW, col = (idx % PER_ROW) * 8;
        if (TOTAL % 256 == 0 || idx < TOTAL)
            v[i] = *reinterpret_cast<const uint4*>(src + (size_t)min(k0 + row, N - 1) * D + col);
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int row = idx / PER_ROW, col = (idx % PER_ROW) * 8;
        if (TOTAL % 256 == 0 || idx < TOTAL) *reinterpret_cast<uint4*>(&dst[row * LSTR + col]) = v[i];
    }
}

// Rows [k0, k0+64) of a [N][D] bf16 matrix (rows clamped to N-1) held in registers
// between a load issued before a tile's math and the LDS store after it.
template <int D, int LSTR>
struct RowTile {
    static constexpr int PER_ROW = D / 8;
    static constexpr int TOTAL = kKeysPerTile * PER_ROW;
    static constexpr int ITERS = (TOTAL + 255) / 256;
    u32x4 v[ITERS];
    __device__ __forceinline__ void load(const u16* __restrict__ src, int k0, int N) {
#pragma unroll
        for (int i = 0; i < ITERS; ++i) {
            const int idx = threadIdx.x + 256 * i;
            const int row = idx / PER_ROW, col = (idx % PER_ROW) * 8;
            if (TOTAL % 256 == 0 || idx < TOTAL)
                v[i] = *reinterpret_cast<const u32x4*>(src + (size_t)min(k0 + row, N - 1) * D + col);
        }
    }
    __device__ __forceinline__ void store(u16* dst) const {
#pragma unroll
        for (int i = 0; i < ITERS; ++i) {
            const int idx = threadIdx.x + 256 * i;
            const int row = idx / PER_ROW, col = (idx % PER_ROW) * 8;
            if (TOTAL % 256 == 0 || idx < TOTAL) *reinterpret_cast<u32x4*>(&dst[row * LSTR + col]) = v[i];
        }
    }
};

// Copy columns [k0, k0+64) of a [D][Npad] bf16 matrix (transposed values) into LDS rows
// of stride LSTR.  All global loads are issued before the first LDS store.
template <int D, int LSTR>
__device__ __forceinline__ void stage_cols(const u16* __restrict__ src, int k0, int Npad, u16* dst) {
    constexpr int PER_ROW = kKeysPerTile / 8;
    constexpr int TOTAL = D * PER_ROW;
    constexpr int ITERS = (TOTAL + 255) / 256;
    uint4 v[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int row = idx / PER_ROW, col = (idx % PER_ROW) * 8;
        if (TOTAL % 256 == 0 || idx < TOTAL)
            v[i] = *reinterpret_cast<const uint4*>(src + (size_t)row * Npad + k0 + col);
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int row = idx / PER_ROW, col = (idx % PER_ROW) * 8;
        if (TOTAL % 256 == 0 || idx < TOTAL) *reinterpret_cast<uint4*>(&dst[row * LSTR + col]) = v[i];
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// pass 1: per query row, m = max_i x_i and l = sum_i 2^(x_i - m), x = scale*log2(e)*q.k
// ---------------------------------------------------------------------------
template <int DK, int G>
__global__ __launch_bounds__(256, 3) void cmp_stats_kernel(const u16* __restrict__ Q, const u16* __restrict__ Kc,
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

    using M = QMap<G, NQ>;
    bf16x8 qf[NQ][NDS];
    int tok[NQ], hl[NQ], nv[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        tok[c] = tok0 + wave * M::TPW + M::token(c, li);
        hl[c] = M::head(c, li);
        const int tt = min(tok[c], T - 1);
        nv[c] = tok[c] < T ? visible_count(tok[c], l, s, N) : 0;
        const u16* qp = Q + (((size_t)b * T + tt) * H + g * G + hl[c]) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[c][ds] = ld8(qp + 32 * ds);
    }
    const int nv_max = visible_count(min(tok0 + TQ - 1, T - 1), l, s, N);
    const int nv_min = visible_count(min(tok0, T - 1), l, s, N);
    const u16* kbase = Kc + ((size_t)b * Hkv + g) * (size_t)N * DK;

    float m[NQ], lsum[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) { m[c] = -INFINITY; lsum[c] = 0.f; }

    // the next tile's rows are in flight (registers) while this tile is computed
    RowTile<DK, KSTR> pre;
    pre.load(kbase, 0, N);
    for (int k0 = 0; k0 < nv_max; k0 += kKeysPerTile) {
        __syncthreads();
        pre.store(ks);
        __syncthreads();
        pre.load(kbase, k0 + kKeysPerTile, N);
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
        const bool full = k0 + kKeysPerTile <= nv_min;  // no key of this tile is masked
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            float x[16];
            float tmax = -INFINITY;
            if (full) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    x[e] = sacc[e >> 2][c][e & 3] * scale_log2;
                    tmax = fmaxf(tmax, x[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = k0 + 16 * (e >> 2) + 4 * lq + (e & 3);
                    x[e] = key < nv[c] ? sacc[e >> 2][c][e & 3] * scale_log2 : -INFINITY;
                    tmax = fmaxf(tmax, x[e]);
                }
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
// pass 2: block scores (+ o_cmp) into the score workspace
// ---------------------------------------------------------------------------
template <int DK, int DV, int G, int MODE, int NQ, bool WITH_O>
__global__ __launch_bounds__(256, 2) void cmp_scores_kernel(SelParams p) {
    constexpr int TQ = kWaves * NQ * 16 / G;
    constexpr int KSTR = DK + 8;
    constexpr int VSTR = kKeysPerTile + 8;
    constexpr int NDS = DK / 32;
    constexpr int NDT = DV / 16;
    constexpr int TPT = 256 / TQ;  // threads per token when emitting block scores
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    u16* ks = reinterpret_cast<u16*>(smem);
    u16* vs = ks + kKeysPerTile * KSTR;                                     // WITH_O only
    float* ring = reinterpret_cast<float*>(vs + (WITH_O ? DV * VSTR : 0));  // [TQ][kRing] (mode 0)

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int b = blockIdx.z, g = blockIdx.y;
    const int T = p.T, N = p.N;
    const int H = p.Hkv * G;
    const int tok0 = (gridDim.x - 1 - blockIdx.x) * TQ;
    const int R = p.lp / p.s, L = p.l / p.s;

    using M = QMap<G, NQ>;
    bf16x8 qf[NQ][NDS];
    int tok[NQ], hl[NQ], nv[NQ];
    float rm[NQ], ril[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        tok[c] = tok0 + wave * M::TPW + M::token(c, li);
        hl[c] = M::head(c, li);
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
    const int nv_min = MODE == 0 ? visible_count(min(tok0, T - 1), p.l, p.s, N) : min(min(tok0, T - 1) / p.lp, N);

    // emitter role: thread -> (token tl_e, first block offset je)
    const int tl_e = threadIdx.x / TPT, je = threadIdx.x % TPT;
    const int t_e = tok0 + tl_e;
    const int jc_e = min(t_e, T - 1) / p.lp;
    float* score_row = p.scores + (((size_t)b * T + min(t_e, T - 1)) * p.Hkv + g) * p.n_slc;
    const float* ring_e = ring + tl_e * kRing;
    // score of block j from the ring (keys at or after `kend` count as 0)
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

    f32x4 oacc[WITH_O ? NDT : 1][NQ];
    if constexpr (WITH_O) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int c = 0; c < NQ; ++c) oacc[dt][c] = zero4();
    }
    const u16* kbase = p.Kc + ((size_t)b * p.Hkv + g) * (size_t)N * DK;
    const u16* vbase = WITH_O ? p.Vct + ((size_t)b * p.Hkv + g) * (size_t)DV * p.Npad : nullptr;

    int k0 = 0;
    for (; k0 < nv_max; k0 += kKeysPerTile) {
        __syncthreads();
        if constexpr (WITH_O) stage_cols<DV, VSTR>(vbase, k0, p.Npad, vs);
        stage_rows<DK, KSTR>(kbase, k0, N, ks);
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
        // probabilities (mode 0) or raw scores (mode 1), zero outside the visible set
        if (k0 + kKeysPerTile <= nv_min) {
            if constexpr (MODE == 0) {
#pragma unroll
                for (int c = 0; c < NQ; ++c)
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            sacc[kt][c][r] = fast_exp2(sacc[kt][c][r] * p.scale_log2 - rm[c]) * ril[c];
            }
        } else {
#pragma unroll
            for (int c = 0; c < NQ; ++c)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = k0 + 16 * kt + 4 * lq + r;
                        float v = sacc[kt][c][r];
                        if constexpr (MODE == 0) v = fast_exp2(v * p.scale_log2 - rm[c]) * ril[c];
                        sacc[kt][c][r] = key < nv[c] ? v : 0.f;
                    }
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
        // sums over the group's heads: in-lane over the token's tiles, then DPP over its lanes
#pragma unroll
        for (int cg = 0; cg < NQ / M::CL; ++cg) {
            const int tl = wave * M::TPW + M::token(cg * M::CL, li);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float hs = 0.f;
#pragma unroll
                    for (int c = cg * M::CL; c < (cg + 1) * M::CL; ++c) hs += sacc[kt][c][r];
                    hs = lane_group_sum<M::GL>(hs);
                    if ((li % M::GL) == 0) {
                        const int key = k0 + 16 * kt + 4 * lq + r;
                        if constexpr (MODE == 0) {
                            ring[tl * kRing + (key & (kRing - 1))] = hs;
                        } else {
                            const int t = tok0 + tl;
                            if (key < nv[cg * M::CL])
                                p.scores[(((size_t)b * T + t) * p.Hkv + g) * p.n_slc + key] = hs;
                        }
                    }
                }
        }
        if constexpr (MODE == 0) {
            __syncthreads();
            // blocks whose last compressed key lies in this tile are complete
            const int kend = k0 + kKeysPerTile;
            for (int j = k0 / R + je; j < kend / R; j += TPT)
                if (t_e < T && j <= jc_e) score_row[j] = block_score(j, kend);
        }
    }
    if constexpr (MODE == 0) {
        __syncthreads();
        // remaining blocks up to the token's own block (their later keys are invisible)
        for (int j = k0 / R + je; j <= jc_e; j += TPT)
            if (t_e < T) score_row[j] = block_score(j, k0);
    }

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
template <int DK, int G>
void stats_g(const u16* Q, const u16* Kc, float* m, float* il, float* lse, int B, int T, int Hkv, int N, int l,
             int s, float sl2, hipStream_t st) {
    constexpr int TQ = kWaves * 2 * 16 / G;
    dim3 grid((T + TQ - 1) / TQ, Hkv, B);
    cmp_stats_kernel<DK, G><<<grid, 256, 0, st>>>(Q, Kc, m, il, lse, T, Hkv, N, l, s, sl2);
}

template <int DK, int DV, int G, int MODE, int NQ, bool WITH_O>
void scores_g(const SelParams& p, int B, hipStream_t st) {
    constexpr int TQ = kWaves * NQ * 16 / G;
    dim3 grid((p.T + TQ - 1) / TQ, p.Hkv, B);
    const size_t lds = score_select_lds_bytes(DK, DV, G, MODE, NQ, WITH_O, p.n_slc);
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(cmp_scores_kernel<DK, DV, G, MODE, NQ, WITH_O>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    cmp_scores_kernel<DK, DV, G, MODE, NQ, WITH_O><<<grid, 256, lds, st>>>(p);
}

template <int DK, int DV, int G>
bool scores_dk(int mode, bool with_o, const SelParams& p, int B, hipStream_t st) {
    if (mode == 0) {
        if (with_o) scores_g<DK, DV, G, 0, 2, true>(p, B, st);
        else scores_g<DK, DV, G, 0, 2, false>(p, B, st);
    } else {
        scores_g<DK, DV, G, 1, (G == 1 ? 1 : 2), false>(p, B, st);
    }
    return true;
}
}  // namespace

size_t score_select_lds_bytes(int DK, int DV, int G, int mode, int NQ, bool with_o, int n_slc) {
    (void)n_slc;
    const int TQ = kWaves * NQ * 16 / G;
    size_t bytes = (size_t)kKeysPerTile * (DK + 8) * 2;
    if (with_o) bytes += (size_t)DV * (kKeysPerTile + 8) * 2;
    if (mode == 0) bytes += (size_t)TQ * kRing * 4;
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

bool launch_cmp_scores(int mode, bool with_o, int DK, int DV, int G, const SelParams& p, int B, hipStream_t st) {
    if (DK == 192 && DV == 128) { NSA_G_SWITCH(G, return scores_dk<192, 128, GG>(mode, with_o, p, B, st)); }
    if (DK == 128 && DV == 128) { NSA_G_SWITCH(G, return scores_dk<128, 128, GG>(mode, with_o, p, B, st)); }
    if (DK == 64 && DV == 64) { NSA_G_SWITCH(G, return scores_dk<64, 64, GG>(mode, with_o, p, B, st)); }
    return false;
}

void launch_select_from_scores(const float* scores, int32_t* sel, int B, int T, int Hkv, int n_slc, int lp,
                               int top_n, int n_init, int n_local, hipStream_t st) {
    const long rows = (long)B * T * Hkv;
    const long blocks = (rows + kWaves - 1) / kWaves;
    NSA_NU_SWITCH(n_slc, select_from_scores_kernel<NU><<<(unsigned)blocks, 256, 0, st>>>(
                             scores, sel, T, Hkv, n_slc, lp, top_n, n_init, n_local, rows));
}

}  // namespace nsa
