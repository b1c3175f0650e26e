// Backward pass of the three branches and of the linear block map (zjai.club notes, section 4:
// the method trains natively, forward and backward; section 14: the top-k choice has no
// derivative, so the selection is held fixed and the compressed branch carries the gradient
// into the block representations).
//
// For one softmax attention o = sum_k p_k v_k with p = softmax(tau q.k) and upstream gradient
// go = sigma dO (sigma: the branch's gate weight), with D = sigma <dO, o> and
// P = exp2(scaled score - lse2) recomputed from the forward's statistics:
//   dS = P (sigma dP - D), dP = <dO, v>;   dq = tau sum_k dS k;   dk = tau dS q;   dv = sigma P dO.
//
// stats_from_saved_kernel  the per-(token, head, branch) LSE, D and sigma, and the gate-logit
//                  gradients, from the training forward's saved branch outputs.
// bwd_dq_kernel    compressed and window branches, writes dQ: a workgroup owns 4 consecutive
//                  tokens of one KV group, a wave per token with the group's G heads as the
//                  16-wide MFMA column tile (as in the forward); 32-key chunks shared by the 4
//                  tokens are staged once in LDS (the next chunk's loads in flight): S^T = K.Q^T
//                  and dP^T = V.dO^T on the MFMA, dS^T in registers, dQ^T += K^T.dS^T with K^T
//                  read through the transposing LDS read (dS as single bf16 values).
// bwd_dq_slc_kernel  selected branch, adds into dQ: the same per-chunk math, each wave
//                  walking its own token's selected chunks through its own LDS tile.
// bwd_dkv_kernel   one workgroup per work item of 16 * NW * KT keys against up to 128 (512
//                  for the compressed branch) query tokens, KT 16-key tiles per wave: the
//                  tokens are taken two at a time (32 head rows staged in LDS, the next pair's
//                  loads in flight), S = Q.K^T and dP = dO.V^T with the keys' fragments held
//                  in registers, then dV^T += dO^T.(sigma P) and dK^T += Q^T.dS (sigma P and dS
//                  as single bf16 values, fp32 sums on the MFMA, as in the usual attention
//                  backward: about 2e-3 relative L2 on dK, dV); the item's sums are added to
//                  the fp32 gradients with atomics.  Items: compressed key blocks x query
//                  tiles (tokens that see the keys), window key blocks x the tokens whose
//                  window covers them, and for the selected branch a selection block x 128 of
//                  the tokens that selected it (the inverted lists of the block-major forward,
//                  own block included).
// compress_bwd_*   the linear block map: column sums of dY, dPE = W.colsum, dW = X^T.dY
//                  (X = block rows + PE, split over row ranges, atomics), dX = dY.W^T added
//                  into the raw key/value gradients as one GEMM per token position within the
//                  stride (a token lies in l/s blocks; no atomics).  fp32 FMA.
// Every MFMA runs under wave-uniform control flow: the instruction reads all 64 lanes'
// operands, so padding rows (heads past G, tokens past a list) are masked in the values.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace nsa {

namespace {

// key `key` of a work item is attended by query token t in branch `kind`
__device__ __forceinline__ bool bwd_visible(const BwdParams& p, int kind, int key, int t) {
    if (t < 0) return false;
    if (kind == 0) return key * p.s + p.l - 1 <= t;
    if (kind == 1) return key <= t;
    return key <= t && key >= t - p.window + 1;
}

}  // namespace

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ x, size_t n) {
    const size_t stride = (size_t)gridDim.x * 256;
    const size_t n4 = n / 4;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride)
        reinterpret_cast<f32x4*>(x)[i] = zero4();
    for (size_t i = n4 * 4 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) x[i] = 0.f;
}

// x[0 .. n) = v (no alignment assumed)
__global__ __launch_bounds__(256) void fill_f32_kernel(float* __restrict__ x, size_t n, float v) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) x[i] = v;
}

// ---------------------------------------------------------------------------
// dQ.  A workgroup owns kDqTok consecutive tokens of one (sequence, group), a wave per token.
// bwd_dq_kernel: the compressed keys and the window range are shared by the tokens: their
// 32-key chunks go through one LDS tile (the next chunk's loads in flight in registers while
// the current one is computed); it writes dQ.  bwd_dq_slc_kernel: the selected blocks differ
// per token, so each wave walks its own chunks through its own LDS tile, the next chunk's K
// rows and V fragments in flight in registers; it adds into dQ.
constexpr int kDqTok = 4;

template <int DK, int DV>
struct DqChunk {   // one 32-key chunk of K and V rows, staged by the whole workgroup
    static constexpr int NK = DK / 64, NV = DV / 64;   // 16-byte pieces per thread
    u32x4 rk[NK], rv[NV];
    __device__ __forceinline__ void load(const u16* Kb, const u16* Vb, int nrows, int key0) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int idx = threadIdx.x + 256 * i, r = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            rk[i] = key0 + r < nrows ? *reinterpret_cast<const u32x4*>(Kb + (size_t)(key0 + r) * DK + col)
                                     : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + 256 * i, r = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            rv[i] = key0 + r < nrows ? *reinterpret_cast<const u32x4*>(Vb + (size_t)(key0 + r) * DV + col)
                                     : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(u16* sk, int kstr, u16* sv, int vstr) const {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int idx = threadIdx.x + 256 * i, r = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            *reinterpret_cast<u32x4*>(&sk[r * kstr + col]) = rk[i];
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + 256 * i, r = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            *reinterpret_cast<u32x4*>(&sv[r * vstr + col]) = rv[i];
        }
    }
};

// orders this wave's LDS writes before its later reads (no other wave shares the region)
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// dQ^T += K^T.dS^T for the 32 keys at key0 of the row-major LDS tile kt (stride KSTR), V rows
// va (A operands of V.dO^T); keys outside [lo, hi] and heads past G masked.  st: lse2, D,
// sigma of this lane's (token, head).  Every lane must take part (MFMA operands).  mid() runs
// once va is consumed (the caller may reload it there).
template <int DK, int DV, typename Mid>
__device__ __forceinline__ void dq_chunk(const u16* kt, const bf16x8 (&va)[2][DV / 32], const bf16x8 (&qf)[DK / 32],
                                         const bf16x8 (&df)[DV / 32], f32x4 (&acc)[DK / 16], int key0, int lo, int hi,
                                         const f32x4& st, bool head_ok, float scale_log2, Mid mid) {
    constexpr int NDS = DK / 32, NDD = DV / 32, NDK = DK / 16, KSTR = DK + 16;
    const int lane = threadIdx.x & 63, li = lane & 15, lq = lane >> 4;
    f32x4 s0 = zero4(), s1 = zero4(), d0 = zero4(), d1 = zero4();
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        s0 = mfma16(ld8(&kt[li * KSTR + 32 * ds + 8 * lq]), qf[ds], s0);
        s1 = mfma16(ld8(&kt[(16 + li) * KSTR + 32 * ds + 8 * lq]), qf[ds], s1);
    }
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd) {
        d0 = mfma16(va[0][dd], df[dd], d0);
        d1 = mfma16(va[1][dd], df[dd], d1);
    }
    mid();
    // C rows: keys key0 + 4lq + r (tile 0) and key0 + 16 + 4lq + r (tile 1); column: head
    f32x4 ga, gb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ka = key0 + 4 * lq + r, kb = ka + 16;
        const float pa = (head_ok && ka >= lo && ka <= hi) ? fast_exp2(s0[r] * scale_log2 - st[0]) : 0.f;
        const float pb = (head_ok && kb >= lo && kb <= hi) ? fast_exp2(s1[r] * scale_log2 - st[0]) : 0.f;
        ga[r] = pa * (st[2] * d0[r] - st[1]);
        gb[r] = pb * (st[2] * d1[r] - st[1]);
    }
    // dS as single bf16 values, as for dK and dV (a high/low pair, 2^-17 relative, cost 12
    // more MFMAs per chunk: 17.9 against 15.2 ms for the dense dQ at 64K)
    const bf16x8 gh = pack_p(ga, gb);
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) {
        const bf16x8 a = ld_vt_tr(kt, KSTR, 0, 16 * dt);
        acc[dt] = mfma16(a, gh, acc[dt]);
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdParams p) {
    constexpr int NDS = DK / 32, NDD = DV / 32, NDK = DK / 16;
    constexpr int KSTR = DK + 16, VSTR = DV + 16;   // 8-byte aligned rows for the transposing read
    __shared__ __attribute__((aligned(16))) u16 sk[32 * KSTR];
    __shared__ __attribute__((aligned(16))) u16 sv[32 * VSTR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, lq = lane >> 4;
    int bg, it;
    if (!xcd_map_tile(blockIdx.x, p.B * p.Hkv, (p.T + kDqTok - 1) / kDqTok, bg, it)) return;
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int t0 = it * kDqTok, t = t0 + wave, tlast = min(t0 + kDqTok, p.T) - 1;
    const bool active = t < p.T;
    const int G = p.G, H = p.Hkv * G;
    const bool head_ok = li < G && active;
    const size_t row = ((size_t)b * p.T + min(t, p.T - 1)) * H + g * G + min(li, G - 1);

    bf16x8 qf[NDS], df[NDD];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = head_ok ? ld8(p.Q + row * DK + 32 * ds + 8 * lq) : zero8();
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd) df[dd] = head_ok ? ld8(p.dO + row * DV + 32 * dd + 8 * lq) : zero8();
    f32x4 acc[NDK];
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) acc[dt] = zero4();

    auto math = [&](const u16* kt, const bf16x8 (&va)[2][NDD], int key0, int lo, int hi, const f32x4& st) {
        dq_chunk<DK, DV>(kt, va, qf, df, acc, key0, lo, hi, st, head_ok, p.scale_log2, [] {});
    };

    // keys kfirst .. klast of Kb/Vb shared by the workgroup's tokens; this wave's token
    // attends [lo, hi]
    auto shared_range = [&](const u16* Kb, const u16* Vb, int nrows, int kfirst, int klast, int lo, int hi,
                            const f32x4& st) {
        if (klast < kfirst) return;   // uniform over the workgroup
        const int c0 = kfirst & ~31, nch = (klast - c0) / 32 + 1;
        DqChunk<DK, DV> ch;
        ch.load(Kb, Vb, nrows, c0);
        __syncthreads();   // the previous range's LDS reads are complete
        ch.store(sk, KSTR, sv, VSTR);
        __syncthreads();
        for (int i = 0; i < nch; ++i) {
            const int key0 = c0 + 32 * i;
            ch.load(Kb, Vb, nrows, c0 + 32 * min(i + 1, nch - 1));   // the last chunk reloads itself
            // wave-uniform condition: the MFMA reads every lane's operands, so no lane may
            // skip the loads (heads past G are masked inside math)
            if (active && key0 + 31 >= lo && key0 <= hi) {
                bf16x8 va[2][NDD];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int dd = 0; dd < NDD; ++dd) va[tt][dd] = ld8(&sv[(16 * tt + li) * VSTR + 32 * dd + 8 * lq]);
                math(sk, va, key0, lo, hi, st);
            }
            __syncthreads();
            ch.store(sk, KSTR, sv, VSTR);
            __syncthreads();
        }
    };

    if (p.branches & 1) {
        const f32x4 st = *reinterpret_cast<const f32x4*>(p.stats + row * 12);
        auto ncmp = [&](int tt) { return tt < p.l - 1 ? 0 : min((tt - p.l + 1) / p.s + 1, p.N); };
        shared_range(p.Kc + (size_t)bg * p.N * DK, p.Vc + (size_t)bg * p.N * DV, p.N, 0, ncmp(tlast) - 1, 0,
                     ncmp(t) - 1, st);
    }
    const u16* Kb = p.K + (size_t)bg * p.T * DK;
    const u16* Vb = p.V + (size_t)bg * p.T * DV;
    if (p.branches & 4) {
        const f32x4 st = *reinterpret_cast<const f32x4*>(p.stats + row * 12 + 8);
        shared_range(Kb, Vb, p.T, max(0, t0 - p.window + 1), tlast, max(0, t - p.window + 1), t, st);
    }
    if (!head_ok) return;
    // dQ^T C layout: rows d = 16 dt + 4 lq + r of head li
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt)
        *reinterpret_cast<f32x4*>(p.dQ + row * DK + 16 * dt + 4 * lq) = acc[dt] * p.scale;
}

template <int DK, int DV>
__global__ __launch_bounds__(256, 2) void bwd_dq_slc_kernel(BwdParams p) {
    constexpr int NDS = DK / 32, NDD = DV / 32, NDK = DK / 16;
    constexpr int KSTR = DK + 16;
    constexpr int NKR = 32 * DK / 8 / 64;   // 16-byte pieces of a 32-key K chunk per lane
    __shared__ __attribute__((aligned(16))) u16 wk[kDqTok][32 * KSTR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, lq = lane >> 4;
    int bg, it;
    if (!xcd_map_tile(blockIdx.x, p.B * p.Hkv, (p.T + kDqTok - 1) / kDqTok, bg, it)) return;
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int t = it * kDqTok + wave;
    if (t >= p.T) return;   // whole wave; no workgroup barrier in this kernel
    const int G = p.G, H = p.Hkv * G;
    const bool head_ok = li < G;
    const size_t row = ((size_t)b * p.T + t) * H + g * G + min(li, G - 1);
    bf16x8 qf[NDS], df[NDD];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = head_ok ? ld8(p.Q + row * DK + 32 * ds + 8 * lq) : zero8();
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd) df[dd] = head_ok ? ld8(p.dO + row * DV + 32 * dd + 8 * lq) : zero8();
    const f32x4 st = *reinterpret_cast<const f32x4*>(p.stats + row * 12 + 4);
    f32x4 acc[NDK];
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) acc[dt] = zero4();
    const u16* Kb = p.K + (size_t)bg * p.T * DK;
    const u16* Vb = p.V + (size_t)bg * p.T * DV;
    u16* kt = wk[wave];
    // the token's block list, one entry per lane, read back with readlane
    const int sel_lane = lane < p.top_n ? p.sel[(((size_t)b * p.T + t) * p.Hkv + g) * p.top_n + lane] : -1;
    auto sl = [&](int c) { return __builtin_amdgcn_readlane(sel_lane, c); };
    // chunk after (c, q) in list order: block slot c, sub-chunk q (32 keys); false past the end
    auto next = [&](int& c, int& q) {
        ++q;
        for (; c < p.top_n; ++c, q = 0) {
            const int j = sl(c);
            if (j >= 0 && j * p.lp <= t && j * p.lp + 32 * q <= min(t, j * p.lp + p.lp - 1)) return true;
        }
        return false;
    };
    int c = 0, q = -1;
    if (!next(c, q)) return;
    // loads of a chunk: K rows into kr (stored to LDS at the next step), V rows as A operands;
    // rows past the sequence are read from its last token (those keys are masked)
    u32x4 kr[NKR];
    bf16x8 va[2][NDD];
    auto load_k = [&](int key0) {
#pragma unroll
        for (int i = 0; i < NKR; ++i) {
            const int idx = lane + 64 * i, r = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            kr[i] = *reinterpret_cast<const u32x4*>(Kb + (size_t)min(key0 + r, p.T - 1) * DK + col);
        }
    };
    auto load_v = [&](int key0) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int dd = 0; dd < NDD; ++dd)
                va[tt][dd] = ld8(Vb + (size_t)min(key0 + 16 * tt + li, p.T - 1) * DV + 32 * dd + 8 * lq);
    };
    int key0 = sl(c) * p.lp + 32 * q;
    load_k(key0);
    load_v(key0);
    for (;;) {
        const int j = sl(c);
        const int lo = j * p.lp, hi = min(t, lo + p.lp - 1);
        wave_lds_sync();   // the previous chunk's LDS reads are complete
#pragma unroll
        for (int i = 0; i < NKR; ++i) {
            const int idx = lane + 64 * i, r = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            *reinterpret_cast<u32x4*>(&kt[r * KSTR + col]) = kr[i];
        }
        int cn = c, qn = q;
        const bool more = next(cn, qn);
        const int key_n = more ? sl(cn) * p.lp + 32 * qn : key0;   // the last chunk reloads itself
        load_k(key_n);   // in flight during this chunk's math
        wave_lds_sync();
        // the next chunk's V rows are requested as soon as this chunk's dP has used va
        dq_chunk<DK, DV>(kt, va, qf, df, acc, key0, lo, hi, st, head_ok, p.scale_log2, [&] { load_v(key_n); });
        if (!more) break;
        c = cn;
        q = qn;
        key0 = key_n;
    }
    if (!head_ok) return;
#pragma unroll
    for (int dt = 0; dt < NDK; ++dt) {
        f32x4* o = reinterpret_cast<f32x4*>(p.dQ + row * DK + 16 * dt + 4 * lq);
        *o = *o + acc[dt] * p.scale;
    }
}

// ---------------------------------------------------------------------------
// dK, dV.  NW waves, 16 keys each; the item's query tokens two at a time.
template <int DK, int DV, int NW>
struct PairStage {   // Q and dO rows of two tokens (32 head rows) and their statistics
    static constexpr int NT = 64 * NW;
    static constexpr int NQ = (32 * DK / 8 + NT - 1) / NT, NO = (32 * DV / 8 + NT - 1) / NT;
    u32x4 rq[NQ], ro[NO];
    f32x4 rst;
    __device__ __forceinline__ void load(const BwdParams& p, int b, int g, int kind, int tA, int tB) {
        const int G = p.G, H = p.Hkv * G;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int idx = threadIdx.x + NT * i, r = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const int tk = r < 16 ? tA : tB, hh = r & 15;
            rq[i] = (idx < 32 * DK / 8 && tk >= 0 && hh < G)
                        ? *reinterpret_cast<const u32x4*>(p.Q + (((size_t)b * p.T + tk) * H + g * G + hh) * DK + col)
                        : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < NO; ++i) {
            const int idx = threadIdx.x + NT * i, r = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            const int tk = r < 16 ? tA : tB, hh = r & 15;
            ro[i] = (idx < 32 * DV / 8 && tk >= 0 && hh < G)
                        ? *reinterpret_cast<const u32x4*>(p.dO + (((size_t)b * p.T + tk) * H + g * G + hh) * DV + col)
                        : u32x4{0u, 0u, 0u, 0u};
        }
        rst = zero4();
        if (threadIdx.x < 32) {
            const int r = threadIdx.x, tk = r < 16 ? tA : tB, hh = r & 15;
            if (tk >= 0 && hh < G)
                rst = *reinterpret_cast<const f32x4*>(p.stats +
                                                      ((((size_t)b * p.T + tk) * H + g * G + hh) * 3 + kind) * 4);
        }
    }
    __device__ __forceinline__ void store(u16* qs, int qstr, u16* os, int ostr, float* rs) const {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int idx = threadIdx.x + NT * i, r = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            if (idx < 32 * DK / 8) *reinterpret_cast<u32x4*>(&qs[r * qstr + col]) = rq[i];
        }
#pragma unroll
        for (int i = 0; i < NO; ++i) {
            const int idx = threadIdx.x + NT * i, r = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            if (idx < 32 * DV / 8) *reinterpret_cast<u32x4*>(&os[r * ostr + col]) = ro[i];
        }
        if (threadIdx.x < 32) *reinterpret_cast<f32x4*>(&rs[threadIdx.x * 4]) = rst;
    }
};

// KT key tiles of 16 per wave: each Q / dO operand read from LDS feeds KT products, so the
// LDS traffic per key falls by KT (with KT = 2 a wave needs more than 256 registers: one
// wave per SIMD).
template <int DK, int DV, int NW, int KT>
__global__ __launch_bounds__(64 * NW, KT == 1 ? 8 / NW : 1) void bwd_dkv_kernel(BwdParams p, int item0) {
    constexpr int NDS = DK / 32, NDD = DV / 32, NDK = DK / 16, NDV = DV / 16;
    constexpr int QSTR = DK + 16, OSTR = DV + 16;
    constexpr int KEYS = 16 * NW * KT;
    __shared__ __attribute__((aligned(16))) u16 qs[32 * QSTR];   // rows: token A heads, token B heads
    __shared__ __attribute__((aligned(16))) u16 os[32 * OSTR];
    __shared__ __attribute__((aligned(16))) float rs[32 * 4];   // lse2, D, sigma per row
    __shared__ int toks[kBwdTile];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, lq = lane >> 4;

    // ---- work item: kind (0 compressed, 1 selected, 2 window), group, keys, query tokens ----
    int kind, bg, kbase, kend, nq, t0 = 0;
    int x = blockIdx.x + item0;
    if (x < p.n_cmp_items) {
        kind = 0;
        const int per_bg = p.n_kb_cmp * p.n_qt;
        bg = x / per_bg;
        const int r = x % per_bg, kb = r / p.n_qt, qt = r % p.n_qt;
        kbase = kb * KEYS;
        kend = min(kbase + KEYS, p.N);
        t0 = max(qt * p.qt_cmp, kbase * p.s + p.l - 1);   // first token that sees key kbase
        const int t1 = min((qt + 1) * p.qt_cmp, p.T);
        if (t0 >= t1) return;
        nq = t1 - t0;
    } else if ((x -= p.n_cmp_items) < p.n_win_items) {
        kind = 2;
        const int per_bg = p.n_kb_win * p.n_qt_win;
        bg = x / per_bg;
        const int r = x % per_bg, kb = r / p.n_qt_win, qt = r % p.n_qt_win;
        kbase = kb * KEYS;
        kend = min(kbase + KEYS, p.T);
        t0 = kbase + qt * kBwdTile;
        const int t1 = min(min(t0 + kBwdTile, kbase + KEYS + p.window - 1), p.T);
        if (t0 >= t1) return;
        nq = t1 - t0;
    } else {
        x -= p.n_win_items;
        kind = 1;
        const int sub = x % p.nsb;
        x /= p.nsb;
        if (x >= p.tile_start[p.n_bucket]) return;
        const int lo = p.tile_bucket[x];   // the bucket owning list tile x
        bg = lo / p.n_slc;
        const int j = lo % p.n_slc;
        kbase = j * p.lp + KEYS * sub;
        kend = min(j * p.lp + p.lp, p.T);
        if (kbase >= kend) return;
        const int e0 = p.bucket_start[lo] + (x - p.tile_start[lo]) * kBwdTile;
        nq = min(kBwdTile, p.bucket_start[lo + 1] - e0);
        for (int i = threadIdx.x; i < kBwdTile; i += 64 * NW) toks[i] = i < nq ? (p.entries[e0 + i] >> 5) : -1;
    }
    __syncthreads();
    auto tok = [&](int i) { return i >= nq ? -1 : kind == 1 ? toks[i] : t0 + i; };
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int G = p.G;
    const int nrows = kind == 0 ? p.N : p.T;
    const u16* Kb = kind == 0 ? p.Kc + (size_t)bg * p.N * DK : p.K + (size_t)bg * p.T * DK;
    const u16* Vb = kind == 0 ? p.Vc + (size_t)bg * p.N * DV : p.V + (size_t)bg * p.T * DV;
    int key[KT];
    bool key_ok[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        key[kt] = kbase + 16 * (wave * KT + kt) + li;
        key_ok[kt] = key[kt] < kend && key[kt] < nrows;
    }

    // this lane's key rows as the B operands of Q.K^T and dO.V^T
    bf16x8 kfr[KT][NDS], vfr[KT][NDD];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
            kfr[kt][ds] = key_ok[kt] ? ld8(Kb + (size_t)key[kt] * DK + 32 * ds + 8 * lq) : zero8();
#pragma unroll
        for (int dd = 0; dd < NDD; ++dd)
            vfr[kt][dd] = key_ok[kt] ? ld8(Vb + (size_t)key[kt] * DV + 32 * dd + 8 * lq) : zero8();
    }
    f32x4 dk_acc[KT][NDK], dv_acc[KT][NDV];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int dt = 0; dt < NDK; ++dt) dk_acc[kt][dt] = zero4();
#pragma unroll
        for (int dt = 0; dt < NDV; ++dt) dv_acc[kt][dt] = zero4();
    }

    PairStage<DK, DV, NW> stage;
    stage.load(p, b, g, kind, tok(0), tok(1));
    for (int i = 0; i < nq; i += 2) {
        const int tA = tok(i), tB = tok(i + 1);
        __syncthreads();   // the previous pair's LDS reads are complete
        stage.store(qs, QSTR, os, OSTR, rs);
        __syncthreads();
        stage.load(p, b, g, kind, tok(i + 2), tok(i + 3));   // in flight during this pair's math
        // S = Q.K^T and dP = dO.V^T: C lane (li = key, lq) holds head rows 4 lq + r
        f32x4 sA[KT], sB[KT], pA[KT], pB[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) sA[kt] = sB[kt] = pA[kt] = pB[kt] = zero4();
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            const bf16x8 qa = ld8(&qs[li * QSTR + 32 * ds + 8 * lq]);
            const bf16x8 qb = ld8(&qs[(16 + li) * QSTR + 32 * ds + 8 * lq]);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                sA[kt] = mfma16(qa, kfr[kt][ds], sA[kt]);
                sB[kt] = mfma16(qb, kfr[kt][ds], sB[kt]);
            }
        }
#pragma unroll
        for (int dd = 0; dd < NDD; ++dd) {
            const bf16x8 oa = ld8(&os[li * OSTR + 32 * dd + 8 * lq]);
            const bf16x8 ob = ld8(&os[(16 + li) * OSTR + 32 * dd + 8 * lq]);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                pA[kt] = mfma16(oa, vfr[kt][dd], pA[kt]);
                pB[kt] = mfma16(ob, vfr[kt][dd], pB[kt]);
            }
        }
        bf16x8 w8[KT], g8[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const bool vA = key_ok[kt] && bwd_visible(p, kind, key[kt], tA);
            const bool vB = key_ok[kt] && bwd_visible(p, kind, key[kt], tB);
            f32x4 wA, wB, gA, gB;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hr = 4 * lq + r;
                const f32x4 stA = *reinterpret_cast<const f32x4*>(&rs[hr * 4]);
                const f32x4 stB = *reinterpret_cast<const f32x4*>(&rs[(16 + hr) * 4]);
                const float PA = (vA && hr < G) ? fast_exp2(sA[kt][r] * p.scale_log2 - stA[0]) : 0.f;
                const float PB = (vB && hr < G) ? fast_exp2(sB[kt][r] * p.scale_log2 - stB[0]) : 0.f;
                wA[r] = stA[2] * PA;
                wB[r] = stB[2] * PB;
                gA[r] = PA * (stA[2] * pA[kt][r] - stA[1]);
                gB[r] = PB * (stB[2] * pB[kt][r] - stB[1]);
            }
            // sigma P and dS as single bf16 values; the row slots of pack_p (head rows
            // 4lq..4lq+3 of token A, then of token B) match the transposing read's key order
            w8[kt] = pack_p(wA, wB);
            g8[kt] = pack_p(gA, gB);
        }
        // dV^T += dO^T . (sigma P) and dK^T += Q^T . dS
#pragma unroll
        for (int dt = 0; dt < NDV; ++dt) {
            const bf16x8 a = ld_vt_tr(os, OSTR, 0, 16 * dt);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) dv_acc[kt][dt] = mfma16(a, w8[kt], dv_acc[kt][dt]);
        }
#pragma unroll
        for (int dt = 0; dt < NDK; ++dt) {
            const bf16x8 a = ld_vt_tr(qs, QSTR, 0, 16 * dt);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) dk_acc[kt][dt] = mfma16(a, g8[kt], dk_acc[kt][dt]);
        }
    }
    // C layout of dK^T / dV^T: lane (li = key, lq) holds dims 16 dt + 4 lq + r
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        if (!key_ok[kt]) continue;
        float* dKr = (kind == 0 ? p.dKc + (size_t)bg * p.N * DK : p.dK + (size_t)bg * p.T * DK) + (size_t)key[kt] * DK;
        float* dVr = (kind == 0 ? p.dVc + (size_t)bg * p.N * DV : p.dV + (size_t)bg * p.T * DV) + (size_t)key[kt] * DV;
#pragma unroll
        for (int dt = 0; dt < NDK; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) unsafeAtomicAdd(dKr + 16 * dt + 4 * lq + r, dk_acc[kt][dt][r] * p.scale);
#pragma unroll
        for (int dt = 0; dt < NDV; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) unsafeAtomicAdd(dVr + 16 * dt + 4 * lq + r, dv_acc[kt][dt][r]);
    }
}

// ---------------------------------------------------------------------------
// Linear block map.  Rows of dY are (sequence-group bg, block i), bg-major; X[row][m] for
// m = r*d + e is K[bg][i*s + r][e] + pe[r][e].

// colsum[o] += sum over 64 rows of dY[row][o]; one thread per column
__global__ __launch_bounds__(256) void compress_bwd_colsum_kernel(const float* __restrict__ dY, int rows, int d,
                                                                  float* __restrict__ colsum) {
    const int o = threadIdx.x;
    if (o >= d) return;
    const int r0 = blockIdx.x * 64, r1 = min(r0 + 64, rows);
    float s = 0.f;
    for (int r = r0; r < r1; ++r) s += dY[(size_t)r * d + o];
    unsafeAtomicAdd(colsum + o, s);
}

// dpe[m] = sum_o W[m][o] colsum[o]
__global__ __launch_bounds__(256) void compress_bwd_dpe_kernel(const u16* __restrict__ W, const float* __restrict__ colsum,
                                                               int KD, int d, float* __restrict__ dpe) {
    const int m = blockIdx.x * 256 + threadIdx.x;
    if (m >= KD) return;
    float s = 0.f;
    for (int o = 0; o < d; ++o) s += bf2f(W[(size_t)m * d + o]) * colsum[o];
    dpe[m] = s;
}

// dW[m][o] += sum over this workgroup's kDwRows rows of X[row][m] dY[row][o]: 64 x 64 output
// tile, 4 x 4 per thread, 16 rows per LDS step (one atomic add per output per row range)
constexpr int kDwRows = 1024;
__global__ __launch_bounds__(256) void compress_bwd_dw_kernel(const u16* __restrict__ X, const u16* __restrict__ pe,
                                                              const float* __restrict__ dY, float* __restrict__ dW,
                                                              int rows, int N, int T, int d, int l, int s) {
    __shared__ float xs[16][64 + 4], ys[16][64 + 4];
    const int KD = l * d;
    const int m0 = blockIdx.x * 64, o0 = blockIdx.y * 64;
    const int rbeg = blockIdx.z * kDwRows, rend = min(rbeg + kDwRows, rows);
    const int tm = threadIdx.x % 16, to = threadIdx.x / 16;
    float acc[4][4] = {};
    const int rr = m0 / d;   // block offset r of this tile (d is a multiple of 64)
    for (int r0 = rbeg; r0 < rend; r0 += 16) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < 16 * 64; idx += 256) {
            const int k = idx / 64, c = idx % 64, row = r0 + k;
            float xv = 0.f, yv = 0.f;
            if (row < rend) {
                const int bg = row / N, i = row % N;
                const int e = m0 % d + c;
                xv = bf2f(X[((size_t)bg * T + (size_t)i * s + rr) * d + e]) + bf2f(pe[(size_t)rr * d + e]);
                if (o0 + c < d) yv = dY[(size_t)row * d + o0 + c];
            }
            xs[k][c] = xv;
            ys[k][c] = yv;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float a[4], bv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                a[u] = xs[k][tm + 16 * u];
                bv[u] = ys[k][to + 16 * u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * bv[v];
        }
    }
    (void)KD;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = m0 + tm + 16 * u, o = o0 + to + 16 * v;
            if (o < d) unsafeAtomicAdd(dW + (size_t)m * d + o, acc[u][v]);
        }
}

// dX added to dK without atomics: token tok = q*s + rho lies in blocks i = q - phi for
// phi = 0 .. l/s - 1 at row rho + phi*s of each, so for a fixed rho
//   dK[tok][e] += sum_phi sum_o dY[q - phi][o] W[(rho + phi*s)*d + e][o]
// is one GEMM over (phi, o).  A workgroup owns 64 token slots q x 64 dims e of one (bg, rho),
// 4 x 4 per thread, 16 o per LDS step; every output element has one writer.
__global__ __launch_bounds__(256) void compress_bwd_dx_kernel(const float* __restrict__ dY, const u16* __restrict__ W,
                                                              float* __restrict__ dX, int N, int T, int d, int l,
                                                              int s) {
    __shared__ float ys[16][64 + 4], ws[16][64 + 4];
    const int q0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    const int bg = blockIdx.z / s, rho = blockIdx.z % s;
    const int tq = threadIdx.x % 16, te = threadIdx.x / 16;
    float acc[4][4] = {};
    for (int phi = 0; phi < l / s; ++phi) {
        const int wrow = (rho + phi * s) * d;
        for (int k0 = 0; k0 < d; k0 += 16) {
            __syncthreads();
            for (int idx = threadIdx.x; idx < 16 * 64; idx += 256) {
                const int k = idx % 16, c = idx / 16;
                const int i = q0 + c - phi;   // block of token slot q0 + c at phase phi
                ys[k][c] = (i >= 0 && i < N) ? dY[((size_t)bg * N + i) * d + k0 + k] : 0.f;
                ws[k][c] = bf2f(W[(size_t)(wrow + e0 + c) * d + k0 + k]);
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                float a[4], bv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    a[u] = ys[k][tq + 16 * u];
                    bv[u] = ws[k][te + 16 * u];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[u][v] += a[u] * bv[v];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int tok = (q0 + tq + 16 * u) * s + rho;
        if (tok >= T) continue;
        float* row = dX + ((size_t)bg * T + tok) * d + e0;
#pragma unroll
        for (int v = 0; v < 4; ++v) row[te + 16 * v] += acc[u][v];
    }
}

// ---------------------------------------------------------------------------
// Statistics from a training forward's saved outputs: 16 lanes per (token, head) row, each
// lane DV/16 consecutive dims read as 16-byte vectors; D_c = sigma_c <dO, o_c> summed over
// the row's lanes (DPP), the LSEs copied (base 2).
template <int DV>
__global__ __launch_bounds__(256) void stats_from_saved_kernel(AttnParams p) {
    constexpr int E = DV / 16;   // dims per lane (8 or 4)
    const int lane = threadIdx.x & 63, l16 = lane & 15;
    const size_t rows = (size_t)p.B * p.T * p.Hkv * p.G;
    const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const bool ok = row < rows;
    const size_t rr = ok ? row : rows - 1;
    const bool on[3] = {(p.branches & 1) != 0, (p.branches & 2) != 0, (p.branches & 4) != 0};
    float g[E];
    {
        const u16* src = p.dO + rr * DV + l16 * E;
        if constexpr (E == 8) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                g[2 * i] = bf2f((u16)(w[i] & 0xFFFFu));
                g[2 * i + 1] = bf2f((u16)(w[i] >> 16));
            }
        } else {
            const u32x2 w = *reinterpret_cast<const u32x2*>(src);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                g[2 * i] = bf2f((u16)(w[i] & 0xFFFFu));
                g[2 * i + 1] = bf2f((u16)(w[i] >> 16));
            }
        }
    }
    const float* srcs[3] = {p.o_cmp + rr * DV, p.saved_o + rr * 2 * DV, p.saved_o + (rr * 2 + 1) * DV};
    float dot[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        if (!on[c]) continue;
#pragma unroll
        for (int i = 0; i < E / 4; ++i) {
            const f32x4 o = ld_stream(reinterpret_cast<const f32x4*>(srcs[c] + l16 * E) + i);
            dot[c] += g[4 * i] * o[0] + g[4 * i + 1] * o[1] + g[4 * i + 2] * o[2] + g[4 * i + 3] * o[3];
        }
        dot[c] = lane_group_sum<16>(dot[c]);
    }
    if (!ok || l16 != 0) return;
    float sg[3] = {1.f, 1.f, 1.f};
    if (p.gates)
#pragma unroll
        for (int c = 0; c < 3; ++c) sg[c] = sigmoidf_(p.gates[row * 3 + c]);
    const float lse2[3] = {on[0] ? p.lse_cmp[row] * kLog2e : 0.f, p.saved_lse[row * 2], p.saved_lse[row * 2 + 1]};
    f32x4* so = reinterpret_cast<f32x4*>(p.stats + row * 12);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        so[c] = f32x4{lse2[c], on[c] ? sg[c] * dot[c] : 0.f, sg[c], 0.f};
        if (p.dgates) p.dgates[row * 3 + c] = on[c] ? sg[c] * (1.f - sg[c]) * dot[c] : 0.f;
    }
}

void launch_stats_from_saved(int DV, const AttnParams& p, hipStream_t st) {
    const size_t rows = (size_t)p.B * p.T * p.Hkv * p.G;
    const unsigned grid = (unsigned)((rows + 15) / 16);
    if (DV == 128) stats_from_saved_kernel<128><<<grid, 256, 0, st>>>(p);
    else stats_from_saved_kernel<64><<<grid, 256, 0, st>>>(p);
}

void launch_fill_zero(float* x, size_t n, hipStream_t st) {
    if (n == 0) return;
    const size_t blocks = std::min<size_t>((n / 4 + 255) / 256 + 1, 8192);
    fill_zero_kernel<<<(unsigned)blocks, 256, 0, st>>>(x, n);
}

void launch_fill_f32(float* x, size_t n, float v, hipStream_t st) {
    if (n == 0) return;
    const size_t blocks = std::min<size_t>((n + 255) / 256, 8192);
    fill_f32_kernel<<<(unsigned)blocks, 256, 0, st>>>(x, n, v);
}

bool launch_bwd_dq(int DK, int DV, const BwdParams& p, hipStream_t st) {
    const int grid = xcd_grid(p.B * p.Hkv, (p.T + kDqTok - 1) / kDqTok);
    const bool slc = (p.branches & 2) != 0;
    if (DK == 192 && DV == 128) {
        bwd_dq_kernel<192, 128><<<grid, 256, 0, st>>>(p);
        if (slc) bwd_dq_slc_kernel<192, 128><<<grid, 256, 0, st>>>(p);
    } else if (DK == 128 && DV == 128) {
        bwd_dq_kernel<128, 128><<<grid, 256, 0, st>>>(p);
        if (slc) bwd_dq_slc_kernel<128, 128><<<grid, 256, 0, st>>>(p);
    } else if (DK == 64 && DV == 64) {
        bwd_dq_kernel<64, 64><<<grid, 256, 0, st>>>(p);
        if (slc) bwd_dq_slc_kernel<64, 64><<<grid, 256, 0, st>>>(p);
    } else {
        return false;
    }
    return true;
}

template <int NW, int KT>
bool launch_dkv_nw(int DK, int DV, const BwdParams& p, int item0, int n, hipStream_t st) {
    if (n <= 0) return true;
    if (DK == 192 && DV == 128) bwd_dkv_kernel<192, 128, NW, KT><<<n, 64 * NW, 0, st>>>(p, item0);
    else if (DK == 128 && DV == 128) bwd_dkv_kernel<128, 128, NW, KT><<<n, 64 * NW, 0, st>>>(p, item0);
    else if (DK == 64 && DV == 64) bwd_dkv_kernel<64, 64, NW, KT><<<n, 64 * NW, 0, st>>>(p, item0);
    else return false;
    return true;
}

// compressed and window items: kDkvWavesDense waves x kDkvTilesDense key tiles; selected
// items: 64 keys (4 waves x 1 tile)
bool launch_bwd_dkv(int DK, int DV, const BwdParams& p, int n_slc_items, hipStream_t st) {
    return launch_dkv_nw<kDkvWavesDense, kDkvTilesDense>(DK, DV, p, 0, p.n_cmp_items + p.n_win_items, st) &&
           launch_dkv_nw<kDkvWavesSlc, 1>(DK, DV, p, p.n_cmp_items + p.n_win_items, n_slc_items, st);
}

void launch_compress_bwd(const u16* X, const u16* W, const u16* pe, const float* dY, float* dX, float* dW, float* dpe,
                         float* colsum, int BG, int T, int N, int d, int l, int s, hipStream_t st) {
    const int rows = BG * N, KD = l * d;
    launch_fill_zero(colsum, (size_t)d, st);
    launch_fill_zero(dW, (size_t)KD * d, st);
    if (rows == 0) {
        launch_fill_zero(dpe, (size_t)KD, st);
        return;
    }
    compress_bwd_colsum_kernel<<<(rows + 63) / 64, 256, 0, st>>>(dY, rows, d, colsum);
    compress_bwd_dpe_kernel<<<(KD + 255) / 256, 256, 0, st>>>(W, colsum, KD, d, dpe);
    compress_bwd_dw_kernel<<<dim3(KD / 64, (d + 63) / 64, (rows + kDwRows - 1) / kDwRows), 256, 0, st>>>(
        X, pe, dY, dW, rows, N, T, d, l, s);
    const int nq = (T + s - 1) / s;   // token slots per position rho
    compress_bwd_dx_kernel<<<dim3((nq + 63) / 64, d / 64, BG * s), 256, 0, st>>>(dY, W, dX, N, T, d, l, s);
}

}  // namespace nsa
