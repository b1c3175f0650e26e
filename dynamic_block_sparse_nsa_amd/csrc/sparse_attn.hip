// Selected-block attention, sliding window and gated sum (zjai.club notes, sections 5-6
// and 10; sunshychen.top: the query's own block is causally masked, the window crosses
// block boundaries).
//
// A workgroup owns 4 consecutive tokens of one KV group, one token per wave.  The group's
// G query heads form the 16-wide MFMA column tile (the pages' NSA kernel packs the
// group's heads into the matrix dimension so every KV tile feeds all of them at once).
// Every attention product is key-major: S^T = K . Q^T on the MFMA, online softmax with
// the running max and sum in registers (base-2), then O^T += V^T . P^T with V^T read
// from a transposed, 32-key-permuted copy of V so both operands are 16-byte loads.
//
// Phase B (per token, first): the selected blocks before the window range are contiguous
//   64-token spans gathered by block index straight from memory in 32-key chunks, two
//   chunks in flight per wave.
// Phase A (shared): the window range of the 4 tokens is streamed once through
//   double-buffered LDS tiles of 32 keys; each wave updates its window softmax and, for
//   selected blocks lying inside that range (the local blocks), its selected-branch
//   softmax from the same S tile.
// Epilogue: sigmoid gates on o_cmp (from the caller), o_slc, o_win; bf16 store.
#include "common.hpp"
#include "launch.hpp"

namespace nsa {

namespace {

constexpr int kTok = 4;      // tokens (= waves) per workgroup
constexpr int kChunk = 32;   // keys per tile

template <int DV>
struct SoftmaxState {
    static constexpr int NDT = DV / 16;
    f32x4 o[NDT];
    float m, l;

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = zero4();
        m = -INFINITY;
        l = 0.f;
    }

    // One 32-key chunk starting at key0: s0 holds keys key0+4q+r, s1 keys key0+16+4q+r
    // (q = lane/16); keys outside [lo, hi] are masked.  va: the V^T operand per d-tile.
    __device__ __forceinline__ void update(const f32x4& s0, const f32x4& s1, int key0, int lo, int hi, float scale_log2,
                           const bf16x8 (&va)[NDT]) {
        const int lq = (threadIdx.x & 63) >> 4;
        float x[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ka = key0 + 4 * lq + r, kb = key0 + 16 + 4 * lq + r;
            x[r] = (ka >= lo && ka <= hi) ? s0[r] * scale_log2 : -INFINITY;
            x[4 + r] = (kb >= lo && kb <= hi) ? s1[r] * scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, fmaxf(x[r], x[4 + r]));
        }
        tmax = col_max(tmax);
        const float mnew = fmaxf(m, tmax);
        const float alpha = fast_exp2(m - mnew);
        f32x4 pa, pb;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pa[r] = fast_exp2(x[r] - mnew);
            pb[r] = fast_exp2(x[4 + r] - mnew);
            ps += pa[r] + pb[r];
        }
        l = l * alpha + ps;
        m = mnew;
        bf16x8 bh, bl;
        pack_p_split(pa, pb, bh, bl);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            o[dt] *= alpha;
            o[dt] = mfma16(va[dt], bh, o[dt]);
            o[dt] = mfma16(va[dt], bl, o[dt]);
        }
    }

    __device__ __forceinline__ void finish() {
        const float L = col_sum(l);
        const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= inv;
    }
};

// Window-range tile staging: K rows [key0, key0+32) (clamped to T-1) and V^T columns
// [key0, key0+32) of the transposed copy.
template <int DK, int DV>
struct WinTile {
    static constexpr int KSTR = DK + 8;
    static constexpr int VSTR = kChunk + 8;
    static constexpr int KPR = DK / 8;              // uint4 per K row
    static constexpr int NK = kChunk * KPR / 256;   // K uint4 per thread
    static constexpr int NV = DV * (kChunk / 8) / 256;  // V uint4 per thread
    static_assert(kChunk * KPR % 256 == 0 && DV * (kChunk / 8) % 256 == 0, "tile must split evenly");
    u32x4 rk[NK], rv[NV];

    __device__ __forceinline__ void load(const u16* kg, const u16* vtg, int key0, int T, int Tpad) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int idx = threadIdx.x + 256 * i;
            const int row = idx / KPR, col = (idx % KPR) * 8;
            rk[i] = *reinterpret_cast<const u32x4*>(kg + (size_t)min(key0 + row, T - 1) * DK + col);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + 256 * i;
            const int row = idx / (kChunk / 8), col = (idx % (kChunk / 8)) * 8;
            rv[i] = *reinterpret_cast<const u32x4*>(vtg + (size_t)row * Tpad + key0 + col);
        }
    }
    __device__ __forceinline__ void store(u16* kb, u16* vb) const {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int idx = threadIdx.x + 256 * i;
            const int row = idx / KPR, col = (idx % KPR) * 8;
            *reinterpret_cast<u32x4*>(&kb[row * KSTR + col]) = rk[i];
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + 256 * i;
            const int row = idx / (kChunk / 8), col = (idx % (kChunk / 8)) * 8;
            *reinterpret_cast<u32x4*>(&vb[row * VSTR + col]) = rv[i];
        }
    }
};

// One gathered 32-key chunk held in registers: K rows as the A operands of S^T = K.Q^T
// and V^T columns as the A operands of O^T += V^T.P^T.
template <int DK, int DV>
struct GatherChunk {
    static constexpr int NDS = DK / 32, NDT = DV / 16;
    bf16x8 ka[NDS], kb[NDS], va[NDT];
    __device__ __forceinline__ void load(const u16* kg, const u16* vtg, int key0, int T, int Tpad) {
        const int lane = threadIdx.x & 63, li = lane & 15, lq = lane >> 4;
        const u16* k0p = kg + (size_t)min(key0 + li, T - 1) * DK + lq * 8;
        const u16* k1p = kg + (size_t)min(key0 + 16 + li, T - 1) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) { ka[ds] = ld8(k0p + 32 * ds); kb[ds] = ld8(k1p + 32 * ds); }
        const u16* vp = vtg + (size_t)li * Tpad + key0 + lq * 8;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) va[dt] = ld8(vp + (size_t)16 * dt * Tpad);
    }
    __device__ __forceinline__ void scores(const bf16x8 (&qf)[NDS], f32x4& s0, f32x4& s1) const {
        s0 = zero4();
        s1 = zero4();
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            s0 = mfma16(ka[ds], qf[ds], s0);
            s1 = mfma16(kb[ds], qf[ds], s1);
        }
    }
};

}  // namespace

template <int DK, int DV>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(AttnParams p) {
    constexpr int NDS = DK / 32;
    constexpr int NDT = DV / 16;
    using Tile = WinTile<DK, DV>;
    __shared__ __attribute__((aligned(16))) u16 kbuf[2][kChunk * Tile::KSTR];
    __shared__ __attribute__((aligned(16))) u16 vbuf[2][DV * Tile::VSTR];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int b = blockIdx.z, g = blockIdx.y;
    const int T = p.T;
    const int tok0 = blockIdx.x * kTok;
    const int t = tok0 + wave;
    const bool active = t < T;
    const int tq = min(t, T - 1);
    const int G = p.G, H = p.Hkv * G;
    const bool head_ok = li < G;
    const int h = g * G + min(li, G - 1);

    bf16x8 qf[NDS];
    {
        const u16* qp = p.Q + (((size_t)b * T + tq) * H + h) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[ds] = head_ok ? ld8(qp + 32 * ds) : zero8();
    }
    const u16* kg = p.K + ((size_t)b * p.Hkv + g) * (size_t)T * DK;
    const u16* vtg = p.Vt + ((size_t)b * p.Hkv + g) * (size_t)DV * p.Tpad;
    const bool use_slc = (p.branches & 2) != 0, use_win = (p.branches & 4) != 0;
    // the token's block list, one entry per lane, read back with readlane (no memory
    // access on the dependency chain of a gather's address)
    const int sel_lane = (use_slc && lane < p.top_n)
                             ? p.sel[(((size_t)b * T + tq) * p.Hkv + g) * p.top_n + lane] : -1;
    auto sl = [&](int c) { return __builtin_amdgcn_readlane(sel_lane, c); };

    SoftmaxState<DV> win, slc;
    win.reset();
    slc.reset();

    // range of keys streamed through LDS for the window (phase A)
    int c_begin = 0, nch = 0;
    if (use_win) {
        const int wlo = max(0, tok0 - p.window + 1);
        const int whi = min(tok0 + kTok - 1, T - 1);
        c_begin = wlo & ~(kChunk - 1);
        nch = (whi - c_begin) / kChunk + 1;
    }

    // ---- phase B: selected blocks before that range, gathered per token ----
    // Chunks are software-pipelined: the next chunk's loads are in flight while the
    // current one is computed (two register buffers used alternately).
    if (active && use_slc) {
        int nb = 0;  // leading list entries outside the shared range (the list is ascending)
        for (; nb < p.top_n; ++nb) {
            const int j = sl(nb);
            if (j < 0 || (nch > 0 && j * p.lp >= c_begin)) break;
        }
        const int cpb = p.lp / kChunk;
        int c = 0, u = 0;
        auto advance = [&](int& key0, int& start) -> bool {
            while (c < nb) {
                start = sl(c) * p.lp;
                key0 = start + kChunk * u;
                if (u < cpb && key0 <= t) { ++u; return true; }
                ++c;
                u = 0;
            }
            return false;
        };
        GatherChunk<DK, DV> A, B;
        int keyA = 0, startA = 0, keyB = 0, startB = 0;
        bool hasA = advance(keyA, startA);
        if (hasA) A.load(kg, vtg, keyA, T, p.Tpad);
        while (hasA) {
            const bool hasB = advance(keyB, startB);
            if (hasB) B.load(kg, vtg, keyB, T, p.Tpad);
            f32x4 s0, s1;
            A.scores(qf, s0, s1);
            slc.update(s0, s1, keyA, startA, t, p.scale_log2, A.va);
            if (!hasB) break;
            hasA = advance(keyA, startA);
            if (hasA) A.load(kg, vtg, keyA, T, p.Tpad);
            B.scores(qf, s0, s1);
            slc.update(s0, s1, keyB, startB, t, p.scale_log2, B.va);
        }
    }

    // ---- phase A: the window range of the workgroup's tokens, shared through LDS ----
    Tile tile;
    if (nch > 0) {
        tile.load(kg, vtg, c_begin, T, p.Tpad);
        tile.store(kbuf[0], vbuf[0]);
    }
    __syncthreads();
    const int wlo_t = t - p.window + 1;
    for (int i = 0; i < nch; ++i) {
        const int key0 = c_begin + kChunk * i;
        const int buf = i & 1;
        if (i + 1 < nch) tile.load(kg, vtg, key0 + kChunk, T, p.Tpad);
        if (active) {
            const bool w_any = key0 + kChunk - 1 >= wlo_t && key0 <= t;
            const int jch = key0 / p.lp;
            bool s_any = false;
            if (use_slc && key0 <= t && jch * p.lp >= c_begin) {
                for (int c = 0; c < p.top_n; ++c) {
                    const int j = sl(c);
                    if (j < 0 || j > jch) break;
                    s_any |= (j == jch);
                }
            }
            if (w_any || s_any) {
                f32x4 s0 = zero4(), s1 = zero4();
                const u16* kb = kbuf[buf];
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) {
                    s0 = mfma16(ld8(&kb[li * Tile::KSTR + 32 * ds + lq * 8]), qf[ds], s0);
                    s1 = mfma16(ld8(&kb[(16 + li) * Tile::KSTR + 32 * ds + lq * 8]), qf[ds], s1);
                }
                bf16x8 va[NDT];
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) va[dt] = ld8(&vbuf[buf][(16 * dt + li) * Tile::VSTR + lq * 8]);
                if (w_any) win.update(s0, s1, key0, wlo_t, t, p.scale_log2, va);
                if (s_any) slc.update(s0, s1, key0, jch * p.lp, t, p.scale_log2, va);
            }
        }
        if (i + 1 < nch) tile.store(kbuf[buf ^ 1], vbuf[buf ^ 1]);
        __syncthreads();
    }

    if (!active) return;
    win.finish();
    slc.finish();
    if (!head_ok) return;

    float gc = 1.f, gs = 1.f, gw = 1.f;
    const size_t row = ((size_t)b * T + t) * H + h;
    if (p.gates) {
        gc = sigmoidf_(p.gates[row * 3 + 0]);
        gs = sigmoidf_(p.gates[row * 3 + 1]);
        gw = sigmoidf_(p.gates[row * 3 + 2]);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        const int d0 = 16 * dt + 4 * lq;
        float4 oc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p.branches & 1) oc = *reinterpret_cast<const float4*>(p.o_cmp + row * DV + d0);
        const float vc[4] = {oc.x, oc.y, oc.z, oc.w};
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float y = 0.f;
            if (p.branches & 1) y += gc * vc[r];
            if (use_slc) y += gs * slc.o[dt][r];
            if (use_win) y += gw * win.o[dt][r];
            v[r] = y;
        }
        const uint32_t w0 = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        const uint32_t w1 = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
        *reinterpret_cast<uint2*>(p.O + row * DV + d0) = make_uint2(w0, w1);
    }
}

bool launch_sparse_attn(int DK, int DV, const AttnParams& p, int B, hipStream_t st) {
    dim3 grid((p.T + kTok - 1) / kTok, p.Hkv, B);
    if (DK == 192 && DV == 128) sparse_attn_kernel<192, 128><<<grid, 256, 0, st>>>(p);
    else if (DK == 128 && DV == 128) sparse_attn_kernel<128, 128><<<grid, 256, 0, st>>>(p);
    else if (DK == 64 && DV == 64) sparse_attn_kernel<64, 64><<<grid, 256, 0, st>>>(p);
    else return false;
    return true;
}

}  // namespace nsa
