// Selected-block attention, sliding window and gated sum of 4 consecutive tokens: the device
// body shared by sparse_attn_kernel (sparse_attn.hip) and the fused prefill kernel
// (prefill.hip).  (zjai.club notes, sections 5-6 and 10; sunshychen.top: the query's own
// block is causally masked, the window crosses block boundaries.)
//
// A workgroup owns 4 consecutive tokens of one KV group, one token per wave.  The group's
// G query heads form the 16-wide MFMA column tile (the pages' NSA kernel packs the
// group's heads into the matrix dimension so every KV tile feeds all of them at once).
// Every attention product is key-major: S^T = K . Q^T on the MFMA, online softmax with a
// lazily moved reference and the sum in registers (base-2), then O^T += V^T . P^T.
//
// K and V are first copied into MFMA fragment order (launch_tile_cmp, the layout pass of
// the compressed branch): the operands a wave needs for 16 keys x 32 dims of K, or 32 keys
// x 16 dims of V^T, are 1 KB of contiguous memory in lane order.  Operand loads straight
// from row-major K would have each lane read a different key row, so every 16-byte lane
// access costs the address unit a cycle; in fragment order a wave's load is one
// contiguous, coalesced 1 KB.  V is copied as fp16 scaled by 2^-e (e per sequence and
// group, from its largest |V|), so O^T += V^T.P^T is one fp16 product with P in fp16.
//
// Phase B (per token, first): the selected blocks before the window range are contiguous
//   64-token spans gathered by block index straight from memory in 32-key chunks, two
//   chunks in flight per wave.
// Phase A (shared): the window range of the 4 tokens is streamed once through
//   double-buffered LDS tiles of 32 keys; each wave updates its window softmax and, for
//   selected blocks lying inside that range (the local blocks), its selected-branch
//   softmax from the same S tile.
// Epilogue: sigmoid gates on o_cmp (from the caller), o_slc, o_win; bf16 store.
#pragma once

#include <climits>

#include "common.hpp"
#include "launch.hpp"

namespace nsa {

namespace sattn {


constexpr int kTok = 4;      // tokens (= waves) per workgroup
constexpr int kChunk = 32;   // keys per tile
constexpr float kLazy = 8.f; // log2 headroom before a column's softmax reference moves

template <int DV>
struct SoftmaxState {
    static constexpr int NDT = DV / 16;
    f32x4 o[NDT];
    float m, l;   // the column's softmax reference (log2 units) and its sum of 2^(x - m)

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = zero4();
        m = -INFINITY;
        l = 0.f;
    }

    // One 32-key chunk starting at key0: s0 holds keys key0+4q+r, s1 keys key0+16+4q+r
    // (q = lane/16); keys outside [lo, hi] are masked.  va: the V^T operand per d-tile, fp16
    // (V scaled by a power of two; finish() undoes it).
    __device__ __forceinline__ void update(const f32x4& s0, const f32x4& s1, int key0, int lo, int hi, float scale_log2,
                           const f16x8 (&va)[NDT]) {
        const int lq = (threadIdx.x & 63) >> 4;
        // raw scores (the scale is positive: the max is taken before scaling and the scale
        // folds into the exponent's fma); a chunk inside [lo, hi] (wave-uniform) is unmasked
        float x[8];
        if (key0 >= lo && key0 + 31 <= hi) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[r] = s0[r];
                x[4 + r] = s1[r];
            }
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ka = key0 + 4 * lq + r, kb = key0 + 16 + 4 * lq + r;
                x[r] = (ka >= lo && ka <= hi) ? s0[r] : -INFINITY;
                x[4 + r] = (kb >= lo && kb <= hi) ? s1[r] : -INFINITY;
            }
        }
        float tmax = vmax(x[0], x[4]);
#pragma unroll
        for (int r = 1; r < 4; ++r) tmax = vmax(vmax(tmax, x[r]), x[4 + r]);
        // m is a lazily moved reference, not the running max: a column's m moves (and its l
        // and o are rescaled) only when the chunk's max exceeds it by more than 2^kLazy, so
        // p = 2^(x - m) <= 2^kLazy (within fp16's range) and the rescale is rare after the
        // first chunk.  The decision is per column, so a column's result does not depend on
        // the other heads in the tile.
        const float mt = col_max(tmax) * scale_log2;
        const bool grow = mt > m + kLazy;
        if (__ballot(grow)) {   // wave-uniform branch
            const float alpha = !grow ? 1.f : m == -INFINITY ? 0.f : fast_exp2(m - mt);
            m = grow ? mt : m;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        }
        f32x4 pa, pb;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pa[r] = fast_exp2(__builtin_fmaf(x[r], scale_log2, -m));
            pb[r] = fast_exp2(__builtin_fmaf(x[4 + r], scale_log2, -m));
            ps += pa[r] + pb[r];
        }
        l += ps;
        // P in fp16 against the fp16 V copy: one product per slice (2^-11 relative rounding
        // of p)
        const f16x8 ph = pack_p_h(pa, pb);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = mfma16h(va[dt], ph, o[dt]);
    }

    // normalizes o (and undoes V's scaling by 2^-vexp); returns the column's sum of exp2(x - m)
    __device__ __forceinline__ float finish(int vexp) {
        const float L = col_sum(l);
        const float inv = L > 0.f ? ldexpf(1.0f / L, vexp) : 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= inv;
        return L;
    }
};

// Fragment-order addressing (elements): K operands of the 16-key group kt, step ds;
// V^T operands of the 32-key chunk c, value slice dt.  A lane reads 8 elements at +8*lane.
template <int DK>
__device__ __forceinline__ size_t kfrag(int kt, int ds) { return ((size_t)kt * (DK / 32) + ds) * 512; }
template <int DV>
__device__ __forceinline__ size_t vfrag(int c, int dt) { return ((size_t)c * (DV / 16) + dt) * 512; }

// Window-range tile staging: the fragments of keys [key0, key0 + 32) copied to LDS in
// the same order (a plain contiguous copy, 16 bytes per thread and step).
template <int DK, int DV>
struct WinTile {
    static constexpr int KE = 2 * (DK / 32) * 512;   // K elements of a 32-key tile
    static constexpr int VE = (DV / 16) * 512;       // V elements
    static constexpr int NK = KE / 8 / 256;           // 16-byte pieces per thread
    static constexpr int NV = VE / 8 / 256;
    static_assert(KE % 2048 == 0 && VE % 2048 == 0, "tile must split evenly");
    u32x4 rk[NK], rv[NV];

    __device__ __forceinline__ void load(const u16* kg, const u16* vg, int key0) {
        const u16* ks = kg + kfrag<DK>(key0 / 16, 0);
        const u16* vs = vg + vfrag<DV>(key0 / 32, 0);
#pragma unroll
        for (int i = 0; i < NK; ++i) rk[i] = *reinterpret_cast<const u32x4*>(ks + (threadIdx.x + 256 * i) * 8);
#pragma unroll
        for (int i = 0; i < NV; ++i) rv[i] = *reinterpret_cast<const u32x4*>(vs + (threadIdx.x + 256 * i) * 8);
    }
    __device__ __forceinline__ void store(u16* kb, u16* vb) const {
#pragma unroll
        for (int i = 0; i < NK; ++i) *reinterpret_cast<u32x4*>(&kb[(threadIdx.x + 256 * i) * 8]) = rk[i];
#pragma unroll
        for (int i = 0; i < NV; ++i) *reinterpret_cast<u32x4*>(&vb[(threadIdx.x + 256 * i) * 8]) = rv[i];
    }
};

// One gathered 32-key chunk held in registers: K rows as the A operands of S^T = K.Q^T
// and V^T columns as the A operands of O^T += V^T.P^T (each a contiguous 1 KB load).
template <int DK, int DV>
struct GatherChunk {
    static constexpr int NDS = DK / 32, NDT = DV / 16;
    bf16x8 ka[NDS], kb[NDS];
    f16x8 va[NDT];
    __device__ __forceinline__ void load(const u16* kg, const u16* vg, int key0) {
        const int lane = threadIdx.x & 63;
        const u16* k0 = kg + kfrag<DK>(key0 / 16, 0) + lane * 8;
        const u16* v0 = vg + vfrag<DV>(key0 / 32, 0) + lane * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            ka[ds] = ld8(k0 + ds * 512);
            kb[ds] = ld8(k0 + (NDS + ds) * 512);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) va[dt] = ld8h(v0 + dt * 512);
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

}  // namespace sattn

// LDS elements (16-bit) the body needs: two K and two V window tiles.
__host__ __device__ constexpr int sparse_lds_elems(int DK, int DV) { return 2 * (2 * (DK / 32) * 512) + 2 * ((DV / 16) * 512); }

using sattn::kTok;

// The kTok = 4 consecutive tokens tok0 .. tok0+3 of KV group `unit`, one per wave (every
// wave of the 256-thread workgroup must call it, with tok0 < T).  lds: sparse_lds_elems(DK,
// DV) 16-byte aligned elements for the window tiles.  Ends after a barrier; what follows is
// per-wave work (no barrier), and waves whose token is past T leave early.
// MODE 0: the forward.  MODE 2: the forward that also saves, for the backward, the selected
// and window branches' base-2 LSE and normalized outputs (training forward).  MODE 1: the
// backward pass's statistics instead of the gated output: per (token, head) and branch c,
// lse2_c = log2 of the branch's sum of exp2(scaled scores), D_c = sigma_c <dO, o_c> and
// sigma_c (1 without gates); dgates = (1 - sigma_c) D_c, the gate logit's gradient
// sigma (1 - sigma) <dO, o_c>.  The compressed branch takes its LSE and o_cmp from the caller.
template <int DK, int DV, int MODE>
__device__ __forceinline__ void sparse_attn_tokens(const AttnParams& p, int unit, int tok0, u16* lds) {
    constexpr bool STATS = MODE == 1, SAVE = MODE == 2;
    constexpr int NDS = DK / 32;
    constexpr int NDT = DV / 16;
    using Tile = sattn::WinTile<DK, DV>;
    u16* kbuf[2] = {lds, lds + Tile::KE};
    u16* vbuf[2] = {lds + 2 * Tile::KE, lds + 2 * Tile::KE + Tile::VE};

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int li = lane & 15, lq = lane >> 4;
    const int T = p.T;
    const int b = unit / p.Hkv, g = unit % p.Hkv;
    const int t = tok0 + wave;
    const bool active = t < T;
    const int tq = min(t, T - 1);
    const int G = p.G, H = p.Hkv * G;
    const bool head_ok = li < G;
    const int h = g * G + min(li, G - 1);

    const bool use_slc = (p.branches & 2) != 0, use_win = (p.branches & 4) != 0;
    // the query rows (not read when only the compressed branch is on: then the call is the
    // gated sum of the caller's o_cmp alone)
    const bool need_q = head_ok && (use_slc || use_win);
    bf16x8 qf[NDS];
    {
        const u16* qp = p.Q + (((size_t)b * T + tq) * H + h) * DK;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
            qf[ds] = need_q ? __builtin_bit_cast(bf16x8, ld_stream(reinterpret_cast<const u32x4*>(qp + 32 * ds + 8 * lq)))
                            : zero8();
    }
    const u16* kg = p.Kf + ((size_t)b * p.Hkv + g) * (size_t)p.Tpad * DK;
    const u16* vg = p.Vf + ((size_t)b * p.Hkv + g) * (size_t)p.Tpad * DV;
    // the token's block list, one entry per lane, read back with readlane (no memory
    // access on the dependency chain of a gather's address)
    const int sel_lane = (use_slc && lane < p.top_n)
                             ? p.sel[(((size_t)b * T + tq) * p.Hkv + g) * p.top_n + lane] : -1;
    auto sl = [&](int c) { return __builtin_amdgcn_readlane(sel_lane, c); };

    sattn::SoftmaxState<DV> win, slc;
    win.reset();
    slc.reset();

    // range of keys streamed through LDS for the window (phase A)
    int c_begin = 0, nch = 0;
    if (use_win) {
        const int wlo = max(0, tok0 - p.window + 1);
        const int whi = min(tok0 + kTok - 1, T - 1);
        c_begin = wlo & ~(sattn::kChunk - 1);
        nch = (whi - c_begin) / sattn::kChunk + 1;
    }

    // ---- phase B: selected blocks before that range, gathered per token ----
    // Chunks are software-pipelined: the next chunk's loads are in flight while the
    // current one is computed (two register buffers used alternately).  Every load is
    // unconditional (a chunk index past the list is clamped to the last chunk and its
    // keys masked), so each wait names only the chunk it consumes.
    if (active && use_slc) {
        int nb = 0;  // leading list entries outside the shared range (the list is ascending)
        for (; nb < p.top_n; ++nb) {
            const int j = sl(nb);
            if (j < 0 || (nch > 0 && j * p.lp >= c_begin)) break;
        }
        const int cpb = p.lp / sattn::kChunk;
        const int nck = nb * cpb;
        auto ckey = [&](int c) {
            const int cc = min(c, nck - 1);
            return sl(cc / cpb) * p.lp + sattn::kChunk * (cc % cpb);
        };
        if (nck > 0) {
            sattn::GatherChunk<DK, DV> A, B;
            A.load(kg, vg, ckey(0));
            for (int c = 0; c < nck; c += 2) {
                const int kA = ckey(c), kB = ckey(c + 1);
                B.load(kg, vg, kB);
                f32x4 s0, s1;
                A.scores(qf, s0, s1);
                slc.update(s0, s1, kA, kA, t, p.scale_log2, A.va);
                A.load(kg, vg, ckey(c + 2));
                B.scores(qf, s0, s1);
                slc.update(s0, s1, kB, c + 1 < nck ? kB : INT_MAX, t, p.scale_log2, B.va);
            }
        }
    }

    // The forward's o_cmp rows are requested here, so they arrive during phase A instead of
    // after it (the gather registers of phase B are free by now).
    f32x4 ocv[NDT];
    if constexpr (!STATS) {
        const bool want = active && head_ok && (p.branches & 1);
        const f32x4* op = reinterpret_cast<const f32x4*>(p.o_cmp + (((size_t)b * T + tq) * H + h) * DV + 4 * lq);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) ocv[dt] = want ? ld_stream(op + 4 * dt) : zero4();
    }

    // ---- phase A: the window range of the workgroup's tokens, shared through LDS ----
    // Tiles are loaded to registers two tiles ahead (two register stages used alternately),
    // stored to the LDS buffer one tile ahead, and computed from LDS.  Tile indices past the
    // range are clamped to the last tile (never computed), so no load is conditional.
    const int wlo_t = t - p.window + 1;
    auto tile_key = [&](int i) { return c_begin + sattn::kChunk * min(i, nch - 1); };
    auto compute = [&](int i) {
        if (!active) return;
        const int key0 = c_begin + sattn::kChunk * i;
        const int buf = i & 1;
        const bool w_any = key0 + sattn::kChunk - 1 >= wlo_t && key0 <= t;
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
            const u16* kb = kbuf[buf] + lane * 8;
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                s0 = mfma16(ld8(kb + ds * 512), qf[ds], s0);
                s1 = mfma16(ld8(kb + (NDS + ds) * 512), qf[ds], s1);
            }
            f16x8 va[NDT];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) va[dt] = ld8h(vbuf[buf] + (dt * 64 + lane) * 8);
            if (w_any) win.update(s0, s1, key0, wlo_t, t, p.scale_log2, va);
            if (s_any) slc.update(s0, s1, key0, jch * p.lp, t, p.scale_log2, va);
        }
    };
    Tile ta, tb;   // register stages: after the prologue tb holds tile 1
    if (nch > 0) {
        ta.load(kg, vg, tile_key(0));
        ta.store(kbuf[0], vbuf[0]);
        tb.load(kg, vg, tile_key(1));
    }
    __syncthreads();
    for (int i = 0; i < nch; i += 2) {
        // tile i in LDS buffer 0, tile i + 1 in tb
        ta.load(kg, vg, tile_key(i + 2));
        compute(i);
        __builtin_amdgcn_sched_barrier(0);   // keep the staging stores after this tile's math
        tb.store(kbuf[1], vbuf[1]);
        __syncthreads();
        if (i + 1 < nch) {   // tile i + 1 in LDS buffer 1, tile i + 2 in ta
            tb.load(kg, vg, tile_key(i + 3));
            compute(i + 1);
            __builtin_amdgcn_sched_barrier(0);
            ta.store(kbuf[0], vbuf[0]);
            __syncthreads();
        }
    }

    if (!active) return;
    const int vexp = p.vexp[unit];
    const float Lw = win.finish(vexp);
    const float Ls = slc.finish(vexp);
    if constexpr (STATS) {
        const size_t row = ((size_t)b * T + t) * H + h;
        float sg[3] = {1.f, 1.f, 1.f};
        if (p.gates && head_ok) {
#pragma unroll
            for (int c = 0; c < 3; ++c) sg[c] = sigmoidf_(p.gates[row * 3 + c]);
        }
        float dc = 0.f, dsl = 0.f, dwn = 0.f;   // <dO, o_c> partial over this lane's dims
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int d0 = 16 * dt + 4 * lq;
            u32x2 raw = {0u, 0u};
            f32x4 oc = zero4();
            if (head_ok) {
                raw = *reinterpret_cast<const u32x2*>(p.dO + row * DV + d0);
                if (p.branches & 1) oc = *reinterpret_cast<const f32x4*>(p.o_cmp + row * DV + d0);
            }
            const float g4[4] = {bf2f((u16)(raw[0] & 0xFFFFu)), bf2f((u16)(raw[0] >> 16)),
                                 bf2f((u16)(raw[1] & 0xFFFFu)), bf2f((u16)(raw[1] >> 16))};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dc += g4[r] * oc[r];
                dsl += g4[r] * slc.o[dt][r];
                dwn += g4[r] * win.o[dt][r];
            }
        }
        dc = col_sum(dc);
        dsl = col_sum(dsl);
        dwn = col_sum(dwn);
        if (head_ok && lq == 0) {
            const bool on[3] = {(p.branches & 1) != 0, use_slc, use_win};
            const float lse2[3] = {on[0] ? p.lse_cmp[row] * kLog2e : 0.f, use_slc ? slc.m + __log2f(Ls) : 0.f,
                                   use_win ? win.m + __log2f(Lw) : 0.f};
            const float dot[3] = {dc, dsl, dwn};
            f32x4* so = reinterpret_cast<f32x4*>(p.stats + row * 12);
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                so[c] = f32x4{lse2[c], on[c] ? sg[c] * dot[c] : 0.f, sg[c], 0.f};
                if (p.dgates) p.dgates[row * 3 + c] = on[c] ? sg[c] * (1.f - sg[c]) * dot[c] : 0.f;
            }
        }
        return;
    }
    if (!head_ok) return;

    float gc = 1.f, gs = 1.f, gw = 1.f;
    const size_t row = ((size_t)b * T + t) * H + h;
    if constexpr (SAVE) {   // training forward: what the backward needs of the two branches
        if (lq == 0)
            *reinterpret_cast<float2*>(p.saved_lse + row * 2) =
                float2{use_slc ? slc.m + __log2f(Ls) : 0.f, use_win ? win.m + __log2f(Lw) : 0.f};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int d0 = 16 * dt + 4 * lq;
            st_stream(slc.o[dt], reinterpret_cast<f32x4*>(p.saved_o + row * 2 * DV + d0));
            st_stream(win.o[dt], reinterpret_cast<f32x4*>(p.saved_o + (row * 2 + 1) * DV + d0));
        }
    }
    if (p.gates) {
        gc = sigmoidf_(p.gates[row * 3 + 0]);
        gs = sigmoidf_(p.gates[row * 3 + 1]);
        gw = sigmoidf_(p.gates[row * 3 + 2]);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        const int d0 = 16 * dt + 4 * lq;
        const f32x4 oc = ocv[dt];
        const float vc[4] = {oc[0], oc[1], oc[2], oc[3]};
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
        st_stream(u32x2{w0, w1}, reinterpret_cast<u32x2*>(p.O + row * DV + d0));
    }
}

}  // namespace nsa
