// One NSA decode step (zjai.club notes, section 13: decoding is memory-bound, so the
// cost is the cache bytes read per step).  For each sequence the new query sits at
// t = cache_len - 1 and the result equals the prefill result for that row.
//
// The compressed cache is the bulk of the bytes (N_cmp keys and values per group), so it
// is streamed exactly once, split over many workgroups:
//   decode_cmp_kernel     split s covers 256 compressed keys of one (sequence, group);
//                         4 waves x 64 keys, the group's heads packed in the MFMA column
//                         tile; every load of the split is issued before any math.
//                         Emits, relative to the split's per-head max m: the sum l, o^T
//                         normalized by l (fp16: |o| <= max |V|), and per-head block sums
//                         A[h][j] = sum over this split's keys overlapping block j of
//                         2^(x - m).  The same launch runs the sliding window's item
//                         groups (below), which do not depend on the selection.
//   decode_select_kernel  per (sequence, group): lse per head from the split (m, l) and
//                         the split weights w_s = 2^(m_s - lse); block score
//                         score[j] = sum_h sum_s w_s,h A_s[h][j] (the exact normalized
//                         compressed probabilities, summed as in prefill); then the
//                         shared top-n.
//   decode_attn_kernel    the selected blocks' item groups.  An item group is 4 waves, one
//                         item each (a selected block, or a 64-token piece of the window):
//                         exact softmax over its keys; the 4 items are combined in LDS into
//                         one partial (m, l, o^T / l).
//   decode_merge_kernel   o_cmp = sum_s w_s l_s o_s (o_s the normalized split partial),
//                         merges the partials of each branch and applies the gates; one
//                         thread per output element.
// Value rows stay key-major: each wave stores its value tile row-major in LDS and builds
// the V^T MFMA operand with the gfx950 transposing LDS read.
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace nsa {

int decode_jb(int l, int s, int lp) { return ((kDecodeSplitKeys - 1) * s + l - 1) / lp + 2; }

int decode_items(int top_n, int window) { return top_n + (window > 0 ? window / 64 + 2 : 0); }

namespace {

constexpr int kPsumStride = kDecodeSplitKeys + 4;   // padded row of the per-head probabilities

// A wave's partial o^T in LDS, head-major: [16 heads][DV + 4] fp32 (lane li holds head li,
// d = 16dt + 4lq + r of its accumulators: one 16-byte store per dt).
template <int DV>
__device__ __forceinline__ void store_partial(float* po_w, const f32x4 (&o)[DV / 16]) {
    const int lane = threadIdx.x & 63, li = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) *reinterpret_cast<f32x4*>(&po_w[li * (DV + 4) + 16 * dt + 4 * lq]) = o[dt];
}

// Partial outputs in memory are fp16 [16 heads][DV]: thread (h, d0) of a 256-thread
// workgroup owns DV/16 consecutive dims of head h.
template <int DV>
struct OutSlice {
    static constexpr int N = DV / 16;
    int h, d0;
    __device__ OutSlice() : h(threadIdx.x >> 4), d0((threadIdx.x & 15) * N) {}
};
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
template <int N>
__device__ __forceinline__ void store_f16(u16* dst, const float (&v)[N]) {
    static_assert(N == 4 || N == 8, "4 or 8 values");
    if constexpr (N == 8) {
        f16x8 h;
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (_Float16)v[i];
        *reinterpret_cast<f16x8*>(dst) = h;
    } else {
        f16x4 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = (_Float16)v[i];
        *reinterpret_cast<f16x4*>(dst) = h;
    }
}
template <int N>
struct HalfSlice;
template <>
struct HalfSlice<8> {
    f16x8 v;
    __device__ void load(const u16* src) { v = *reinterpret_cast<const f16x8*>(src); }
    __device__ float operator[](int i) const { return (float)v[i]; }
};
template <>
struct HalfSlice<4> {
    f16x4 v;
    __device__ void load(const u16* src) { v = *reinterpret_cast<const f16x4*>(src); }
    __device__ float operator[](int i) const { return (float)v[i]; }
};

__device__ __forceinline__ int query_pos(const int32_t* cache_len, int b, int L) {
    const int n = min(max(cache_len[b], 1), L);
    return n - 1;
}

// A wave's 64-key tile: K rows as the A operands of S^T = K.Q^T (4 tiles of 16 keys) and
// the value rows (clamped to < nrows), loaded to registers in one burst.
template <int DK, int DV>
struct KeyTile64 {
    static constexpr int NDS = DK / 32;
    static constexpr int NVC = 64 * DV / 8 / 64;   // 16-byte value chunks per lane
    bf16x8 ka[4][NDS];
    u32x4 vr[NVC];
    __device__ __forceinline__ void load_k(const u16* kg, int key0, int nrows) {
        const int lane = threadIdx.x & 63, li = lane & 15, lq = lane >> 4;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const u16* kp = kg + (size_t)min(key0 + 16 * kt + li, nrows - 1) * DK;
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) ka[kt][ds] = ld8(kp + kpair_off(ds, lq));
        }
    }
    __device__ __forceinline__ void load_v(const u16* vg, int key0, int nrows) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < NVC; ++i) {
            const int idx = lane + 64 * i;
            const int row = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            vr[i] = *reinterpret_cast<const u32x4*>(vg + (size_t)min(key0 + row, nrows - 1) * DV + col);
        }
    }
    __device__ __forceinline__ void load(const u16* kg, const u16* vg, int key0, int nrows) {
        load_k(kg, key0, nrows);
        load_v(vg, key0, nrows);
    }
    // value rows to a row-major LDS tile [64][STR]
    template <int STR>
    __device__ __forceinline__ void store_v(u16* vs) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < NVC; ++i) {
            const int idx = lane + 64 * i;
            const int row = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            *reinterpret_cast<u32x4*>(&vs[row * STR + col]) = vr[i];
        }
    }
    __device__ __forceinline__ void scores(const bf16x8 (&qf)[NDS], f32x4 (&s)[4]) const {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            s[kt] = zero4();
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) s[kt] = mfma16(ka[kt][ds], qf[ds], s[kt]);
        }
    }
};

template <int DK>
__device__ __forceinline__ void load_q(const u16* q, int b, int H, int g, int G, bf16x8 (&qf)[DK / 32]) {
    const int lane = threadIdx.x & 63, li = lane & 15, lq = lane >> 4;
    const int h = g * G + min(li, G - 1);
    const u16* qp = q + ((size_t)b * H + h) * DK;
#pragma unroll
    for (int ds = 0; ds < DK / 32; ++ds) qf[ds] = li < G ? ld8(qp + kpair_off(ds, lq)) : zero8();
}

}  // namespace

// ---------------------------------------------------------------------------
// A workgroup holds 4 waves; wave w takes item 4*gi + w of one branch (a selected block,
// or a 64-token piece of the window) and computes its exact softmax partial (m, l, o^T);
// the 4 partials are combined in LDS and one partial per workgroup is written.
template <int DK, int DV>
__device__ void attn_group(const DecodeParams& p, int gi, int g, int b, unsigned char* smem) {
    constexpr int NDS = DK / 32, NDT = DV / 16;
    constexpr int VSTR = DV + 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, li = lane & 15, lq = lane >> 4;
    u16* vs = reinterpret_cast<u16*>(smem) + wave * 64 * VSTR;   // this wave's value tile
    // after the items: [4 waves][16][DV + 4] partial o, then [4][16] m and l
    float* mo = reinterpret_cast<float*>(smem);
    float* mm = mo + 4 * 16 * (DV + 4);
    float* ml = mm + 64;
    const int G = p.G, H = p.Hkv * G;
    const int t = query_pos(p.cache_len, b, p.L);
    const int n_sg = (p.top_n + 3) / 4;
    const int n_win = p.n_items - p.top_n;

    int lo = 0, hi = -1, c0 = 0;
    if (gi < n_sg) {
        const int it = 4 * gi + wave;
        const int j = ((p.branches & 2) && it < p.top_n) ? p.sel_ws[((size_t)b * p.Hkv + g) * p.top_n + it] : -1;
        if (j >= 0) { lo = j * p.lp; hi = min(j * p.lp + p.lp - 1, t); c0 = lo; }
    } else if (p.branches & 4) {
        const int it = 4 * (gi - n_sg) + wave;
        const int t0 = max(0, t - p.window + 1);
        const int base = (t0 & ~63) + 64 * it;
        if (it < n_win && base <= t) { lo = max(t0, base); hi = min(t, base + 63); c0 = base; }
    }
    bf16x8 qf[NDS];
    load_q<DK>(p.q, b, H, g, G, qf);
    const u16* kg = p.K + ((size_t)b * p.Hkv + g) * (size_t)p.L * DK;
    const u16* vg = p.V + ((size_t)b * p.Hkv + g) * (size_t)p.L * DV;
    float m = -INFINITY, l = 0.f;
    f32x4 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = zero4();
    // a selection block spans l' / 64 pieces of 64 keys; a window piece is one.  Only this
    // wave touches its value tile: a wave-scope barrier orders its LDS accesses.
    for (int key0 = c0; key0 <= hi; key0 += 64) {
        KeyTile64<DK, DV> tile;
        tile.load(kg, vg, key0, p.L);
        f32x4 sacc[4];
        tile.scores(qf, sacc);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        tile.template store_v<VSTR>(vs);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float x[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 16 * kt + 4 * lq + r;
                x[kt * 4 + r] = (key >= lo && key <= hi) ? sacc[kt][r] * p.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, x[kt * 4 + r]);
            }
        tmax = col_max(tmax);
        const float mnew = fmaxf(m, tmax);
        const float alpha = fast_exp2(m - mnew);
        f32x4 pv[4];
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pv[kt][r] = fast_exp2(x[kt * 4 + r] - mnew);
                ps += pv[kt][r];
            }
        l = l * alpha + ps;
        m = mnew;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            bf16x8 bh, bl;
            pack_p_split(pv[2 * u], pv[2 * u + 1], bh, bl);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16x8 a = ld_vt_tr(vs, VSTR, 32 * u, 16 * dt);
                o[dt] = mfma16(a, bh, o[dt]);
                o[dt] = mfma16(a, bl, o[dt]);
            }
        }
    }
    l = col_sum(l);
    __syncthreads();   // every wave is done with its value tile: reuse the region
    store_partial<DV>(mo + wave * 16 * (DV + 4), o);
    if (lq == 0) {
        mm[wave * 16 + li] = m;
        ml[wave * 16 + li] = l;
    }
    __syncthreads();
    // combine the four partials of every (head, d); empty items carry m = -inf, l = 0, o = 0
    const size_t ib = ((size_t)b * p.Hkv + g) * p.n_items + gi;
    const OutSlice<DV> os;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mm[w * 16 + os.h]);
    float e[4], L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        e[w] = M > -INFINITY ? fast_exp2(mm[w * 16 + os.h] - M) : 0.f;
        L += e[w] * ml[w * 16 + os.h];
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;   // stored normalized (within fp16's range)
    float acc[OutSlice<DV>::N];
#pragma unroll
    for (int i = 0; i < OutSlice<DV>::N; ++i) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) a += e[w] * mo[(w * 16 + os.h) * (DV + 4) + os.d0 + i];
        acc[i] = a * inv;
    }
    store_f16(p.att_o + (ib * 16 + os.h) * DV + os.d0, acc);
    if (os.d0 == 0) {
        p.att_m[ib * 16 + os.h] = M;
        p.att_l[ib * 16 + os.h] = L;
    }
}

// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256, 2) void decode_cmp_kernel(DecodeParams p) {
    constexpr int NDS = DK / 32, NDT = DV / 16;
    constexpr int VSTR = DV + 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    u16* vs_all = reinterpret_cast<u16*>(smem);                              // [4][64][VSTR]
    float* wm = reinterpret_cast<float*>(vs_all + 4 * 64 * VSTR);            // [4][16]
    float* wl = wm + 64;                                                     // [4][16]
    // after the value products the tile region is reused:
    float* po = reinterpret_cast<float*>(smem);                              // [4][16][DV + 4]
    float* psum = po + 4 * 16 * (DV + 4);                                    // [16][kPsumStride]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int b = blockIdx.z, g = blockIdx.y, sp = blockIdx.x;
    if (sp >= p.n_split) {   // a window item group (independent of the selection)
        attn_group<DK, DV>(p, (p.top_n + 3) / 4 + sp - p.n_split, g, b, smem);
        return;
    }
    const int G = p.G, H = p.Hkv * G, Nc = p.Nc;
    const int t = query_pos(p.cache_len, b, p.L);
    const int nv = visible_count(t, p.l, p.s, Nc);
    const int kbeg = sp * kDecodeSplitKeys;
    const int kw = kbeg + 64 * wave;
    const size_t pbase = ((size_t)b * p.Hkv + g) * p.n_split + sp;
    if (kbeg >= nv) {
        if (threadIdx.x < 16) {
            p.part_m[pbase * 16 + threadIdx.x] = -INFINITY;
            p.part_l[pbase * 16 + threadIdx.x] = 0.f;
        }
        return;
    }
    KeyTile64<DK, DV> tile;
    tile.load(p.Kc + ((size_t)b * p.Hkv + g) * (size_t)Nc * DK, p.Vc + ((size_t)b * p.Hkv + g) * (size_t)Nc * DV, kw,
              Nc);
    bf16x8 qf[NDS];
    load_q<DK>(p.q, b, H, g, G, qf);
    f32x4 sacc[4];
    tile.scores(qf, sacc);
    u16* vs = vs_all + wave * 64 * VSTR;
    tile.template store_v<VSTR>(vs);

    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = kw + 16 * kt + 4 * lq + r;
            x[kt * 4 + r] = key < nv ? sacc[kt][r] * p.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, x[kt * 4 + r]);
        }
    tmax = col_max(tmax);
    if (lq == 0) wm[wave * 16 + li] = tmax;
    __syncthreads();
    const float M = fmaxf(fmaxf(wm[li], wm[16 + li]), fmaxf(wm[32 + li], wm[48 + li]));
    f32x4 pv[4];
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pr = fast_exp2(x[kt * 4 + r] - M);
            pv[kt][r] = pr;
            ls += pr;
        }
    ls = col_sum(ls);
    if (lq == 0) wl[wave * 16 + li] = ls;
    f32x4 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = zero4();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        bf16x8 bh, bl;
        pack_p_split(pv[2 * u], pv[2 * u + 1], bh, bl);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const bf16x8 a = ld_vt_tr(vs, VSTR, 32 * u, 16 * dt);
            oacc[dt] = mfma16(a, bh, oacc[dt]);
            oacc[dt] = mfma16(a, bl, oacc[dt]);
        }
    }
    __syncthreads();  // every wave is done with its value tile: reuse the region
    store_partial<DV>(po + wave * 16 * (DV + 4), oacc);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) psum[li * kPsumStride + 64 * wave + 16 * kt + 4 * lq + r] = pv[kt][r];
    __syncthreads();
    {   // stored normalized by the split's sum (|o| <= max |V|: within fp16's range)
        const OutSlice<DV> os;
        const float Ls = wl[os.h] + wl[16 + os.h] + wl[32 + os.h] + wl[48 + os.h];
        const float inv = Ls > 0.f ? 1.0f / Ls : 0.f;
        float v[OutSlice<DV>::N];
#pragma unroll
        for (int i = 0; i < OutSlice<DV>::N; ++i) {
            const float* q = po + os.h * (DV + 4) + os.d0 + i;
            v[i] = (((q[0] + q[16 * (DV + 4)]) + q[2 * 16 * (DV + 4)]) + q[3 * 16 * (DV + 4)]) * inv;
        }
        store_f16(p.part_o + (pbase * 16 + os.h) * DV + os.d0, v);
    }
    if (threadIdx.x < 16) {
        const int hh = threadIdx.x;
        p.part_m[pbase * 16 + hh] = fmaxf(fmaxf(wm[hh], wm[16 + hh]), fmaxf(wm[32 + hh], wm[48 + hh]));
        p.part_l[pbase * 16 + hh] = wl[hh] + wl[16 + hh] + wl[32 + hh] + wl[48 + hh];
    }
    // per-head partial block sums over this split's keys (ascending key order).  With
    // s | l and s | l', compressed key i overlaps block j iff j*a - c < i < j*a + a, where
    // a = l'/s and c = l/s.  Thread (jj, hh) takes head hh of blocks jlo + jj + 16k.
    const int a = p.lp / p.s, c = p.l / p.s;
    const int jlo = kbeg / a;
    const int jhi = min((kbeg + kDecodeSplitKeys - 1 + c - 1) / a, p.n_slc - 1);
    const int hh = threadIdx.x & 15;
    if (hh < G) {
        const float* row = psum + hh * kPsumStride - kbeg;
        for (int j = jlo + (threadIdx.x >> 4); j <= jhi; j += 16) {
            const int ilo = max(kbeg, j * a - c + 1);
            const int ihi = min(kbeg + kDecodeSplitKeys - 1, j * a + a - 1);
            float acc = 0.f;
            for (int i = ilo; i <= ihi; ++i) acc += row[i];
            p.part_a[(pbase * p.jb + (j - jlo)) * 16 + hh] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// Selection of one (sequence, group) by a 1024-thread workgroup (the block-score loads of
// 16 waves in flight together); sm holds n_split * 16 + n_slc floats.
template <int NU>
__device__ void select_unit(const DecodeParams& p, int g, int b, float* sm) {
    float* f = sm;                       // [n_split][16]
    float* sc = f + p.n_split * 16;      // [n_slc]
    const int lane = threadIdx.x & 63;
    const int t = query_pos(p.cache_len, b, p.L);
    const int nv = visible_count(t, p.l, p.s, p.Nc);
    const int ns = (nv + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
    const int jc = t / p.lp;
    const size_t bg = (size_t)b * p.Hkv + g;
    const size_t pb0 = bg * p.n_split;
    // block scores: compressed keys [ilo, ihi] overlap block j (s | l and s | l': with
    // a = l'/s and c = l/s they are j*a - c + 1 .. j*a + a - 1); at most two splits hold them
    // Thread tid scores blocks tid + 1024r (NU * 64 / 1024 of them).  The partial sums depend
    // on cache_len only, so they are requested first and arrive while the split weights are
    // formed.  Rows past jc read block jc's rows and are not stored.
    const int a = p.lp / p.s, c = p.l / p.s;
    constexpr int NR = NU * 64 / 1024 > 0 ? NU * 64 / 1024 : 1;
    f32x4 v[NR][2][4];
    int sa[NR], sb[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int j = min((int)threadIdx.x + 1024 * r, jc);
        const int ilo = max(0, j * a - c + 1);
        const int ihi = max(ilo, min(j * a + a - 1, nv - 1));
        sa[r] = ilo / kDecodeSplitKeys;
        sb[r] = ihi / kDecodeSplitKeys;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            // clamped into the workspace; a clamped (unused) row may be any split's
            const int s0 = min(min(sa[r] + h2, sb[r]), p.n_split - 1);
            const int jj = min(max(j - (s0 * kDecodeSplitKeys) / a, 0), p.jb - 1);
            const f32x4* pa = reinterpret_cast<const f32x4*>(p.part_a + ((pb0 + s0) * p.jb + jj) * 16);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) v[r][h2][q4] = pa[q4];
        }
    }
    // per-head log-sum-exp over the splits: lane = head + 16 * q holds splits q + 4i
    // (at most kDecodeMaxSplits splits, all loads issued together)
    if (threadIdx.x < 64) {
        constexpr int NI = kDecodeMaxSplits / 4;
        const int hh = lane & 15, q = lane >> 4;
        float mv[NI], lv[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int s0 = q + 4 * i;
            mv[i] = s0 < ns ? p.part_m[(pb0 + s0) * 16 + hh] : -INFINITY;
            lv[i] = s0 < ns ? p.part_l[(pb0 + s0) * 16 + hh] : 0.f;
        }
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < NI; ++i) M = fmaxf(M, mv[i]);
        M = col_max(M);
        float L = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            if (mv[i] > -INFINITY) L += lv[i] * fast_exp2(mv[i] - M);
        L = col_sum(L);
        const float lse2 = M + __log2f(L);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int s0 = q + 4 * i;
            if (s0 < ns) {
                const float w = (L > 0.f && mv[i] > -INFINITY) ? fast_exp2(mv[i] - lse2) : 0.f;
                f[s0 * 16 + hh] = w;                            // block scores: the split's probabilities
                p.cmp_w[(pb0 + s0) * 16 + hh] = w * lv[i];      // o_cmp: the split's normalized partial
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int j = (int)threadIdx.x + 1024 * r;
        if (j > jc) continue;
        const int ilo = max(0, j * a - c + 1);
        const int ihi = min(j * a + a - 1, nv - 1);
        float acc = 0.f;
        if (ilo <= ihi) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                if (sa[r] + h2 > sb[r]) continue;
                const int s0 = sa[r] + h2;
#pragma unroll
                for (int hh = 0; hh < 16; ++hh)
                    acc += hh < p.G ? f[s0 * 16 + hh] * v[r][h2][hh >> 2][hh & 3] : 0.f;
            }
        }
        sc[j] = acc;
    }
    __syncthreads();
    if (threadIdx.x < 64)
        select_blocks_wave<NU>(sc, jc, p.top_n, p.n_init, p.n_local, p.sel_ws + bg * p.top_n,
                               p.sel_out ? p.sel_out + bg * p.top_n : nullptr);
}

// ---------------------------------------------------------------------------
template <int NU>
__global__ __launch_bounds__(1024) void decode_select_kernel(DecodeParams p) {
    extern __shared__ float sm[];
    select_unit<NU>(p, blockIdx.x, blockIdx.y, sm);
}

// The selected blocks' item groups: grid (ceil(top_n / 4), Hkv, B).
template <int DK, int DV>
__global__ __launch_bounds__(256, 2) void decode_attn_kernel(DecodeParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    attn_group<DK, DV>(p, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

// ---------------------------------------------------------------------------
// One workgroup per (sequence, group); thread (h, d0) owns DV/16 consecutive outputs of head
// h and reads one fp16 slice per partial, every load issued before the merge weights are
// known (indices clamped to valid partials; the sums skip the clamped ones).
template <int DV>
__device__ void merge_unit(const DecodeParams& p, int g, int b, float* wsm) {   // wsm: [n_items][16]
    constexpr int NO = DV / 16, SB = 16, NG = kDecodeMaxItems / 4;
    const int G = p.G, H = p.Hkv * G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t bg = (size_t)b * p.Hkv + g;
    const size_t ib0 = bg * p.n_items;
    // partials: the selected branch's groups of 4 items, then the window's
    const int n_sg = (p.top_n + 3) / 4, n_grp = n_sg + (p.n_items - p.top_n + 3) / 4;
    const OutSlice<DV> os;
    const int hh = os.h;
    const int t = query_pos(p.cache_len, b, p.L);
    const int ns = (visible_count(t, p.l, p.s, p.Nc) + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
    const bool use_c = (p.branches & 1) && ns > 0, use_s = (p.branches & 2) && n_sg > 0,
               use_w = (p.branches & 4) && n_grp > n_sg;
    const size_t pb0 = bg * p.n_split;
    HalfSlice<NO> so[NG], wo[NG], co[SB];
    float cw[SB], z[3] = {0.f, 0.f, 0.f};
    if (hh < G) {
        if (use_c) {   // the first SB splits (the rest below)
#pragma unroll
            for (int i = 0; i < SB; ++i) {
                const int sp = min(i, ns - 1);
                cw[i] = p.cmp_w[(pb0 + sp) * 16 + hh];
                co[i].load(p.part_o + ((pb0 + sp) * 16 + hh) * DV + os.d0);
            }
        }
        if (use_s) {
#pragma unroll
            for (int i = 0; i < NG; ++i) so[i].load(p.att_o + ((ib0 + min(i, n_sg - 1)) * 16 + hh) * DV + os.d0);
        }
        if (use_w) {
#pragma unroll
            for (int i = 0; i < NG; ++i)
                wo[i].load(p.att_o + ((ib0 + min(n_sg + i, n_grp - 1)) * 16 + hh) * DV + os.d0);
        }
        if (p.gates) {
            const float* zp = p.gates + ((size_t)b * H + g * G + hh) * 3;
            z[0] = zp[0];
            z[1] = zp[1];
            z[2] = zp[2];
        }
    }
    // wave 0: selected-branch partials, wave 1: window partials; lane = head + 16 * q holds
    // partials i0 + q + 4i (loads issued together)
    if (wave < 2) {
        constexpr int NI = kDecodeMaxItems / 4;
        const int h4 = lane & 15, q = lane >> 4;
        const int i0 = wave == 0 ? 0 : n_sg, i1 = wave == 0 ? n_sg : n_grp;
        float mv[NI], lv[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int it = i0 + q + 4 * i;
            mv[i] = it < i1 ? p.att_m[(ib0 + it) * 16 + h4] : -INFINITY;
            lv[i] = it < i1 ? p.att_l[(ib0 + it) * 16 + h4] : 0.f;
        }
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < NI; ++i) M = fmaxf(M, mv[i]);
        M = col_max(M);
        float L = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            if (mv[i] > -INFINITY) L += fast_exp2(mv[i] - M) * lv[i];
        L = col_sum(L);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int it = i0 + q + 4 * i;
            if (it < i1) wsm[it * 16 + h4] = (mv[i] > -INFINITY && L > 0.f) ? fast_exp2(mv[i] - M) * lv[i] / L : 0.f;
        }
    }
    __syncthreads();
    if (hh >= G) return;
    float oc[NO], osl[NO], ow[NO];
#pragma unroll
    for (int k = 0; k < NO; ++k) oc[k] = osl[k] = ow[k] = 0.f;
    if (use_c) {
#pragma unroll
        for (int i = 0; i < SB; ++i)
#pragma unroll
            for (int k = 0; k < NO; ++k) oc[k] += i < ns ? cw[i] * co[i][k] : 0.f;
        for (int s0 = SB; s0 < ns; s0 += SB) {   // more than SB splits (caches past 65536 tokens)
#pragma unroll
            for (int i = 0; i < SB; ++i) {
                const int sp = min(s0 + i, ns - 1);
                cw[i] = p.cmp_w[(pb0 + sp) * 16 + hh];
                co[i].load(p.part_o + ((pb0 + sp) * 16 + hh) * DV + os.d0);
            }
#pragma unroll
            for (int i = 0; i < SB; ++i)
#pragma unroll
                for (int k = 0; k < NO; ++k) oc[k] += s0 + i < ns ? cw[i] * co[i][k] : 0.f;
        }
    }
    if (use_s) {
#pragma unroll
        for (int i = 0; i < NG; ++i)
#pragma unroll
            for (int k = 0; k < NO; ++k) osl[k] += i < n_sg ? wsm[i * 16 + hh] * so[i][k] : 0.f;
    }
    if (use_w) {
#pragma unroll
        for (int i = 0; i < NG; ++i)
#pragma unroll
            for (int k = 0; k < NO; ++k) ow[k] += n_sg + i < n_grp ? wsm[(n_sg + i) * 16 + hh] * wo[i][k] : 0.f;
    }
    float gc = 1.f, gs = 1.f, gw = 1.f;
    if (p.gates) {
        gc = sigmoidf_(z[0]);
        gs = sigmoidf_(z[1]);
        gw = sigmoidf_(z[2]);
    }
    u16 y[NO];
#pragma unroll
    for (int k = 0; k < NO; ++k) {
        float v = 0.f;
        if (p.branches & 1) v += gc * oc[k];
        if (p.branches & 2) v += gs * osl[k];
        if (p.branches & 4) v += gw * ow[k];
        y[k] = f2bf(v);
    }
    u16* op = p.O + ((size_t)b * H + g * G + hh) * DV + os.d0;
#pragma unroll
    for (int k = 0; k < NO; ++k) op[k] = y[k];
}

template <int DV>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
    extern __shared__ float wsm[];
    merge_unit<DV>(p, blockIdx.x, blockIdx.y, wsm);
}

// ---------------------------------------------------------------------------
namespace {
template <typename K>
void allow_lds(K kernel, size_t bytes) {
    if (bytes > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)bytes);
}

template <int DK, int DV>
void decode_impl(const DecodeParams& p, hipStream_t st) {
    const size_t lds_attn = (size_t)4 * 64 * (DV + 16) * 2;   // >= the combine buffers
    const size_t reuse = (size_t)4 * 16 * (DV + 4) * 4 + (size_t)16 * kPsumStride * 4;
    const size_t lds1 = (lds_attn > reuse ? lds_attn : reuse) + 128 * 4;
    const int n_sg = (p.top_n + 3) / 4, n_wg = (p.n_items - p.top_n + 3) / 4;
    allow_lds(decode_cmp_kernel<DK, DV>, lds1);
    decode_cmp_kernel<DK, DV><<<dim3(p.n_split + n_wg, p.Hkv, p.B), 256, lds1, st>>>(p);
    const size_t lds2 = ((size_t)p.n_split * 16 + p.n_slc) * 4;
    NSA_NU_SWITCH(p.n_slc, {
        allow_lds(decode_select_kernel<NU>, lds2);
        decode_select_kernel<NU><<<dim3(p.Hkv, p.B), 1024, lds2, st>>>(p);
    });
    if (n_sg > 0) {
        allow_lds(decode_attn_kernel<DK, DV>, lds_attn);
        decode_attn_kernel<DK, DV><<<dim3(n_sg, p.Hkv, p.B), 256, lds_attn, st>>>(p);
    }
    decode_merge_kernel<DV><<<dim3(p.Hkv, p.B), 256, (size_t)p.n_items * 16 * 4, st>>>(p);
}
}  // namespace

bool launch_decode(int DK, int DV, const DecodeParams& p, hipStream_t st) {
    if (DK == 192 && DV == 128) decode_impl<192, 128>(p, st);
    else if (DK == 128 && DV == 128) decode_impl<128, 128>(p, st);
    else if (DK == 64 && DV == 64) decode_impl<64, 64>(p, st);
    else return false;
    return true;
}

}  // namespace nsa
