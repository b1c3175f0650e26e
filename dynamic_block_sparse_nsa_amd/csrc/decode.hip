// One NSA decode step (zjai.club notes, section 13: decoding is memory-bound, so the
// cost is the cache bytes read per step).  For each sequence the new query sits at
// t = cache_len - 1 and the result equals the prefill result for that row.
//
// The compressed cache is the bulk of the bytes (N_cmp keys and values per group), so it
// is streamed exactly once, split over many workgroups:
//   decode_cmp_kernel     split s covers 256 compressed keys of one (sequence, group);
//                         4 waves x 64 keys, the group's heads packed in the MFMA column
//                         tile.  Emits, relative to the split's per-head max m: the sum
//                         l, the unnormalized o^T, and per-head partial block sums
//                         A[h][j] = sum over this split's keys overlapping block j of
//                         2^(x - m).
//   decode_select_kernel  per (sequence, group): lse per head from the split (m, l);
//                         o_cmp = sum_s 2^(m_s - lse) o_s; block score
//                         score[j] = sum_h sum_s 2^(m_s,h - lse_h) A_s[h][j] (the exact
//                         normalized compressed probabilities, summed as in prefill);
//                         then the shared top-n.
//   decode_attn_kernel    one wave per item: a selected block, or a 64-token piece of the
//                         window; online softmax over its keys, partial (m, l, o^T).
//   decode_merge_kernel   merges the items of each branch and applies the gates.
// Value rows are key-major in the caches, so each wave transposes its value tile into
// LDS (d-major, 32-key groups permuted as in the prefill kernels) before the MFMA.
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace nsa {

int decode_jb(int l, int s, int lp) { return ((kDecodeSplitKeys - 1) * s + l - 1) / lp + 2; }

int decode_items(int top_n, int window) { return top_n + (window > 0 ? window / 64 + 2 : 0); }

namespace {

__device__ __forceinline__ int query_pos(const int32_t* cache_len, int b, int L) {
    const int n = min(max(cache_len[b], 1), L);
    return n - 1;
}

// Stage value rows [key0, key0 + NK) (clamped to < nrows) of a key-major tile into
// LDS transposed: vt[d * VSTR + (k & ~31) + vt_pos(k & 31)], k relative to key0.
template <int DV, int NK, int VSTR>
__device__ __forceinline__ void stage_vt(const u16* __restrict__ V, int key0, int nrows, u16* vt) {
    const int lane = threadIdx.x & 63;
    for (int idx = lane; idx < NK * (DV / 8); idx += 64) {
        const int k = idx / (DV / 8), d8 = (idx % (DV / 8)) * 8;
        const int row = min(key0 + k, nrows - 1);
        const uint4 v = *reinterpret_cast<const uint4*>(V + (size_t)row * DV + d8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        const int pos = (k & ~31) + vt_pos(k & 31);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vt[(d8 + 2 * i) * VSTR + pos] = (u16)(w[i] & 0xFFFFu);
            vt[(d8 + 2 * i + 1) * VSTR + pos] = (u16)(w[i] >> 16);
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void decode_cmp_kernel(DecodeParams p) {
    constexpr int NDS = DK / 32, NDT = DV / 16;
    constexpr int VSTR = 64 + 8;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    u16* vt_all = reinterpret_cast<u16*>(smem);                             // [4][DV][VSTR]
    float* psum = reinterpret_cast<float*>(vt_all + 4 * DV * VSTR);          // [16][256]
    float* wm = psum + 16 * kDecodeSplitKeys;                               // [4][16]
    float* wl = wm + 64;                                                    // [4][16]
    float* po = reinterpret_cast<float*>(smem);                              // [4][DV][16] (reuses vt)

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int b = blockIdx.z, g = blockIdx.y, sp = blockIdx.x;
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
    const bool head_ok = li < G;
    const int h = g * G + min(li, G - 1);
    bf16x8 qf[NDS];
    {
        const u16* qp = p.q + ((size_t)b * H + h) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[ds] = head_ok ? ld8(qp + 32 * ds) : zero8();
    }
    const u16* kc = p.Kc + ((size_t)b * p.Hkv + g) * (size_t)Nc * DK;
    const u16* vc = p.Vc + ((size_t)b * p.Hkv + g) * (size_t)Nc * DV;
    u16* vt = vt_all + wave * DV * VSTR;

    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        sacc[kt] = zero4();
        const u16* kp = kc + (size_t)min(kw + 16 * kt + li, Nc - 1) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) sacc[kt] = mfma16(ld8(kp + 32 * ds), qf[ds], sacc[kt]);
    }
    stage_vt<DV, 64, VSTR>(vc, kw, Nc, vt);

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
            psum[li * kDecodeSplitKeys + 64 * wave + 16 * kt + 4 * lq + r] = pr;
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
            const bf16x8 a = ld8(&vt[(16 * dt + li) * VSTR + 32 * u + lq * 8]);
            oacc[dt] = mfma16(a, bh, oacc[dt]);
            oacc[dt] = mfma16(a, bl, oacc[dt]);
        }
    }
    __syncthreads();  // every wave is done with its vt region: reuse as po
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) po[(wave * DV + 16 * dt + 4 * lq + r) * 16 + li] = oacc[dt][r];
    __syncthreads();
    for (int idx = threadIdx.x; idx < DV * 16; idx += 256) {
        const float v = po[idx] + po[DV * 16 + idx] + po[2 * DV * 16 + idx] + po[3 * DV * 16 + idx];
        p.part_o[pbase * DV * 16 + idx] = v;
    }
    if (threadIdx.x < 16) {
        const int hh = threadIdx.x;
        p.part_m[pbase * 16 + hh] = fmaxf(fmaxf(wm[hh], wm[16 + hh]), fmaxf(wm[32 + hh], wm[48 + hh]));
        p.part_l[pbase * 16 + hh] = wl[hh] + wl[16 + hh] + wl[32 + hh] + wl[48 + hh];
    }
    // per-head partial block sums over this split's keys (ascending key order)
    const int jlo = (kbeg * p.s) / p.lp;
    const int jhi = min(((kbeg + kDecodeSplitKeys - 1) * p.s + p.l - 1) / p.lp, p.n_slc - 1);
    const int nj = jhi - jlo + 1;
    for (int idx = threadIdx.x; idx < G * nj; idx += 256) {
        const int hh = idx / nj, j = jlo + idx % nj;
        const int num = j * p.lp - p.l + 1;
        const int ilo = max(kbeg, num > 0 ? (num + p.s - 1) / p.s : 0);
        const int ihi = min(kbeg + kDecodeSplitKeys - 1, (j * p.lp + p.lp - 1) / p.s);
        float acc = 0.f;
        for (int i = ilo; i <= ihi; ++i) acc += psum[hh * kDecodeSplitKeys + (i - kbeg)];
        p.part_a[(pbase * 16 + hh) * p.jb + (j - jlo)] = acc;
    }
}

// ---------------------------------------------------------------------------
template <int DV>
__global__ __launch_bounds__(256) void decode_select_kernel(DecodeParams p) {
    extern __shared__ float sm[];
    float* f = sm;                       // [n_split][16]
    float* sc = f + p.n_split * 16;      // [n_slc]
    const int g = blockIdx.x, b = blockIdx.y;
    const int t = query_pos(p.cache_len, b, p.L);
    const int nv = visible_count(t, p.l, p.s, p.Nc);
    const int ns = (nv + kDecodeSplitKeys - 1) / kDecodeSplitKeys;
    const int jc = t / p.lp;
    const size_t pb0 = ((size_t)b * p.Hkv + g) * p.n_split;
    if (threadIdx.x < 16) {
        const int hh = threadIdx.x;
        float M = -INFINITY;
        for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, p.part_m[(pb0 + sp) * 16 + hh]);
        float L = 0.f;
        for (int sp = 0; sp < ns; ++sp) L += p.part_l[(pb0 + sp) * 16 + hh] * fast_exp2(p.part_m[(pb0 + sp) * 16 + hh] - M);
        const float lse2 = M + __log2f(L);
        for (int sp = 0; sp < ns; ++sp) f[sp * 16 + hh] = fast_exp2(p.part_m[(pb0 + sp) * 16 + hh] - lse2);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * DV; idx += 256) {
        const int hh = idx / DV, d = idx % DV;
        float acc = 0.f;
        for (int sp = 0; sp < ns; ++sp) acc += f[sp * 16 + hh] * p.part_o[((pb0 + sp) * DV + d) * 16 + hh];
        p.ocmp_ws[(((size_t)b * p.Hkv + g) * 16 + hh) * DV + d] = acc;
    }
    for (int j = threadIdx.x; j <= jc; j += 256) {
        float acc = 0.f;
        for (int sp = 0; sp < ns; ++sp) {
            const int kbeg = sp * kDecodeSplitKeys;
            const int jlo = (kbeg * p.s) / p.lp;
            const int jhi = min(((kbeg + kDecodeSplitKeys - 1) * p.s + p.l - 1) / p.lp, p.n_slc - 1);
            if (j < jlo || j > jhi) continue;
            for (int hh = 0; hh < p.G; ++hh) acc += f[sp * 16 + hh] * p.part_a[((pb0 + sp) * 16 + hh) * p.jb + (j - jlo)];
        }
        sc[j] = acc;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        select_blocks_wave(sc, jc, p.top_n, p.n_init, p.n_local, p.sel_ws + ((size_t)b * p.Hkv + g) * p.top_n);
        if (p.sel_out)
            select_blocks_wave(sc, jc, p.top_n, p.n_init, p.n_local, p.sel_out + ((size_t)b * p.Hkv + g) * p.top_n);
    }
}

// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(64) void decode_attn_kernel(DecodeParams p) {
    constexpr int NDS = DK / 32, NDT = DV / 16;
    constexpr int VSTR = 32 + 8;
    __shared__ __attribute__((aligned(16))) u16 vt[DV * VSTR];
    const int lane = threadIdx.x, li = lane & 15, lq = lane >> 4;
    const int it = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int G = p.G, H = p.Hkv * G;
    const int t = query_pos(p.cache_len, b, p.L);
    const size_t ib = ((size_t)b * p.Hkv + g) * p.n_items + it;

    int lo = 0, hi = -1, c0 = 0;
    if (it < p.top_n) {
        const int j = (p.branches & 2) ? p.sel_ws[((size_t)b * p.Hkv + g) * p.top_n + it] : -1;
        if (j >= 0) { lo = j * p.lp; hi = min(j * p.lp + p.lp - 1, t); c0 = lo; }
    } else if (p.branches & 4) {
        const int t0 = max(0, t - p.window + 1);
        const int base = (t0 & ~63) + 64 * (it - p.top_n);
        if (base <= t) { lo = max(t0, base); hi = min(t, base + 63); c0 = base; }
    }
    if (hi < lo) {
        if (lq == 0) {
            p.att_m[ib * 16 + li] = -INFINITY;
            p.att_l[ib * 16 + li] = 0.f;
        }
        return;
    }
    const bool head_ok = li < G;
    const int h = g * G + min(li, G - 1);
    bf16x8 qf[NDS];
    {
        const u16* qp = p.q + ((size_t)b * H + h) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[ds] = head_ok ? ld8(qp + 32 * ds) : zero8();
    }
    const u16* kg = p.K + ((size_t)b * p.Hkv + g) * (size_t)p.L * DK;
    const u16* vg = p.V + ((size_t)b * p.Hkv + g) * (size_t)p.L * DV;
    float m = -INFINITY, l = 0.f;
    f32x4 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = zero4();
    for (int key0 = c0; key0 <= hi; key0 += 32) {
        f32x4 s0 = zero4(), s1 = zero4();
        const u16* k0p = kg + (size_t)min(key0 + li, p.L - 1) * DK + lq * 8;
        const u16* k1p = kg + (size_t)min(key0 + 16 + li, p.L - 1) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            s0 = mfma16(ld8(k0p + 32 * ds), qf[ds], s0);
            s1 = mfma16(ld8(k1p + 32 * ds), qf[ds], s1);
        }
        __syncthreads();
        stage_vt<DV, 32, VSTR>(vg, key0, p.L, vt);
        __syncthreads();
        float x[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ka = key0 + 4 * lq + r, kb = key0 + 16 + 4 * lq + r;
            x[r] = (ka >= lo && ka <= hi) ? s0[r] * p.scale_log2 : -INFINITY;
            x[4 + r] = (kb >= lo && kb <= hi) ? s1[r] * p.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, fmaxf(x[r], x[4 + r]));
        }
        tmax = col_max(tmax);
        const float mnew = fmaxf(m, tmax);
        if (mnew == -INFINITY) continue;
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
            const bf16x8 a = ld8(&vt[(16 * dt + li) * VSTR + lq * 8]);
            o[dt] *= alpha;
            o[dt] = mfma16(a, bh, o[dt]);
            o[dt] = mfma16(a, bl, o[dt]);
        }
    }
    l = col_sum(l);
    if (lq == 0) {
        p.att_m[ib * 16 + li] = m;
        p.att_l[ib * 16 + li] = l;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p.att_o[(ib * DV + 16 * dt + 4 * lq + r) * 16 + li] = o[dt][r];
}

// ---------------------------------------------------------------------------
template <int DV>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
    const int g = blockIdx.x, b = blockIdx.y;
    const int G = p.G, H = p.Hkv * G;
    const size_t ib0 = ((size_t)b * p.Hkv + g) * p.n_items;
    for (int idx = threadIdx.x; idx < G * DV; idx += 256) {
        const int hh = idx / DV, d = idx % DV;
        const int h = g * G + hh;
        float ob[2] = {0.f, 0.f};
        for (int br = 0; br < 2; ++br) {
            const int i0 = br == 0 ? 0 : p.top_n, i1 = br == 0 ? p.top_n : p.n_items;
            float M = -INFINITY;
            for (int i = i0; i < i1; ++i) M = fmaxf(M, p.att_m[(ib0 + i) * 16 + hh]);
            if (M == -INFINITY) continue;
            float L = 0.f, acc = 0.f;
            for (int i = i0; i < i1; ++i) {
                const float mi = p.att_m[(ib0 + i) * 16 + hh];
                if (mi == -INFINITY) continue;
                const float w = fast_exp2(mi - M);
                L += w * p.att_l[(ib0 + i) * 16 + hh];
                acc += w * p.att_o[((ib0 + i) * DV + d) * 16 + hh];
            }
            ob[br] = acc / L;
        }
        float gc = 1.f, gs = 1.f, gw = 1.f;
        if (p.gates) {
            const float* z = p.gates + ((size_t)b * H + h) * 3;
            gc = sigmoidf_(z[0]);
            gs = sigmoidf_(z[1]);
            gw = sigmoidf_(z[2]);
        }
        float y = 0.f;
        if (p.branches & 1) y += gc * p.ocmp_ws[(((size_t)b * p.Hkv + g) * 16 + hh) * DV + d];
        if (p.branches & 2) y += gs * ob[0];
        if (p.branches & 4) y += gw * ob[1];
        p.O[((size_t)b * H + h) * DV + d] = f2bf(y);
    }
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
    const size_t lds1 = (size_t)4 * DV * (64 + 8) * 2 + 16 * kDecodeSplitKeys * 4 + 128 * 4;
    allow_lds(decode_cmp_kernel<DK, DV>, lds1);
    decode_cmp_kernel<DK, DV><<<dim3(p.n_split, p.Hkv, p.B), 256, lds1, st>>>(p);
    const size_t lds2 = ((size_t)p.n_split * 16 + p.n_slc) * 4;
    allow_lds(decode_select_kernel<DV>, lds2);
    decode_select_kernel<DV><<<dim3(p.Hkv, p.B), 256, lds2, st>>>(p);
    decode_attn_kernel<DK, DV><<<dim3(p.n_items, p.Hkv, p.B), 64, 0, st>>>(p);
    decode_merge_kernel<DV><<<dim3(p.Hkv, p.B), 256, 0, st>>>(p);
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
