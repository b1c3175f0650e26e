// Selected-block attention, sliding window and gated sum (zjai.club notes, sections 5-6
// and 10; sunshychen.top: the query's own block is causally masked, the window crosses
// block boundaries).
//
// One wave owns one (batch, token, KV group).  The group's G query heads form the
// 16-wide MFMA column tile (the pages' NSA kernel packs the group's heads into the
// matrix dimension so every gathered KV block feeds all of them at once).  Each selected
// block is a contiguous token span, read as 32-key chunks: S^T = K_chunk . Q^T on the MFMA
// (K rows straight from memory, 16-byte loads), online softmax with the running max and
// sum in registers (base-2), then O^T += V^T_chunk . P^T with V^T taken from a
// transposed, permuted copy of V so both operands are 16-byte loads.  The window branch
// runs the same loop over its token range; the epilogue applies the sigmoid gates to
// the compressed-branch output (from the caller), o_slc and o_win and stores bf16.
#include "common.hpp"
#include "launch.hpp"

namespace nsa {


namespace {

template <int DK, int DV>
struct WaveAttn {
    static constexpr int NDS = DK / 32;
    static constexpr int NDT = DV / 16;
    f32x4 o[NDT];
    float m, l;

    __device__ void reset() {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = zero4();
        m = -INFINITY;
        l = 0.f;
    }

    // 32 keys starting at key0 (a multiple of 32); keys outside [lo, hi] are masked.
    __device__ void chunk(const bf16x8 (&qf)[NDS], const u16* kg, const u16* vtg, int Tpad, int T, int key0,
                          int lo, int hi, float scale_log2) {
        const int lane = threadIdx.x & 63, li = lane & 15, lq = lane >> 4;
        const u16* k0p = kg + (size_t)min(key0 + li, T - 1) * DK + lq * 8;
        const u16* k1p = kg + (size_t)min(key0 + 16 + li, T - 1) * DK + lq * 8;
        bf16x8 ka[NDS], kb[NDS];
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) { ka[ds] = ld8(k0p + 32 * ds); kb[ds] = ld8(k1p + 32 * ds); }
        bf16x8 va[NDT];
        const u16* vp = vtg + (size_t)li * Tpad + key0 + lq * 8;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) va[dt] = ld8(vp + (size_t)16 * dt * Tpad);
        f32x4 s0 = zero4(), s1 = zero4();
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            s0 = mfma16(ka[ds], qf[ds], s0);
            s1 = mfma16(kb[ds], qf[ds], s1);
        }
        float x[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ka_ = key0 + 4 * lq + r, kb_ = key0 + 16 + 4 * lq + r;
            x[r] = (ka_ >= lo && ka_ <= hi) ? s0[r] * scale_log2 : -INFINITY;
            x[4 + r] = (kb_ >= lo && kb_ <= hi) ? s1[r] * scale_log2 : -INFINITY;
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

    __device__ void finish() {
        const float L = col_sum(l);
        const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= inv;
    }
};

}  // namespace

template <int DK, int DV>
__global__ __launch_bounds__(256) void sparse_attn_kernel(AttnParams p) {
    constexpr int NDS = DK / 32;
    constexpr int NDT = DV / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int b = blockIdx.z, g = blockIdx.y;
    const int t = blockIdx.x * 4 + wave;
    if (t >= p.T) return;
    const int G = p.G, H = p.Hkv * G;
    const bool head_ok = li < G;
    const int h = g * G + min(li, G - 1);

    bf16x8 qf[NDS];
    {
        const u16* qp = p.Q + (((size_t)b * p.T + t) * H + h) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[ds] = head_ok ? ld8(qp + 32 * ds) : zero8();
    }
    const u16* kg = p.K + ((size_t)b * p.Hkv + g) * (size_t)p.T * DK;
    const u16* vtg = p.Vt + ((size_t)b * p.Hkv + g) * (size_t)DV * p.Tpad;

    WaveAttn<DK, DV> acc;
    f32x4 oslc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oslc[dt] = zero4();

    if (p.branches & 2) {
        acc.reset();
        const int32_t* sl = p.sel + (((size_t)b * p.T + t) * p.Hkv + g) * p.top_n;
        for (int c = 0; c < p.top_n; ++c) {
            const int j = sl[c];
            if (j < 0) break;
            const int start = j * p.lp;
            for (int key0 = start; key0 < start + p.lp && key0 <= t; key0 += 32)
                acc.chunk(qf, kg, vtg, p.Tpad, p.T, key0, start, t, p.scale_log2);
        }
        acc.finish();
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oslc[dt] = acc.o[dt];
    }
    if (p.branches & 4) {
        acc.reset();
        const int t0 = max(0, t - p.window + 1);
        for (int key0 = t0 & ~31; key0 <= t; key0 += 32)
            acc.chunk(qf, kg, vtg, p.Tpad, p.T, key0, t0, t, p.scale_log2);
        acc.finish();
    }
    if (!head_ok) return;
    float gc = 1.f, gs = 1.f, gw = 1.f;
    const size_t row = ((size_t)b * p.T + t) * H + h;
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
        float v[4] = {oc.x, oc.y, oc.z, oc.w};
        uint32_t w[2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float y = 0.f;
            if (p.branches & 1) y += gc * v[r];
            if (p.branches & 2) y += gs * oslc[dt][r];
            if (p.branches & 4) y += gw * acc.o[dt][r];
            v[r] = y;
        }
        w[0] = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        w[1] = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
        *reinterpret_cast<uint2*>(p.O + row * DV + d0) = make_uint2(w[0], w[1]);
    }
}

bool launch_sparse_attn(int DK, int DV, const AttnParams& p, int B, hipStream_t st) {
    dim3 grid((p.T + 3) / 4, p.Hkv, B);
    if (DK == 192 && DV == 128) sparse_attn_kernel<192, 128><<<grid, 256, 0, st>>>(p);
    else if (DK == 128 && DV == 128) sparse_attn_kernel<128, 128><<<grid, 256, 0, st>>>(p);
    else if (DK == 64 && DV == 64) sparse_attn_kernel<64, 64><<<grid, 256, 0, st>>>(p);
    else return false;
    return true;
}

}  // namespace nsa
