// Dense causal attention with grouped query heads: every query row attends all keys at or
// before its position.  This is the computation NSA is measured against (zjai.club notes,
// summary bullets and section 13: a full-attention kernel written the same way, close to
// 10x slower near 64K tokens, the gap growing with length); it also computes the
// select-every-block special case of the selected branch.
//
// full_attn_kernel: a workgroup of 4 waves owns 128 query rows of one KV group (G heads of
// 128/G consecutive tokens; each wave two 16-column MFMA tiles laid out by QMap).  Keys and
// values come from the fragment-order copies that the compressed branch's layout kernel
// writes (K in bf16, V in fp16 scaled by a power of two per (b, g)), 64 keys per tile,
// copied global -> LDS asynchronously: K double-buffered, V single-buffered.  Per tile:
// S^T = K.Q^T (bf16 MFMA), online softmax with a lazily moved reference (the running max
// is raised only when a tile exceeds it by more than 2^8, so the accumulators are rarely
// rescaled and p stays below 2^8), O^T += V^T.P^T with P in fp16.  Every tile but the one
// holding the workgroup's own tokens is visible to all rows.
#include "common.hpp"
#include "launch.hpp"

namespace nsa {

namespace {

constexpr int kWaves = 4;
constexpr int kKeys = 64;
constexpr float kLazy = 8.f;   // log2 headroom before the softmax reference moves

}  // namespace

template <int DK, int DV, int G, int NQ>
__global__ __launch_bounds__(256, 2) void full_attn_kernel(FullParams p) {
    constexpr int TQ = kWaves * NQ * 16 / G;   // tokens per workgroup (divides 64)
    constexpr int NDS = DK / 32, NDT = DV / 16;
    constexpr int KE = 4 * NDS * 512;          // K elements of a 64-key tile (fragment order)
    constexpr int VE = 2 * NDT * 512;          // V elements
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    u16* kslot = reinterpret_cast<u16*>(smem);   // [2][KE]
    u16* vbuf = kslot + 2 * KE;                   // [VE]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lq = lane >> 4;
    const int T = p.T;
    const int n_tiles = (T + TQ - 1) / TQ;
    int unit, it;
    if (!xcd_map_tile(blockIdx.x, p.B * p.Hkv, n_tiles, unit, it)) return;
    const int b = unit / p.Hkv, g = unit % p.Hkv;
    const int H = p.Hkv * G;
    const int tok0 = (n_tiles - 1 - it) * TQ;   // the longest rows first
    const float sl2 = p.scale_log2;

    using M = QMap<G, NQ>;
    bf16x8 qf[NQ][NDS];
    int tok[NQ], hl[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        tok[c] = tok0 + wave * M::TPW + M::token(c, li);
        hl[c] = M::head(c, li);
        const u16* qp = p.Q + (((size_t)b * T + min(tok[c], T - 1)) * H + g * G + hl[c]) * DK + lq * 8;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
            qf[c][ds] = __builtin_bit_cast(bf16x8, ld_stream(reinterpret_cast<const u32x4*>(qp + 32 * ds)));
    }
    // keys 0 .. last token; tiles [0, nfull) lie entirely at or before the first token
    const int t_last = min(tok0 + TQ - 1, T - 1);
    const int ntile = t_last / kKeys + 1;
    const int nfull = tok0 / kKeys;
    const u16* kg = p.Kf + (size_t)unit * p.Tpad * DK;
    const u16* vg = p.Vf + (size_t)unit * p.Tpad * DV;

    auto issue_k = [&](int tix, u16* dst) {
        const u16* src = kg + (size_t)tix * KE;
        for (int ch = wave; ch < KE / 512; ch += kWaves)
            __builtin_amdgcn_global_load_lds(src + ch * 512 + lane * 8, (lds_void*)(dst + ch * 512), 16, 0, 0);
    };
    auto issue_v = [&](int tix) {
        const u16* src = vg + (size_t)tix * VE;
        for (int ch = wave; ch < VE / 512; ch += kWaves)
            __builtin_amdgcn_global_load_lds(src + ch * 512 + lane * 8, (lds_void*)(vbuf + ch * 512), 16, 0, 0);
    };

    float m[NQ], l[NQ];   // m: the column's reference (same in its four lanes); l: this lane's partial sum
    f32x4 oacc[NDT][NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        m[c] = -INFINITY;
        l[c] = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt][c] = zero4();
    }

    auto step = [&](int tix, bool full) {
        // this thread's copies of tile tix have landed, then everyone's have
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tix + 1 < ntile) issue_k(tix + 1, kslot + ((tix + 1) & 1) * KE);
        const u16* kb = kslot + (tix & 1) * KE;
        const int k0 = tix * kKeys;
        f32x4 s[4][NQ];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int c = 0; c < NQ; ++c) s[kt][c] = zero4();
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const bf16x8 a = ld8(&kb[((kt * NDS + ds) * 64 + lane) * 8]);
#pragma unroll
                for (int c = 0; c < NQ; ++c) s[kt][c] = mfma16(a, qf[c][ds], s[kt][c]);
            }
        if (!full) {   // keys after a row's own token
#pragma unroll
            for (int c = 0; c < NQ; ++c)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (k0 + 16 * kt + 4 * lq + r > tok[c]) s[kt][c][r] = -INFINITY;
        }
        // tile maximum of each column (the scale is positive: max of raw scores)
        float mt[NQ];
        bool grow = false;
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            float tmax = vmax(s[0][c][0], s[0][c][1]);
#pragma unroll
            for (int e = 2; e < 16; e += 2) tmax = vmax(vmax(tmax, s[e >> 2][c][e & 3]), s[e >> 2][c][(e & 3) + 1]);
            mt[c] = col_max(tmax) * sl2;
            grow |= mt[c] > m[c] + kLazy;
        }
        if (__any(grow)) {   // move the references (wave-uniform branch)
#pragma unroll
            for (int c = 0; c < NQ; ++c) {
                const float mnew = fmaxf(m[c], mt[c]);
                const float alpha = m[c] == -INFINITY ? 0.f : fast_exp2(m[c] - mnew);
                l[c] *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) oacc[dt][c] *= alpha;
                m[c] = mnew;
            }
        }
        // p = 2^(x - m) <= 2^8, masked keys give 0
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = fast_exp2(__builtin_fmaf(s[kt][c][r], sl2, -m[c]));
                    s[kt][c][r] = v;
                    acc += v;
                }
            l[c] += acc;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f16x8 pb[NQ];
#pragma unroll
            for (int c = 0; c < NQ; ++c) pb[c] = pack_p_h(s[2 * u][c], s[2 * u + 1][c]);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const f16x8 a = ld8h(&vbuf[((u * NDT + dt) * 64 + lane) * 8]);
#pragma unroll
                for (int c = 0; c < NQ; ++c) oacc[dt][c] = mfma16h(a, pb[c], oacc[dt][c]);
            }
        }
        // every wave has issued its value products, so its reads of the V slot returned;
        // no wait on this thread's outstanding copies
        asm volatile("s_barrier" ::: "memory");
        if (tix + 1 < ntile) issue_v(tix + 1);
    };

    issue_k(0, kslot);
    issue_v(0);
    for (int tix = 0; tix < nfull; ++tix) step(tix, true);
    for (int tix = nfull; tix < ntile; ++tix) step(tix, false);

    const float vs = ldexpf(1.0f, p.vexp[unit]);   // undo the fp16 value copy's scaling
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
        const float L = col_sum(l[c]);
        if (tok[c] >= T) continue;
        const float inv = vs / L;
        u16* op = p.O + (((size_t)b * T + tok[c]) * H + g * G + hl[c]) * DV + 4 * lq;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const uint32_t w0 = (uint32_t)f2bf(oacc[dt][c][0] * inv) | ((uint32_t)f2bf(oacc[dt][c][1] * inv) << 16);
            const uint32_t w1 = (uint32_t)f2bf(oacc[dt][c][2] * inv) | ((uint32_t)f2bf(oacc[dt][c][3] * inv) << 16);
            st_stream(u32x2{w0, w1}, reinterpret_cast<u32x2*>(op + 16 * dt));
        }
    }
}

// ---------------------------------------------------------------------------
namespace {
template <int DK, int DV, int G>
void full_g(const FullParams& p, hipStream_t st) {
    constexpr int NQ = G == 1 ? 1 : 2;
    constexpr int TQ = kWaves * NQ * 16 / G;
    const size_t lds = full_attn_lds_bytes(DK, DV);
    const void* fn = reinterpret_cast<const void*>(full_attn_kernel<DK, DV, G, NQ>);
    if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    full_attn_kernel<DK, DV, G, NQ><<<xcd_grid(p.B * p.Hkv, (p.T + TQ - 1) / TQ), 256, lds, st>>>(p);
}

template <int DK, int DV>
bool full_dk(int G, const FullParams& p, hipStream_t st) {
    switch (G) {
        case 1: full_g<DK, DV, 1>(p, st); return true;
        case 2: full_g<DK, DV, 2>(p, st); return true;
        case 4: full_g<DK, DV, 4>(p, st); return true;
        case 8: full_g<DK, DV, 8>(p, st); return true;
        case 16: full_g<DK, DV, 16>(p, st); return true;
        default: return false;
    }
}
}  // namespace

size_t full_attn_lds_bytes(int DK, int DV) { return (size_t)kKeys * (2 * DK + DV) * 2; }

bool launch_full_attn(int DK, int DV, int G, const FullParams& p, hipStream_t st) {
    if (DK == 192 && DV == 128) return full_dk<192, 128>(G, p, st);
    if (DK == 128 && DV == 128) return full_dk<128, 128>(G, p, st);
    if (DK == 64 && DV == 64) return full_dk<64, 64>(G, p, st);
    return false;
}

}  // namespace nsa
