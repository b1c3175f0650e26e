// Selected-block attention with one query head per KV head (G = 1) and the selected branch
// only: the MoBA configuration (zjai.club notes, sections 16-17: every head scores and picks
// its own blocks; 512-token blocks, top 3 with the current block; sunshychen.top: the
// current block is causally masked).
//
// With G = 1 a query-centric kernel fills one of the 16 MFMA columns and gathers whole
// blocks per query.  Here the schedule is inverted: for every (sequence, head, block) the
// queries that selected the block are listed, and a workgroup runs flash attention of one
// block's keys against up to 128 of those queries, writing a partial (m, l, o) for the
// query's list slot; a merge combines each query's slots.
//   moba_hist_kernel      per 1024-token chunk: LDS histogram of selected blocks (the query's
//                         own block is excluded; it is scheduled implicitly, see below)
//   moba_prefix_kernel    per bucket (bh, j): exclusive prefix over chunks, bucket total
//   moba_scan_kernel      one workgroup: bucket starts and 128-query tile starts
//   moba_scatter_kernel   per chunk: (token, slot) entries into their bucket
//   moba_attn_kernel      work item = own-block item (128 consecutive tokens of block j,
//                         causal) or bucket item (128 listed queries of block j, no mask)
//   moba_merge_kernel     per (token, head): combine the slots, gate, bf16 store
// The partial of a (token, slot) is written by exactly one work item, so results do not
// depend on the order in which entries land in a bucket.
#include "common.hpp"
#include "launch.hpp"

namespace nsa {

namespace {

constexpr int kCol = 128;    // query columns per work item (4 waves x 2 tiles x 16)
constexpr int kKeys = 64;    // keys per LDS tile
static_assert(kCol == kBwdTile, "the backward's work items use the lists' 128-entry tiles");

}  // namespace

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moba_hist_kernel(MobaParams p) {
    extern __shared__ int hist[];   // [n_slc]
    const int c = blockIdx.x, bh = blockIdx.y;
    const int b = bh / p.Hkv, h = bh % p.Hkv;
    for (int j = threadIdx.x; j < p.n_slc; j += 256) hist[j] = 0;
    __syncthreads();
    const int t0 = c * kMobaChunk, t1 = min(t0 + kMobaChunk, p.T);
    for (int e = threadIdx.x; e < (t1 - t0) * p.top_n; e += 256) {
        const int t = t0 + e / p.top_n, s = e % p.top_n;
        const int j = p.sel[(((size_t)b * p.T + t) * p.Hkv + h) * p.top_n + s];
        if (j >= 0 && j < p.n_slc && (p.keep_own || j != t / p.lp)) atomicAdd(&hist[j], 1);
    }
    __syncthreads();
    int* out = p.hist + ((size_t)bh * p.n_chunk + c) * p.n_slc;
    for (int j = threadIdx.x; j < p.n_slc; j += 256) out[j] = hist[j];
}

// per bucket: counts over chunks -> exclusive prefix (in place), total -> bucket_cnt
__global__ __launch_bounds__(256) void moba_prefix_kernel(MobaParams p) {
    const int bk = blockIdx.x * 256 + threadIdx.x;
    if (bk >= p.n_bucket) return;
    const int bh = bk / p.n_slc, j = bk % p.n_slc;
    int* col = p.hist + (size_t)bh * p.n_chunk * p.n_slc + j;
    int run = 0;
    int c = 0;
    for (; c + 8 <= p.n_chunk; c += 8) {
        int v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = col[(size_t)(c + i) * p.n_slc];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            col[(size_t)(c + i) * p.n_slc] = run;
            run += v[i];
        }
    }
    for (; c < p.n_chunk; ++c) {
        const int v = col[(size_t)c * p.n_slc];
        col[(size_t)c * p.n_slc] = run;
        run += v;
    }
    p.bucket_cnt[bk] = run;
}

// one workgroup of 1024 threads: exclusive scans of bucket sizes and of their tile counts
__global__ __launch_bounds__(1024) void moba_scan_kernel(MobaParams p) {
    __shared__ int part_e[1024], part_t[1024];
    const int per = (p.n_bucket + 1023) / 1024;
    const int lo = threadIdx.x * per, hi = min(lo + per, p.n_bucket);
    int se = 0, st = 0;
    for (int k = lo; k < hi; ++k) {
        const int n = p.bucket_cnt[k];
        se += n;
        st += (n + kCol - 1) / kCol;
    }
    part_e[threadIdx.x] = se;
    part_t[threadIdx.x] = st;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {   // inclusive Hillis-Steele scan
        const int ae = threadIdx.x >= off ? part_e[threadIdx.x - off] : 0;
        const int at = threadIdx.x >= off ? part_t[threadIdx.x - off] : 0;
        __syncthreads();
        part_e[threadIdx.x] += ae;
        part_t[threadIdx.x] += at;
        __syncthreads();
    }
    int re = threadIdx.x > 0 ? part_e[threadIdx.x - 1] : 0;
    int rt = threadIdx.x > 0 ? part_t[threadIdx.x - 1] : 0;
    for (int k = lo; k < hi; ++k) {
        const int n = p.bucket_cnt[k];
        p.bucket_start[k] = re;
        p.tile_start[k] = rt;
        re += n;
        rt += (n + kCol - 1) / kCol;
    }
    if (threadIdx.x == 1023) {
        p.bucket_start[p.n_bucket] = part_e[1023];
        p.tile_start[p.n_bucket] = part_t[1023];
    }
}

__global__ __launch_bounds__(256) void moba_scatter_kernel(MobaParams p) {
    extern __shared__ int cursor[];   // [n_slc]
    const int c = blockIdx.x, bh = blockIdx.y;
    const int b = bh / p.Hkv, h = bh % p.Hkv;
    const int* pre = p.hist + ((size_t)bh * p.n_chunk + c) * p.n_slc;
    for (int j = threadIdx.x; j < p.n_slc; j += 256) cursor[j] = p.bucket_start[bh * p.n_slc + j] + pre[j];
    __syncthreads();
    const int t0 = c * kMobaChunk, t1 = min(t0 + kMobaChunk, p.T);
    for (int e = threadIdx.x; e < (t1 - t0) * p.top_n; e += 256) {
        const int t = t0 + e / p.top_n, s = e % p.top_n;
        const int j = p.sel[(((size_t)b * p.T + t) * p.Hkv + h) * p.top_n + s];
        if (j >= 0 && j < p.n_slc && (p.keep_own || j != t / p.lp)) {
            const int pos = atomicAdd(&cursor[j], 1);
            p.entries[pos] = (t << 5) | s;
        }
    }
}

// ---------------------------------------------------------------------------
// Work items: [0, n_own) own-block items, then bucket tiles.  Item -> workgroup mapping is
// XCD-aware: workgroups i, i + 8, i + 16, ... run on one XCD, so consecutive items (the
// tiles of one bucket, sharing the block's K and V) are given to the same XCD's L2.
template <int DK, int DV>
__global__ __launch_bounds__(256, 2) void moba_attn_kernel(MobaParams p) {
    constexpr int NDS = DK / 32, NDT = DV / 16;
    constexpr int KE = 4 * NDS * 512;       // K elements of a 64-key tile (fragment order)
    constexpr int VE = 2 * NDT * 512;       // V elements
    __shared__ __attribute__((aligned(16))) u16 kbuf[2][KE];
    __shared__ __attribute__((aligned(16))) u16 vbuf[2][VE];
    __shared__ int col_tok[kCol], col_slot[kCol];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int nwg = gridDim.x;
    const int item = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;   // nwg is a multiple of 8
    const int n_tiles = p.n_own + p.tile_start[p.n_bucket];
    if (item >= n_tiles) return;

    int bh, j, ncol;
    bool own;
    if (item < p.n_own) {
        own = true;
        const int per_blk = (p.lp + kCol - 1) / kCol;
        bh = item / (p.n_slc * per_blk);
        const int r = item % (p.n_slc * per_blk);
        j = r / per_blk;
        const int t0 = j * p.lp + (r % per_blk) * kCol;
        const int t1 = min(min(t0 + kCol, (j + 1) * p.lp), p.T);
        ncol = max(0, t1 - t0);
        const int b = bh / p.Hkv, h = bh % p.Hkv;
        for (int cix = threadIdx.x; cix < kCol; cix += 256) {
            int tk = -1, sl = 0;
            if (cix < ncol) {
                const int t = t0 + cix;
                const int32_t* row = p.sel + (((size_t)b * p.T + t) * p.Hkv + h) * p.top_n;
                for (int s = 0; s < p.top_n; ++s)
                    if (row[s] == j) { tk = t; sl = s; }
            }
            col_tok[cix] = tk;
            col_slot[cix] = sl;
        }
    } else {
        own = false;
        const int it = item - p.n_own;
        int lo = 0, hi = p.n_bucket - 1;   // bucket with tile_start[bk] <= it < tile_start[bk + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.tile_start[mid] <= it) lo = mid;
            else hi = mid - 1;
        }
        const int bk = lo;
        bh = bk / p.n_slc;
        j = bk % p.n_slc;
        const int e0 = p.bucket_start[bk] + (it - p.tile_start[bk]) * kCol;
        ncol = min(kCol, p.bucket_start[bk + 1] - e0);
        for (int cix = threadIdx.x; cix < kCol; cix += 256) {
            const int e = cix < ncol ? p.entries[e0 + cix] : -1;
            col_tok[cix] = e >= 0 ? (e >> 5) : -1;
            col_slot[cix] = e >= 0 ? (e & 31) : 0;
        }
    }
    __syncthreads();
    const int b = bh / p.Hkv, h = bh % p.Hkv;

    // this wave's two column tiles
    int tok[2], slot[2];
    bf16x8 qf[2][NDS];
    int tmax_wg = -1;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int cix = wave * 32 + c * 16 + li;
        tok[c] = col_tok[cix];
        slot[c] = col_slot[cix];
        const int tt = max(tok[c], 0);
        const u16* qp = p.Q + (((size_t)b * p.T + tt) * p.Hkv + h) * DK + 8 * lq;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[c][ds] = tok[c] >= 0 ? ld8(qp + 32 * ds) : zero8();
    }
    // keys of block j to visit: all of it, or (own block) up to the last listed token
    int kend = min((j + 1) * p.lp, p.T) - 1;
    if (own) {
        for (int cix = 0; cix < kCol; ++cix) tmax_wg = max(tmax_wg, col_tok[cix]);
        kend = min(kend, tmax_wg);
    }
    const int kbeg = j * p.lp;
    const int ntile = kend >= kbeg ? (kend - kbeg) / kKeys + 1 : 0;

    const u16* kg = p.Kf + (size_t)bh * p.Tpad * DK;
    const u16* vg = p.Vf + (size_t)bh * p.Tpad * DV;
    // a 64-key tile in fragment order is KE + VE contiguous elements of the copies; it is
    // loaded to registers before a tile's math and stored to the other LDS buffer after it
    u32x4 rk[KE / 2048], rv[VE / 2048];
    auto load = [&](int tix) {
        const int key0 = kbeg + kKeys * min(tix, max(ntile - 1, 0));
        const u16* ks = kg + (size_t)(key0 / 16) * NDS * 512;
        const u16* vs = vg + (size_t)(key0 / 32) * NDT * 512;
#pragma unroll
        for (int i = 0; i < KE / 2048; ++i) rk[i] = *reinterpret_cast<const u32x4*>(ks + (threadIdx.x + 256 * i) * 8);
#pragma unroll
        for (int i = 0; i < VE / 2048; ++i) rv[i] = *reinterpret_cast<const u32x4*>(vs + (threadIdx.x + 256 * i) * 8);
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KE / 2048; ++i) *reinterpret_cast<u32x4*>(&kbuf[buf][(threadIdx.x + 256 * i) * 8]) = rk[i];
#pragma unroll
        for (int i = 0; i < VE / 2048; ++i) *reinterpret_cast<u32x4*>(&vbuf[buf][(threadIdx.x + 256 * i) * 8]) = rv[i];
    };

    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    f32x4 o[2][NDT];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[c][dt] = zero4();

    if (ntile > 0) {
        load(0);
        store(0);
    }
    __syncthreads();
    for (int tix = 0; tix < ntile; ++tix) {
        const int buf = tix & 1;
        load(tix + 1);   // unconditional (clamped): every wait covers only what it consumes
        const int key0 = kbeg + kKeys * tix;
        f32x4 s[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int c = 0; c < 2; ++c) s[kt][c] = zero4();
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                const bf16x8 a = ld8(&kbuf[buf][((kt * NDS + ds) * 64 + lane) * 8]);
#pragma unroll
                for (int c = 0; c < 2; ++c) s[kt][c] = mfma16(a, qf[c][ds], s[kt][c]);
            }
        }
        f32x4 pv[4][2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int hi_key = tok[c];   // causal limit of this column (whole block for earlier blocks)
            float x[16];
            float tm = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = key0 + 16 * kt + 4 * lq + r;
                    x[kt * 4 + r] = key <= hi_key ? s[kt][c][r] * p.scale_log2 : -INFINITY;
                    tm = fmaxf(tm, x[kt * 4 + r]);
                }
            tm = col_max(tm);
            const float mnew = fmaxf(m[c], tm);
            const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(m[c] - mnew);
            float ps = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = mnew == -INFINITY ? 0.f : fast_exp2(x[kt * 4 + r] - mnew);
                    pv[kt][c][r] = e;
                    ps += e;
                }
            l[c] = l[c] * alpha + ps;
            m[c] = mnew;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[c][dt] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {   // P in fp16 against the scaled fp16 V copy: one product
            f16x8 ph[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) ph[c] = pack_p_h(pv[2 * u][c], pv[2 * u + 1][c]);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const f16x8 a = ld8h(&vbuf[buf][((u * NDT + dt) * 64 + lane) * 8]);
#pragma unroll
                for (int c = 0; c < 2; ++c) o[c][dt] = mfma16h(a, ph[c], o[c][dt]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // the staging stores stay after this tile's math
        store(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const float L = col_sum(l[c]);
        if (tok[c] < 0) continue;
        const size_t pr = (((size_t)b * p.T + tok[c]) * p.Hkv + h) * p.top_n + slot[c];
        if (lq == 0) {
            p.part_m[pr] = m[c];
            p.part_l[pr] = L;
        }
        // the slot's output normalized by its own sum, in V's scaled units (|o| <= 2^14), in
        // fp16: half the bytes of the partial round trip, 2^-11 relative rounding
        const float inv = L > 0.f ? 1.f / L : 0.f;
        u16* op = p.part_o + pr * DV + 4 * lq;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const _Float16 h0 = (_Float16)(o[c][dt][0] * inv), h1 = (_Float16)(o[c][dt][1] * inv);
            const _Float16 h2 = (_Float16)(o[c][dt][2] * inv), h3 = (_Float16)(o[c][dt][3] * inv);
            const u32x2 w = {(uint32_t)__builtin_bit_cast(u16, h0) | ((uint32_t)__builtin_bit_cast(u16, h1) << 16),
                             (uint32_t)__builtin_bit_cast(u16, h2) | ((uint32_t)__builtin_bit_cast(u16, h3) << 16)};
            *reinterpret_cast<u32x2*>(op + 16 * dt) = w;
        }
    }
}

// per (token, head): combine the slots of the token's list.  A row of DV values is DV/4
// lanes with 4 values each (a wave covers 64*4/DV rows); the slots' fp16 partial outputs
// are read once (non-temporal, 8 bytes per lane) and weighted by sum * 2^(m - M); the bf16
// row is stored with 8-byte writes.
template <int DV>
__global__ __launch_bounds__(256) void moba_merge_kernel(MobaParams p) {
    constexpr int LPR = DV / 4;      // lanes per row
    constexpr int RPB = 256 / LPR;   // rows per workgroup
    const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;   // (b, t, h)
    const int li = threadIdx.x % LPR;
    if (row >= (size_t)p.B * p.T * p.Hkv) return;
    const int32_t* sel = p.sel + row * p.top_n;
    float M = -INFINITY;
    float L = 0.f;
    f32x4 acc = zero4();
    auto half4 = [](const u32x2& hv) {
        return f32x4{(float)__builtin_bit_cast(_Float16, (u16)(hv[0] & 0xFFFFu)),
                     (float)__builtin_bit_cast(_Float16, (u16)(hv[0] >> 16)),
                     (float)__builtin_bit_cast(_Float16, (u16)(hv[1] & 0xFFFFu)),
                     (float)__builtin_bit_cast(_Float16, (u16)(hv[1] >> 16))};
    };
    constexpr int SMAX = 8;
    if (p.top_n <= SMAX) {
        // every slot's list entry, (max, sum) and output slice requested together (one round
        // trip); slots with no block may hold stale values and are dropped by selects
        int js[SMAX];
        float ms[SMAX], ls[SMAX];
        u32x2 hv[SMAX];
#pragma unroll
        for (int s = 0; s < SMAX; ++s)
            if (s < p.top_n) {
                js[s] = sel[s];
                ms[s] = p.part_m[row * p.top_n + s];
                ls[s] = p.part_l[row * p.top_n + s];
                hv[s] = ld_stream(reinterpret_cast<const u32x2*>(p.part_o + (row * p.top_n + s) * DV) + li);
            }
        bool ok[SMAX];
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
            ok[s] = s < p.top_n && js[s] >= 0 && ms[s] > -INFINITY;
            M = ok[s] ? fmaxf(M, ms[s]) : M;
        }
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
            const float w = ok[s] ? fast_exp2(ms[s] - M) * ls[s] : 0.f;   // the slot's weight
            L += w;
            const f32x4 o = half4(hv[s]);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] += ok[s] ? w * o[k] : 0.f;
        }
    } else {
    for (int s = 0; s < p.top_n; ++s)
        if (sel[s] >= 0) M = fmaxf(M, p.part_m[row * p.top_n + s]);
    if (M > -INFINITY) {
        for (int s = 0; s < p.top_n; ++s) {
            if (sel[s] < 0) continue;
            const float ms = p.part_m[row * p.top_n + s];
            if (ms == -INFINITY) continue;
            const float w = fast_exp2(ms - M) * p.part_l[row * p.top_n + s];   // the slot's weight
            L += w;
            const u32x2 hv = ld_stream(reinterpret_cast<const u32x2*>(p.part_o + (row * p.top_n + s) * DV) + li);
            acc += w * half4(hv);
        }
    }
    }
    const float g = p.gates ? sigmoidf_(p.gates[row * 3 + 1]) : 1.f;
    const size_t bh = row / ((size_t)p.T * p.Hkv) * p.Hkv + row % p.Hkv;
    const float inv = L > 0.f ? ldexpf(g / L, p.vexp[bh]) : 0.f;   // V's scaling undone
    const u32x2 v = {(uint32_t)f2bf(acc[0] * inv) | ((uint32_t)f2bf(acc[1] * inv) << 16),
                     (uint32_t)f2bf(acc[2] * inv) | ((uint32_t)f2bf(acc[3] * inv) << 16)};
    st_stream(v, reinterpret_cast<u32x2*>(p.O + row * DV) + li);
}

// ---------------------------------------------------------------------------
int moba_n_chunk(int T) { return (T + kMobaChunk - 1) / kMobaChunk; }

int moba_n_own(int BH, int n_slc, int lp) { return BH * n_slc * ((lp + kCol - 1) / kCol); }

int moba_max_tiles(int BH, int T, int top_n, int n_slc) {
    // every bucket contributes at most ceil(n / 128) <= n / 128 + 1 tiles
    return (int)(((long long)BH * T * top_n) / kCol) + BH * n_slc;
}

void launch_block_lists(const MobaParams& p, hipStream_t st) {
    const size_t lds_cnt = (size_t)p.n_slc * 4;
    moba_hist_kernel<<<dim3(p.n_chunk, p.B * p.Hkv), 256, lds_cnt, st>>>(p);
    moba_prefix_kernel<<<(p.n_bucket + 255) / 256, 256, 0, st>>>(p);
    moba_scan_kernel<<<1, 1024, 0, st>>>(p);
    moba_scatter_kernel<<<dim3(p.n_chunk, p.B * p.Hkv), 256, lds_cnt, st>>>(p);
}

bool launch_moba_attn(int DK, int DV, const MobaParams& p, hipStream_t st) {
    launch_block_lists(p, st);
    int nwg = p.n_own + moba_max_tiles(p.B * p.Hkv, p.T, p.top_n, p.n_slc);
    nwg = (nwg + 7) / 8 * 8;
    if (DK == 128 && DV == 128) moba_attn_kernel<128, 128><<<nwg, 256, 0, st>>>(p);
    else if (DK == 64 && DV == 64) moba_attn_kernel<64, 64><<<nwg, 256, 0, st>>>(p);
    else if (DK == 192 && DV == 128) moba_attn_kernel<192, 128><<<nwg, 256, 0, st>>>(p);
    else return false;
    const size_t rows = (size_t)p.B * p.T * p.Hkv;
    if (DV == 128) moba_merge_kernel<128><<<(unsigned)((rows + 7) / 8), 256, 0, st>>>(p);
    else moba_merge_kernel<64><<<(unsigned)((rows + 15) / 16), 256, 0, st>>>(p);
    return true;
}

}  // namespace nsa
