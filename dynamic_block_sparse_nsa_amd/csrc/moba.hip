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
//   moba_scatter_kernel   per chunk: (token, slot) entries into their bucket, and the
//                         bucket of every 128-entry list tile
//   moba_attn_kernel      work item = own-block item (128 consecutive tokens of block j,
//                         causal) or bucket item (128 listed queries of block j, no mask)
//   moba_merge_kernel     per (token, head): combine the slots, gate, bf16 store
// The partial of a (token, slot) is written by exactly one work item, so results do not
// depend on the order in which entries land in a bucket.
#include <climits>

#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace nsa {

namespace {

constexpr int kCol = 128;    // query columns per work item (4 waves x 2 tiles x 16)
constexpr int kKeys = 64;    // keys per LDS tile
constexpr float kMobaLazy = 8.f;   // log2 headroom before a column's softmax reference moves
constexpr int kRun = 16;     // consecutive work items dealt to one XCD

// dynamic LDS of moba_attn_kernel: one K tile and two V tiles of 64 keys
constexpr size_t moba_attn_lds(int DK, int DV) { return (size_t)kKeys * (DK + 2 * DV) * 2; }
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

// per chunk: (token, slot) entries into their bucket.  The chunks' workgroups of a
// (sequence, head) also write the bucket of every list tile of its buckets (a direct lookup
// for the work items, instead of a search over the tile starts), the buckets split over the
// chunks.
__global__ __launch_bounds__(256) void moba_scatter_kernel(MobaParams p) {
    extern __shared__ int cursor[];   // [n_slc]
    const int c = blockIdx.x, bh = blockIdx.y;
    const int b = bh / p.Hkv, h = bh % p.Hkv;
    {
        const int jb0 = (int)((long long)c * p.n_slc / p.n_chunk);
        const int jb1 = (int)((long long)(c + 1) * p.n_slc / p.n_chunk);
        for (int jj = jb0; jj < jb1; ++jj) {
            const int bk = bh * p.n_slc + jj;
            for (int t = p.tile_start[bk] + (int)threadIdx.x; t < p.tile_start[bk + 1]; t += 256) p.tile_bucket[t] = bk;
        }
    }
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
// XCD-aware: workgroups i, i + 8, i + 16, ... run on one XCD, and the items are dealt to the
// XCDs in runs of kRun consecutive ones, so the tiles of one bucket (which share the block's
// K and V) mostly meet in one XCD's L2, while every XCD walks the item range in the same
// order: the items past the real count (the grid is an upper bound) fall at the end on every
// XCD alike.  (Dealing each XCD one contiguous eighth of the grid left the last XCDs with
// nothing but those empty items.)
template <int DK, int DV>
__global__ __launch_bounds__(256, DK >= 192 ? 2 : 3) void moba_attn_kernel(MobaParams p) {
    constexpr int NDS = DK / 32, NDT = DV / 16;
    constexpr int KE = 4 * NDS * 512;       // K elements of a 64-key tile (fragment order)
    constexpr int VE = 2 * NDT * 512;       // V elements
    // the K tile single-buffered, V tiles double-buffered, all filled by global -> LDS copies
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    u16* kslot = reinterpret_cast<u16*>(smem);   // [KE]
    u16* vslot = kslot + KE;                      // [2][VE]
    __shared__ int col_tok[kCol], col_slot[kCol];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lq = lane >> 4;
    const int xq = blockIdx.x & 7, kq = blockIdx.x >> 3;   // gridDim.x is a multiple of 8 * kRun
    const int item = (kq / kRun) * (8 * kRun) + xq * kRun + kq % kRun;
    const int n_tiles = p.n_own + p.tile_start[p.n_bucket];
    if (item >= n_tiles) return;

    // the item's (sequence, head) and block: arithmetic for own-block items, one table read
    // for bucket tiles (tile_start[bk] <= it < tile_start[bk + 1])
    const bool own = item < p.n_own;
    const int per_blk = (p.lp + kCol - 1) / kCol;
    const int it = item - p.n_own;
    const int bk = own ? 0 : p.tile_bucket[it];
    const int bh = own ? item / (p.n_slc * per_blk) : bk / p.n_slc;
    const int j = own ? (item % (p.n_slc * per_blk)) / per_blk : bk % p.n_slc;
    const int kbeg = j * p.lp;   // < T: every block holds a token

    // K rows are gathered straight from [B,Hkv,T,DK] into the fragment order of the LDS tile
    // (lane (li, lq) of 16-key group kt and step ds brings K[16kt + li][32ds + 8lq ..+8];
    // rows past T are clamped, their scores are masked or never formed); V comes from the
    // scaled fp16 copy.  (Requesting tile 0 before the lists are read was slower: the list
    // and query loads then wait behind the copies.)
    const u16* kg = p.K + (size_t)bh * p.T * DK;
    const u16* vg = p.Vf + (size_t)bh * p.Tpad * DV;
    auto issue_k = [&](int tix, u16* dst) {
        const int key_t = kbeg + kKeys * tix;
        for (int ch = wave; ch < KE / 512; ch += 4) {
            const int kt = ch / NDS, ds = ch % NDS;
            const int row = min(key_t + 16 * kt + li, p.T - 1);
            __builtin_amdgcn_global_load_lds(kg + (size_t)row * DK + 32 * ds + 8 * lq, (lds_void*)(dst + ch * 512), 16,
                                             0, 0);
        }
    };
    auto issue_v = [&](int tix) {
        const u16* src = vg + (size_t)((kbeg + kKeys * tix) / 32) * NDT * 512;
        u16* dst = vslot + (tix & 1) * VE;
        for (int ch = wave; ch < VE / 512; ch += 4)
            __builtin_amdgcn_global_load_lds(src + ch * 512 + lane * 8, (lds_void*)(dst + ch * 512), 16, 0, 0);
    };

    int ncol;
    if (own) {
        const int r = item % (p.n_slc * per_blk);
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
    const int ntile = kend >= kbeg ? (kend - kbeg) / kKeys + 1 : 0;
    // a column's last visible key (empty columns: none masked, their values are never stored)
    int hi[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) hi[c] = tok[c] >= 0 ? tok[c] : INT_MAX;
    const int hi_min = (int)wave_min_u32((uint32_t)min(hi[0], hi[1]));   // the wave's earliest limit
    if (ntile > 0) {
        issue_k(0, kslot);
        issue_v(0);
    }

    // m: the column's reference (the same in its four lanes), moved only when a tile exceeds
    // it by more than 2^8, so that o is rarely rescaled; p = 2^(x - m) <= 2^8 fits fp16
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    f32x4 o[2][NDT];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[c][dt] = zero4();

    // Copy schedule of tile tix: V(tix + 1) is requested at the tile's start (its slot held
    // V(tix - 1), whose reads ended before the barrier) and K(tix + 1) once every wave has
    // read K(tix) (the barrier after the QK products); the start of the next tile waits for
    // both.  So V's copy has a whole tile to land and K's the value products.  (A single V
    // slot refilled after the value products left V's copy no compute to hide under: the
    // barriers' own waits cover every outstanding copy.)
    static_assert(KE % 2048 == 0 && VE % 2048 == 0, "the waves split a tile's copies evenly");
    for (int tix = 0; tix < ntile; ++tix) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's copies, then everyone's
        __syncthreads();
        if (tix + 1 < ntile) issue_v(tix + 1);
        const u16* kb = kslot;
        const int key0 = kbeg + kKeys * tix;
        f32x4 s[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int c = 0; c < 2; ++c) s[kt][c] = zero4();
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const bf16x8 a = ld8(&kb[((kt * NDS + ds) * 64 + lane) * 8]);
#pragma unroll
                for (int c = 0; c < 2; ++c) s[kt][c] = mfma16(a, qf[c][ds], s[kt][c]);
            }
        if (key0 + kKeys - 1 > hi_min) {   // some column's causal limit falls in this tile
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (key0 + 16 * kt + 4 * lq + r > hi[c]) s[kt][c][r] = -INFINITY;
        }
        // a column's reference moves only on its own tile maximum, so its result does not
        // depend on which columns share its wave
        float mt[2];
        bool grow[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float tmax = vmax(s[0][c][0], s[0][c][1]);
#pragma unroll
            for (int e = 2; e < 16; e += 2) tmax = vmax(vmax(tmax, s[e >> 2][c][e & 3]), s[e >> 2][c][(e & 3) + 1]);
            mt[c] = col_max(tmax) * p.scale_log2;
            grow[c] = mt[c] > m[c] + kMobaLazy;
        }
        if (__any(grow[0] || grow[1])) {   // rescale (wave-uniform branch; factor 1 elsewhere)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const float mnew = grow[c] ? mt[c] : m[c];
                const float alpha = !grow[c] ? 1.f : m[c] == -INFINITY ? 0.f : fast_exp2(m[c] - mnew);
                l[c] *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) o[c][dt] *= alpha;
                m[c] = mnew;
            }
        }
        // masked keys give 2^-inf = 0 (every column has a visible key in its first tile)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = fast_exp2(__builtin_fmaf(s[kt][c][r], p.scale_log2, -m[c]));
                    s[kt][c][r] = e;
                    acc += e;
                }
            l[c] += acc;
        }
        // every wave's reads of K(tix) have returned (no wait on the copies in flight)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (tix + 1 < ntile) issue_k(tix + 1, kslot);
#pragma unroll
        for (int u = 0; u < 2; ++u) {   // P in fp16 against the scaled fp16 V copy: one product
            f16x8 ph[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) ph[c] = pack_p_h(s[2 * u][c], s[2 * u + 1][c]);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const f16x8 a = ld8h(&vslot[(tix & 1) * VE + ((u * NDT + dt) * 64 + lane) * 8]);
#pragma unroll
                for (int c = 0; c < 2; ++c) o[c][dt] = mfma16h(a, ph[c], o[c][dt]);
            }
        }
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
// lanes with 4 values each (a wave covers 64*4/DV rows); each thread takes R rows (RPB rows
// apart) and requests every slot's list entry, (max, sum) and fp16 output slice of all of
// them in one round trip (slots with no block may hold stale values and are dropped by
// selects), so that a wave has R times the bytes in flight; the partial outputs are read
// once (non-temporal, 8 bytes per lane) and weighted by sum * 2^(m - M); the bf16 rows are
// stored with 8-byte writes.  SM >= top_n.
template <int DV, int SM, int R>
__global__ __launch_bounds__(256) void moba_merge_kernel(MobaParams p) {
    constexpr int LPR = DV / 4;      // lanes per row
    constexpr int RPB = 256 / LPR;   // rows per workgroup and step
    const size_t nrows = (size_t)p.B * p.T * p.Hkv;
    const int li = threadIdx.x % LPR;
    auto half4 = [](const u32x2& hv) {
        return f32x4{(float)__builtin_bit_cast(_Float16, (u16)(hv[0] & 0xFFFFu)),
                     (float)__builtin_bit_cast(_Float16, (u16)(hv[0] >> 16)),
                     (float)__builtin_bit_cast(_Float16, (u16)(hv[1] & 0xFFFFu)),
                     (float)__builtin_bit_cast(_Float16, (u16)(hv[1] >> 16))};
    };
    size_t row[R];
    int js[R][SM];
    float ms[R][SM], ls[R][SM];
    u32x2 hv[R][SM];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        row[r] = ((size_t)blockIdx.x * R + r) * RPB + threadIdx.x / LPR;   // (b, t, h)
        const size_t rr = row[r] < nrows ? row[r] : nrows - 1;
#pragma unroll
        for (int s = 0; s < SM; ++s)
            if (s < p.top_n) {
                js[r][s] = p.sel[rr * p.top_n + s];
                ms[r][s] = p.part_m[rr * p.top_n + s];
                ls[r][s] = p.part_l[rr * p.top_n + s];
                hv[r][s] = ld_stream(reinterpret_cast<const u32x2*>(p.part_o + (rr * p.top_n + s) * DV) + li);
            }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (row[r] >= nrows) continue;
        float M = -INFINITY, L = 0.f;
        f32x4 acc = zero4();
        bool ok[SM];
#pragma unroll
        for (int s = 0; s < SM; ++s) {
            ok[s] = s < p.top_n && js[r][s] >= 0 && js[r][s] < p.n_slc && ms[r][s] > -INFINITY;
            M = ok[s] ? fmaxf(M, ms[r][s]) : M;
        }
#pragma unroll
        for (int s = 0; s < SM; ++s) {
            const float w = ok[s] ? fast_exp2(ms[r][s] - M) * ls[r][s] : 0.f;   // the slot's weight
            L += w;
            const f32x4 o = half4(hv[r][s]);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] += ok[s] ? w * o[k] : 0.f;
        }
        const float g = p.gates ? sigmoidf_(p.gates[row[r] * 3 + 1]) : 1.f;
        const size_t bh = row[r] / ((size_t)p.T * p.Hkv) * p.Hkv + row[r] % p.Hkv;
        const float inv = L > 0.f ? ldexpf(g / L, p.vexp[bh]) : 0.f;   // V's scaling undone
        const u32x2 v = {(uint32_t)f2bf(acc[0] * inv) | ((uint32_t)f2bf(acc[1] * inv) << 16),
                         (uint32_t)f2bf(acc[2] * inv) | ((uint32_t)f2bf(acc[3] * inv) << 16)};
        st_stream(v, reinterpret_cast<u32x2*>(p.O + row[r] * DV) + li);
    }
}

// The same merge for exactly S <= 4 slots and fewer than 2^32 rows (the MoBA workloads):
// the slot count is a compile-time constant (no per-slot branches), a lane owns 8
// consecutive values of a row (16-byte partial loads and output stores), row indices are
// 32-bit, and the (sequence, head) of a row comes from two divisions by constants the host
// passes (th = T * Hkv, hkv).  Rows past the end are clamped for the loads and not stored.
template <int DV, int S, int R>
__global__ __launch_bounds__(256) void moba_merge_small_kernel(MobaParams p, uint32_t nrows, uint32_t th, uint32_t hkv) {
    constexpr int LPR = DV / 8;      // lanes per row
    constexpr int RPB = 256 / LPR;   // rows per workgroup and step
    const uint32_t li = threadIdx.x % LPR;
    uint32_t row[R];
    int js[R][S];
    float ms[R][S], ls[R][S];
    f16x8 hv[R][S];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        row[r] = ((uint32_t)blockIdx.x * R + r) * RPB + threadIdx.x / LPR;   // (b, t, h)
        const uint32_t rr = min(row[r], nrows - 1);
#pragma unroll
        for (int s = 0; s < S; ++s) {
            js[r][s] = p.sel[rr * S + s];
            ms[r][s] = p.part_m[rr * S + s];
            ls[r][s] = p.part_l[rr * S + s];
            hv[r][s] = ld_stream(reinterpret_cast<const f16x8*>(p.part_o + (size_t)(rr * S + s) * DV) + li);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float M = -INFINITY;
        bool ok[S];
#pragma unroll
        for (int s = 0; s < S; ++s) {
            ok[s] = js[r][s] >= 0 && js[r][s] < p.n_slc && ms[r][s] > -INFINITY;
            M = ok[s] ? fmaxf(M, ms[r][s]) : M;
        }
        float L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const float w = ok[s] ? fast_exp2(ms[r][s] - M) * ls[r][s] : 0.f;   // the slot's weight
            L += w;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(w, ok[s] ? (float)hv[r][s][k] : 0.f, acc[k]);
        }
        const uint32_t rr = min(row[r], nrows - 1);
        const float g = p.gates ? sigmoidf_(p.gates[(size_t)rr * 3 + 1]) : 1.f;
        const uint32_t bh = rr / th * hkv + rr % hkv;
        const float inv = L > 0.f ? ldexpf(g / L, p.vexp[bh]) : 0.f;   // V's scaling undone
        u32x4 v;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (uint32_t)f2bf(acc[2 * k] * inv) | ((uint32_t)f2bf(acc[2 * k + 1] * inv) << 16);
        if (row[r] < nrows) st_stream(v, reinterpret_cast<u32x4*>(p.O + (size_t)row[r] * DV) + li);
    }
}

namespace {
template <int DV>
void moba_merge(const MobaParams& p, hipStream_t st) {
    constexpr int RPB = 256 / (DV / 4);
    const size_t rows = (size_t)p.B * p.T * p.Hkv;
    if (p.top_n <= 4 && rows * (size_t)p.top_n < (1ull << 32)) {
        constexpr int R = 4;
        constexpr int RPBS = 256 / (DV / 8);
        const unsigned grid = (unsigned)((rows + RPBS * R - 1) / (RPBS * R));
        const uint32_t n = (uint32_t)rows, th = (uint32_t)p.T * (uint32_t)p.Hkv, hkv = (uint32_t)p.Hkv;
        switch (p.top_n) {
            case 1: moba_merge_small_kernel<DV, 1, R><<<grid, 256, 0, st>>>(p, n, th, hkv); break;
            case 2: moba_merge_small_kernel<DV, 2, R><<<grid, 256, 0, st>>>(p, n, th, hkv); break;
            case 3: moba_merge_small_kernel<DV, 3, R><<<grid, 256, 0, st>>>(p, n, th, hkv); break;
            default: moba_merge_small_kernel<DV, 4, R><<<grid, 256, 0, st>>>(p, n, th, hkv); break;
        }
    } else if (p.top_n <= 4) {
        constexpr int R = 4;
        moba_merge_kernel<DV, 4, R><<<(unsigned)((rows + RPB * R - 1) / (RPB * R)), 256, 0, st>>>(p);
    } else if (p.top_n <= 8) {
        constexpr int R = 2;
        moba_merge_kernel<DV, 8, R><<<(unsigned)((rows + RPB * R - 1) / (RPB * R)), 256, 0, st>>>(p);
    } else {
        moba_merge_kernel<DV, 32, 1><<<(unsigned)((rows + RPB - 1) / RPB), 256, 0, st>>>(p);
    }
}
}  // namespace

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
    nwg = (nwg + 8 * kRun - 1) / (8 * kRun) * (8 * kRun);
    if (DK == 128 && DV == 128) moba_attn_kernel<128, 128><<<nwg, 256, moba_attn_lds(128, 128), st>>>(p);
    else if (DK == 64 && DV == 64) moba_attn_kernel<64, 64><<<nwg, 256, moba_attn_lds(64, 64), st>>>(p);
    else if (DK == 192 && DV == 128) moba_attn_kernel<192, 128><<<nwg, 256, moba_attn_lds(192, 128), st>>>(p);
    else return false;
    if (DV == 128) moba_merge<128>(p, st);
    else moba_merge<64>(p, st);
    return true;
}

}  // namespace nsa
