// Decode cache maintenance (zjai.club notes, section 5: the compressed cache grows by one
// entry every s tokens; section 13: decoding runs against these caches).  Appending n_new
// tokens to a sequence writes them into the raw caches and computes every compressed block
// whose last token is among them, with exactly the arithmetic of the prefill compression
// (compress_linear_kernel: the same four reduction ranges, each in the same MFMA order, added
// in the same order, the same fp32 bias vec(PE).W, one bf16 rounding), so an appended entry
// equals the prefill's bit for bit.
//
// cache_append_kernel, grid (ceil(BG * R / 64), n_ct + 1): rows are (sequence-group,
// candidate block) pairs, R candidates per group (the most blocks one append can complete);
// a wave computes 16 rows x 64 output columns, so W streams once per 16 groups.  Column
// tiles 0 .. dk/64-1 produce K entries, the next dv/64 tiles V entries; the last grid row
// copies the new tokens into the raw caches.  Block tokens at or past the old length are
// read from the new-token arrays, so the copy and the compression need no ordering.
// cache_advance_kernel then moves every cache_len past the new tokens.
#include "common.hpp"
#include "launch.hpp"

namespace nsa {

namespace {

__device__ __forceinline__ int old_len(const AppendParams& p, int b) { return min(max(p.cache_len[b], 0), p.L); }

// blocks [lo, hi] of a sequence whose last token falls in [c0, c_end)
__device__ __forceinline__ void completed_blocks(const AppendParams& p, int c0, int& lo, int& hi) {
    const int c_end = min(c0 + p.n_new, p.L);
    const int num = c0 - p.l + 1;   // block i is complete at c0 iff i*s + l - 1 < c0
    lo = num > 0 ? (num + p.s - 1) / p.s : 0;
    hi = c_end >= p.l ? min((c_end - p.l) / p.s, p.N - 1) : -1;
}

}  // namespace

__global__ __launch_bounds__(256) void cache_append_kernel(AppendParams p) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int BG = p.B * p.Hkv;
    const int nct_k = p.dk / 64, nct = nct_k + p.dv / 64;
    if ((int)blockIdx.y == nct) {   // copy the new tokens into the raw caches
        for (int bg = blockIdx.x; bg < BG; bg += gridDim.x) {
            const int c0 = old_len(p, bg / p.Hkv);
            const int n = min(p.n_new, p.L - c0);
            const u32x4* ks = reinterpret_cast<const u32x4*>(p.K_new + (size_t)bg * p.n_new * p.dk);
            const u32x4* vs = reinterpret_cast<const u32x4*>(p.V_new + (size_t)bg * p.n_new * p.dv);
            u32x4* kd = reinterpret_cast<u32x4*>(p.K_cache + ((size_t)bg * p.L + c0) * p.dk);
            u32x4* vd = reinterpret_cast<u32x4*>(p.V_cache + ((size_t)bg * p.L + c0) * p.dv);
            for (int i = threadIdx.x; i < n * p.dk / 8; i += 256) kd[i] = ks[i];
            for (int i = threadIdx.x; i < n * p.dv / 8; i += 256) vd[i] = vs[i];
        }
        return;
    }
    if (p.N == 0) return;   // the capacity holds no compressed block
    const bool is_k = (int)blockIdx.y < nct_k;
    const int d = is_k ? p.dk : p.dv;
    const int col0 = 64 * (is_k ? blockIdx.y : blockIdx.y - nct_k);
    const u16* cache = is_k ? p.K_cache : p.V_cache;
    const u16* fresh = is_k ? p.K_new : p.V_new;
    const u16* Wt = is_k ? p.wt_k : p.wt_v;
    const float* bias = is_k ? p.bias_k : p.bias_v;
    u16* out = is_k ? p.K_cmp : p.V_cmp;
    const int KD = p.l * d;
    const int li = lane & 15, lq = lane >> 4;
    const int rowbase = (blockIdx.x * 4 + wave) * 16;

    // this lane's A row: pair (bg, candidate q) -> block lo + q of that group
    auto row_block = [&](int row, int& bg, int& c0, int& blk) {
        bg = row / p.R;
        if (bg >= BG) return false;
        c0 = old_len(p, bg / p.Hkv);
        int lo, hi;
        completed_blocks(p, c0, lo, hi);
        blk = lo + row % p.R;
        return blk <= hi;
    };
    int bg, c0, blk;
    const bool valid = row_block(rowbase + li, bg, c0, blk);
    if (!valid) {   // a row past the list: compute on token 0 of group 0, never stored
        bg = 0;
        c0 = p.L;
        blk = 0;
    }
    if (!__any(valid)) return;
    const u16* wb = Wt + (size_t)(col0 + li) * KD + lq * 8;
    // flattened block element kk + 8*lq: token kk / d of the block (32 | d), dim kk % d + 8*lq
    auto xa_at = [&](int kk) {
        const int tok = kk / d, e = kk - tok * d;
        const int pos = blk * p.s + tok;
        const u16* src = pos >= c0 ? fresh + ((size_t)bg * p.n_new + (pos - c0)) * d
                                   : cache + ((size_t)bg * p.L + pos) * d;
        return src + e + lq * 8;
    };
    // the prefill compression's order: four reduction ranges, each ascending, added in order
    f32x4 acc[4];
    for (int q = 0; q < 4; ++q) {
        int k_lo, k_hi;
        compress_k_range(KD, q, k_lo, k_hi);
        f32x4 part[4] = {zero4(), zero4(), zero4(), zero4()};
        compress_mfma_range_at(xa_at, wb, KD, k_lo, k_hi, part);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = q == 0 ? part[c] : acc[c] + part[c];
    }
    // C layout: lane owns column col0 + 16c + li and rows 4*lq + r of the wave's 16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int obg, oc0, oblk;
        if (!row_block(rowbase + 4 * lq + r, obg, oc0, oblk)) continue;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int o = col0 + 16 * c + li;
            out[((size_t)obg * p.N + oblk) * d + o] = f2bf(acc[c][r] + bias[o]);
        }
    }
}

__global__ void cache_advance_kernel(int32_t* cache_len, int B, int n_new, int L) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) cache_len[b] = min(min(max(cache_len[b], 0), L) + n_new, L);
}

int append_rows_per_group(int n_new, int s) { return (n_new + s - 1) / s + 1; }

void launch_cache_append(const AppendParams& p, hipStream_t st) {
    const int BG = p.B * p.Hkv;
    const int nct = p.dk / 64 + p.dv / 64;
    const int gx = (BG * p.R + 63) / 64;
    cache_append_kernel<<<dim3(gx, nct + 1), 256, 0, st>>>(p);
    cache_advance_kernel<<<(p.B + 255) / 256, 256, 0, st>>>(p.cache_len, p.B, p.n_new, p.L);
}

}  // namespace nsa
