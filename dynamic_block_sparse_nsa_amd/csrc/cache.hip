// Decode cache maintenance (zjai.club notes, section 5: the compressed cache grows by one
// entry every s tokens; section 13: decoding runs against these caches).  Appending n_new
// tokens to a sequence writes them into the raw caches and computes every compressed block
// whose last token is among them, with exactly the arithmetic of the prefill compression
// (compress_linear_kernel: the same four reduction ranges, each in the same MFMA order, added
// in the same order, the same fp32 bias vec(PE).W, one bf16 rounding), so an appended entry
// equals the prefill's bit for bit.
//
// cache_append_kernel, grid (max(ceil(BG * R / 16), copy workgroups), n_ct + 1): rows are (sequence-group, candidate
// block) pairs, R = ceil(n_new / s) candidates per group (the most blocks one append can
// complete); a workgroup computes 16 rows x 64 output columns, its 4 waves taking the four
// reduction ranges of the prefill compression and the partials added in the same order, so
// W streams once per 16 groups.  Column tiles 0 .. dk/64-1 produce K entries, the next dv/64
// tiles V entries.  Block tokens at or past the old length are read from the new-token
// arrays, so the copy (the last grid row, one 16-byte piece per thread) and the compression
// need no ordering.  cache_advance_kernel then moves every cache_len past the new tokens.
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

// the new tokens into the raw caches: one 16-byte piece per thread
__device__ __forceinline__ void copy_tokens(const AppendParams& p) {
    const int kp = p.dk / 8, per_tok = kp + p.dv / 8;   // 16-byte pieces per token row
    const long long total = (long long)p.B * p.Hkv * p.n_new * per_tok;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int piece = (int)(idx % per_tok);
    const long long rest = idx / per_tok;
    const int tok = (int)(rest % p.n_new), bg = (int)(rest / p.n_new);
    const int pos = old_len(p, bg / p.Hkv) + tok;
    if (pos >= p.L) return;   // past the capacity: dropped
    if (piece < kp) {
        reinterpret_cast<u32x4*>(p.K_cache + ((size_t)bg * p.L + pos) * p.dk)[piece] =
            reinterpret_cast<const u32x4*>(p.K_new + ((size_t)bg * p.n_new + tok) * p.dk)[piece];
    } else {
        reinterpret_cast<u32x4*>(p.V_cache + ((size_t)bg * p.L + pos) * p.dv)[piece - kp] =
            reinterpret_cast<const u32x4*>(p.V_new + ((size_t)bg * p.n_new + tok) * p.dv)[piece - kp];
    }
}

__global__ __launch_bounds__(256) void cache_append_kernel(AppendParams p) {
    __shared__ f32x4 part[3][4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int BG = p.B * p.Hkv;
    const int nct_k = p.dk / 64, nct = nct_k + p.dv / 64;
    if ((int)blockIdx.y == nct) {   // the last grid row copies the new tokens
        copy_tokens(p);
        return;
    }
    if (p.N == 0 || (int)blockIdx.x * 16 >= BG * p.R) return;   // no block / past the rows
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
    const int rowbase = blockIdx.x * 16;

    // row -> (group bg, its old length c0, block blk); false when the row has no block
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
    // the rows depend on blockIdx.x only, so every wave of the workgroup leaves together
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
    // the prefill compression's order: wave w takes reduction range w (ascending), the
    // partials are added in range order
    int k_lo, k_hi;
    compress_k_range(KD, wave, k_lo, k_hi);
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
    compress_mfma_range_at(xa_at, wb, KD, k_lo, k_hi, acc);
    if (wave > 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) part[wave - 1][c][lane] = acc[c];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = ((acc[c] + part[0][c][lane]) + part[1][c][lane]) + part[2][c][lane];
    // C layout: lane owns column col0 + 16c + li and rows 4*lq + r of the 16
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

// at most ceil(n_new / s) blocks end among n_new consecutive tokens
int append_rows_per_group(int n_new, int s) { return (n_new + s - 1) / s; }

void launch_cache_append(const AppendParams& p, hipStream_t st) {
    const int BG = p.B * p.Hkv;
    const int nct = p.dk / 64 + p.dv / 64;
    const int gx = (BG * p.R + 15) / 16;
    const long long pieces = (long long)BG * p.n_new * (p.dk + p.dv) / 8;
    const int gc = (int)((pieces + 255) / 256);
    cache_append_kernel<<<dim3(gx > gc ? gx : gc, nct + 1), 256, 0, st>>>(p);
    cache_advance_kernel<<<(p.B + 255) / 256, 256, 0, st>>>(p.cache_len, p.B, p.n_new, p.L);
}

}  // namespace nsa
