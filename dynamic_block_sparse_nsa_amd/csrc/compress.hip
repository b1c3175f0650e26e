// Block compression (zjai.club notes, section 5: one key and one value per contiguous
// block; MoBA mean pooling, section 16) and the layout transforms used by the
// attention kernels.
//
// Linear phi:  cmp[i, :] = vec(X[i*s : i*s+l, :]) . W + bias,  bias = vec(PE) . W.
// Row i of the GEMM operand is the l*d contiguous bf16 values starting at token i*s, so
// the overlapping blocks are read straight from X with a row stride of s*d; W is
// transposed once into the workspace so that both MFMA operands are 16-byte row loads.
#include "common.hpp"
#include "launch.hpp"

namespace nsa {


// ---------------------------------------------------------------------------
// W [KD, dout] -> Wt [dout, KD]  (bf16, 64x64 tiles through LDS)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_w_kernel(const u16* __restrict__ W, u16* __restrict__ Wt,
                                                          int KD, int dout) {
    __shared__ u16 tile[64][65];
    const int k0 = blockIdx.x * 64, o0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) {
        const int k = k0 + r, o = o0 + tx;
        tile[r][tx] = (k < KD && o < dout) ? W[(size_t)k * dout + o] : (u16)0;
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int o = o0 + r, k = k0 + tx;
        if (o < dout && k < KD) Wt[(size_t)o * KD + k] = tile[tx][r];
    }
}

// bias[o] = sum_k pe_flat[k] * W[k][o], fp32, fixed-order tree reduction.
__global__ __launch_bounds__(256) void pe_bias_kernel(const u16* __restrict__ pe, const u16* __restrict__ Wt,
                                                      float* __restrict__ bias, int KD) {
    __shared__ float red[256];
    const int o = blockIdx.x;
    float acc = 0.f;
    for (int k = threadIdx.x; k < KD; k += 256) acc += bf2f(pe[k]) * bf2f(Wt[(size_t)o * KD + k]);
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) bias[o] = red[0];
}

// ---------------------------------------------------------------------------
// Linear phi.  Grid (ceil(N/(16 RT)), dout/64, B*Hkv): a workgroup owns 16 RT output rows x
// 64 output columns, and its 4 waves split the reduction (KD = l*d) into four 32-aligned
// ranges (compress_k_range).  Each step of 32 k loads RT row fragments of X and the four
// column fragments of W^T and runs RT x 4 products, so a W^T fragment read from L2 feeds RT
// row tiles (the reads of W^T, 786 KB per 64 columns of a 192-wide head, were most of the
// kernel's traffic with one row tile).  Every output still sums its products in ascending
// k within a wave's range and the four partials in wave order, then the bias: the decode
// cache append reproduces exactly this order.  X: [BG][T][d]; out: [BG][N][dout].
// ---------------------------------------------------------------------------
template <int RT>
__global__ __launch_bounds__(256) void compress_linear_kernel(const u16* __restrict__ X,
                                                              const u16* __restrict__ Wt,
                                                              const float* __restrict__ bias,
                                                              u16* __restrict__ out, int T, int d, int dout,
                                                              int l, int s, int N) {
    constexpr int U = 8 / RT;   // steps whose loads are issued together
    __shared__ f32x4 part[3][RT][4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bg = blockIdx.z;
    const int KD = l * d;
    const int row0 = blockIdx.x * 16 * RT;
    const int col0 = blockIdx.y * 64;
    const int li = lane & 15, lq = lane >> 4;
    const u16* xa[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int my_row = min(row0 + 16 * rt + li, N - 1);  // clamp: rows past N are computed but not stored
        xa[rt] = X + (size_t)bg * T * d + (size_t)my_row * s * d + lq * 8;
    }
    const u16* wb = Wt + (size_t)(col0 + li) * KD + lq * 8;
    int k_lo, k_hi;
    compress_k_range(KD, wave, k_lo, k_hi);
    f32x4 acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[rt][c] = zero4();
    int kk = k_lo;
    for (; kk + 32 * U <= k_hi; kk += 32 * U) {
        bf16x8 a[U][RT], bw[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) a[u][rt] = ld8(xa[rt] + kk + 32 * u);
#pragma unroll
            for (int c = 0; c < 4; ++c) bw[u][c] = ld8(wb + (size_t)c * 16 * KD + kk + 32 * u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[rt][c] = mfma16(a[u][rt], bw[u][c], acc[rt][c]);
    }
    for (; kk < k_hi; kk += 32) {
        bf16x8 a[RT], bw[4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) a[rt] = ld8(xa[rt] + kk);
#pragma unroll
        for (int c = 0; c < 4; ++c) bw[c] = ld8(wb + (size_t)c * 16 * KD + kk);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[rt][c] = mfma16(a[rt], bw[c], acc[rt][c]);
    }
    if (wave > 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int c = 0; c < 4; ++c) part[wave - 1][rt][c][lane] = acc[rt][c];
    }
    __syncthreads();
    if (wave > 0) return;
    // C layout: lane owns column col0 + 16c + li and rows row0 + 16rt + 4*lq + r.
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const f32x4 v = ((acc[rt][c] + part[0][rt][c][lane]) + part[1][rt][c][lane]) + part[2][rt][c][lane];
            const int o = col0 + 16 * c + li;
            const float bo = bias[o];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = row0 + 16 * rt + 4 * lq + r;
                if (i < N) out[((size_t)bg * N + i) * dout + o] = f2bf(v[r] + bo);
            }
        }
}

// Mean pooling: out[bg][i][e] = (1/l) sum_{r<l} X[bg][i*s + r][e]; grid (N, BG), 256 threads.
// Thread (rg, c) adds the 8 dims 8c..8c+7 of rows rg, rg + RG, ... of the block with 16-byte
// loads (RG = 256 / (D/8) rows in flight per step, a streaming read of the block); the RG
// partial sums of each dim are then added in LDS.  fp32 sums, one bf16 rounding.
template <int D>
__global__ __launch_bounds__(256) void compress_mean_kernel(const u16* __restrict__ X, u16* __restrict__ out, int T,
                                                            int l, int s, int N) {
    constexpr int CPR = D / 8, RG = 256 / CPR;
    __shared__ float part[RG][D + 4];
    const int i = blockIdx.x, bg = blockIdx.y;
    const int c = threadIdx.x % CPR, rg = threadIdx.x / CPR;
    float acc[8] = {};
    if (rg < RG) {
        const u16* x = X + ((size_t)bg * T + (size_t)i * s) * D + 8 * c;
#pragma unroll 4
        for (int r = rg; r < l; r += RG) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(x + (size_t)r * D);
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] += bf2f((u16)(v[k >> 1] >> (16 * (k & 1))));
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) part[rg][8 * c + k] = acc[k];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < D; e += 256) {
        float sum = 0.f;
        for (int q = 0; q < RG; ++q) sum += part[q][e];
        out[((size_t)bg * N + i) * D + e] = f2bf(sum / (float)l);
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
void launch_transpose_w(const u16* W, u16* Wt, int KD, int dout, hipStream_t st) {
    dim3 grid((KD + 63) / 64, (dout + 63) / 64);
    transpose_w_kernel<<<grid, 256, 0, st>>>(W, Wt, KD, dout);
}

void launch_pe_bias(const u16* pe, const u16* Wt, float* bias, int KD, int dout, hipStream_t st) {
    pe_bias_kernel<<<dout, 256, 0, st>>>(pe, Wt, bias, KD);
}

void launch_compress_linear(const u16* X, const u16* Wt, const float* bias, u16* out, int BG, int T, int d,
                            int dout, int l, int s, int N, hipStream_t st) {
    // the most row tiles per workgroup (1, 2 or 4) that still give every CU a workgroup; the
    // results do not depend on the choice (nsa_compress with 1 / 4 row tiles: 64K workload
    // 0.53 / 0.27 ms, at 32K 0.31 / 0.20 ms, at 8K 0.146 / 0.156 ms)
    auto n_wg = [&](int rt) { return (size_t)((N + 16 * rt - 1) / (16 * rt)) * (dout / 64) * BG; };
    const int rt = n_wg(4) >= 256 ? 4 : n_wg(2) >= 256 ? 2 : 1;
    dim3 grid((N + 16 * rt - 1) / (16 * rt), dout / 64, BG);
    if (rt == 4) compress_linear_kernel<4><<<grid, 256, 0, st>>>(X, Wt, bias, out, T, d, dout, l, s, N);
    else if (rt == 2) compress_linear_kernel<2><<<grid, 256, 0, st>>>(X, Wt, bias, out, T, d, dout, l, s, N);
    else compress_linear_kernel<1><<<grid, 256, 0, st>>>(X, Wt, bias, out, T, d, dout, l, s, N);
}

void launch_compress_mean(const u16* X, u16* out, int BG, int T, int d, int l, int s, int N, hipStream_t st) {
    dim3 grid(N, BG);
    if (d == 192) compress_mean_kernel<192><<<grid, 256, 0, st>>>(X, out, T, l, s, N);
    else if (d == 128) compress_mean_kernel<128><<<grid, 256, 0, st>>>(X, out, T, l, s, N);
    else compress_mean_kernel<64><<<grid, 256, 0, st>>>(X, out, T, l, s, N);
}

}  // namespace nsa
