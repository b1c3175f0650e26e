// Internal device helpers shared by the gfx950 kernels of the NSA library.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (wave64, checked on gfx950):
//   A[16][32]: lane l holds row l%16, k = 8*(l/16) .. 8*(l/16)+7 (one 16-byte vector)
//   B[32][16]: lane l holds column l%16, k = 8*(l/16) .. +7
//   C[16][16]: lane l holds column l%16, rows 4*(l/16) .. 4*(l/16)+3
// Attention products are written key-major (S^T = K . Q^T) so that a lane owns one query
// row (column) and several keys (rows): the softmax row statistics are then mostly
// in-lane, and P^T comes out of the C layout already in the B-operand layout that the
// value product O^T = V^T . P^T needs.  For that the value rows are stored transposed
// (d-major) with each 32-key group permuted so that lane group q (= l/16) finds its
// keys {4q..4q+3, 16+4q..16+4q+3} as 8 contiguous values (see vt_pos).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;
// 16 bytes as a native vector (the HIP uint4 wrapper struct can defeat register promotion)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp16 variant (P in fp16, 2^-11 relative rounding, against fp16 values)
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
// LDS address space, for the destination of the global -> LDS copies
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ f32x4 mfma16h(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 16-byte global/LDS load of 8 bf16 values (address must be 16-byte aligned).
__device__ __forceinline__ bf16x8 ld8(const u16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, uint4{0u, 0u, 0u, 0u}); }

__device__ __forceinline__ u16 f2bf(float x) { return __builtin_bit_cast(u16, static_cast<__bf16>(x)); }

__device__ __forceinline__ float bf2f(u16 x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

// P^T operand from two 16-key C tiles: slots 0..3 from tile a, 4..7 from tile b.
__device__ __forceinline__ bf16x8 pack_p(const f32x4& a, const f32x4& b) {
    bf16x8 r;
    r[0] = static_cast<__bf16>(a[0]); r[1] = static_cast<__bf16>(a[1]);
    r[2] = static_cast<__bf16>(a[2]); r[3] = static_cast<__bf16>(a[3]);
    r[4] = static_cast<__bf16>(b[0]); r[5] = static_cast<__bf16>(b[1]);
    r[6] = static_cast<__bf16>(b[2]); r[7] = static_cast<__bf16>(b[3]);
    return r;
}

// P^T operand in fp16 (round to nearest even), same slot order as pack_p.
__device__ __forceinline__ f16x8 pack_p_h(const f32x4& a, const f32x4& b) {
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = static_cast<_Float16>(a[i]);
        r[4 + i] = static_cast<_Float16>(b[i]);
    }
    return r;
}

__device__ __forceinline__ f16x8 ld8h(const u16* p) {
    return __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(p));
}

// Split P^T into bf16 high and low parts (p ~= hi + lo to about 2^-17 relative), so that
// V^T.P^T = V^T.hi + V^T.lo keeps the probabilities' fp32 precision on the bf16 MFMA.
__device__ __forceinline__ void pack_p_split(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const __bf16 ha = static_cast<__bf16>(a[r]), hb = static_cast<__bf16>(b[r]);
        hi[r] = ha;
        hi[4 + r] = hb;
        lo[r] = static_cast<__bf16>(a[r] - static_cast<float>(ha));
        lo[4 + r] = static_cast<__bf16>(b[r] - static_cast<float>(hb));
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Position of key k (0..31) inside its permuted 32-key group of a transposed value row.
__host__ __device__ __forceinline__ int vt_pos(int k) {
    return (k < 16) ? (8 * (k >> 2) + (k & 3)) : (8 * ((k - 16) >> 2) + 4 + (k & 3));
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Exchanges across 16-lane rows without the LDS crossbar: gfx950's v_permlane16_swap
// (v_permlane32_swap) swaps the odd rows (upper half) of one register with the even rows
// (lower half) of another.  Swapping a value with itself leaves, in each lane, v[i] in one
// result and v[i ^ 16] (v[i ^ 32]) in the other, so a commutative op of the two results
// combines lane i with its partner.  All 64 lanes must be active.
__device__ __forceinline__ u32x2 swap16(uint32_t v) { return __builtin_amdgcn_permlane16_swap(v, v, false, false); }
__device__ __forceinline__ u32x2 swap32(uint32_t v) { return __builtin_amdgcn_permlane32_swap(v, v, false, false); }

// IEEE maximum of two floats.  fmaxf first quiets each operand that is not known to be
// canonical (one extra instruction per MFMA result); this form needs none, and chains of it
// become gfx950's three-input v_maximum3_f32.  NaN propagates and -0 < +0, which no softmax
// reference here depends on.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Max / sum over the four lanes that share a query column (lanes l, l^16, l^32, l^48);
// every lane ends with the result.
__device__ __forceinline__ float col_max(float v) {
    u32x2 r = swap16(__float_as_uint(v));
    v = vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = swap32(__float_as_uint(v));
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float col_sum(float v) {
    u32x2 r = swap16(__float_as_uint(v));
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = swap32(__float_as_uint(v));
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// DPP lane moves within a 16-lane row (VALU, no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within each 16 lanes

// Sum over aligned groups of N lanes (N = 1, 2, 4, 8 or 16) inside a 16-lane row; every
// lane of a group ends with the group total.
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
    if constexpr (N >= 2) v += dpp_mov<kDppQuadXor1>(v);
    if constexpr (N >= 4) v += dpp_mov<kDppQuadXor2>(v);
    if constexpr (N >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_mov<kDppRowMirror>(v);
    return v;
}

// Query-row layout of a wave holding NQ MFMA column tiles (16 columns each) of the
// query rows of one KV group: tile c, column li holds (token, head).  The G heads of a
// token sit in CL = min(G, NQ) tiles of the same lane and GL = G / CL neighbouring lanes,
// so a sum over the group's heads is CL-1 in-lane adds plus log2(GL) DPP adds.
template <int G, int NQ>
struct QMap {
    static constexpr int CL = G < NQ ? G : NQ;
    static constexpr int GL = G / CL;
    static constexpr int TPW = 16 * NQ / G;  // tokens per wave
    __device__ static int token(int c, int li) { return (li / GL) * (NQ / CL) + c / CL; }
    __device__ static int head(int c, int li) { return CL * (li % GL) + c % CL; }
};

// The linear block map's reduction (KD = l*d elements) split into four 32-aligned ranges,
// one per wave; range w is [k_lo, k_hi).
__device__ __forceinline__ void compress_k_range(int KD, int w, int& k_lo, int& k_hi) {
    const int steps = KD / 32;
    k_lo = 32 * (steps * w / 4);
    k_hi = 32 * (steps * (w + 1) / 4);
}

// acc[c] += A . B over k in [k_lo, k_hi) (ascending, 32 per MFMA) for the 16-row A operand
// whose element kk (this lane's row) is at xa_at(kk) and the four 16-column B tiles at
// wb + c*16*KD; loads are issued 8 steps ahead of their products.  The cache append uses
// it; compress_linear_kernel runs the same per-output order over several row tiles.
template <typename XAt>
__device__ __forceinline__ void compress_mfma_range_at(XAt xa_at, const u16* wb, int KD, int k_lo, int k_hi,
                                                       f32x4 (&acc)[4]) {
    constexpr int U = 8;
    int kk = k_lo;
    for (; kk + 32 * U <= k_hi; kk += 32 * U) {
        bf16x8 a[U], bw[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            a[u] = ld8(xa_at(kk + 32 * u));
#pragma unroll
            for (int c = 0; c < 4; ++c) bw[u][c] = ld8(wb + (size_t)c * 16 * KD + kk + 32 * u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = mfma16(a[u], bw[u][c], acc[c]);
    }
    for (; kk < k_hi; kk += 32) {
        const bf16x8 a = ld8(xa_at(kk));
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = mfma16(a, ld8(wb + (size_t)c * 16 * KD + kk), acc[c]);
    }
}

// Workgroup barrier that orders LDS accesses only: this wave's LDS operations complete,
// then s_barrier.  Unlike __syncthreads it does not wait for outstanding global loads or
// stores, so prefetched tiles stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Offset (in elements) of the 8 contraction elements a lane of row-group lq holds for
// MFMA step ds when a row of the operand is read straight from memory.  The contraction
// is order-free, so steps 2p and 2p+1 take a lane's two adjacent 16-byte pieces of the
// 64-element span p: every lane reads 32 contiguous bytes and four lanes a full 128-byte
// line.  Both operands of a product must use the same mapping (d must be a multiple of 64).
__device__ __forceinline__ int kpair_off(int ds, int lq) { return 64 * (ds >> 1) + 16 * lq + 8 * (ds & 1); }

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Inside each 16-lane row, lane c
// names 4 consecutive 16-bit values; lane j receives, as its element r, value j % 4 of
// the 4 values named by lane 4r + j / 4 of the same row.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ s16x4 lds_read_tr16(const u16* p) {
    typedef __attribute__((address_space(3))) s16x4* lds_ptr;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p));
}

// V^T operand of O^T += V^T.P^T from a row-major value tile in LDS (row = key, STR
// elements per row, 8-byte aligned rows): lane (li, lq) receives V[key0 + k][d0 + li] for
// k = 4lq..4lq+3 and 16+4lq..16+4lq+3, the key order of pack_p / pack_p_split.
__device__ __forceinline__ bf16x8 ld_vt_tr(const u16* tile, int STR, int key0, int d0) {
    const int lane = threadIdx.x & 63, c = lane & 15, lq = (lane >> 4) & 3;
    const u16* a = tile + (key0 + 4 * lq + (c >> 2)) * STR + d0 + 4 * (c & 3);
    const s16x4 x = lds_read_tr16(a);
    const s16x4 y = lds_read_tr16(a + 16 * STR);
    const s16x8 v = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Workgroup -> (unit, tile) for a 1-D grid over units (unit = b * Hkv + g, one KV group of
// one sequence) and n_tiles tiles per unit.  Workgroups are dispatched to the 8 XCDs
// round-robin (workgroup L runs on XCD L % 8).  When the units split evenly over the
// XCDs, every XCD serves one unit (or a fixed set), so the unit's keys and values stay in
// that XCD's L2; otherwise units are interleaved tile by tile.
__device__ __forceinline__ bool xcd_map_tile(int L, int U, int n_tiles, int& u, int& it) {
    const int xcd = L & 7, r = L >> 3;
    if (8 % U == 0) {
        const int xpu = 8 / U;   // XCDs per unit, tiles interleaved between them
        u = xcd / xpu;
        it = r * xpu + xcd % xpu;
    } else if (U % 8 == 0) {
        u = xcd + 8 * (r / n_tiles);
        it = r % n_tiles;
    } else {
        u = L % U;
        it = L / U;
    }
    return u < U && it < n_tiles;
}

// Grid size that xcd_map_tile covers.
inline int xcd_grid(int U, int n_tiles) {
    if (8 % U == 0) return 8 * ((n_tiles + 8 / U - 1) / (8 / U));
    return U * n_tiles;
}

// Loads and stores of data touched once (streaming: not worth keeping in the caches).
template <typename V>
__device__ __forceinline__ V ld_stream(const V* p) { return __builtin_nontemporal_load(p); }
template <typename V>
__device__ __forceinline__ void st_stream(V v, V* p) { __builtin_nontemporal_store(v, p); }

}  // namespace nsa
