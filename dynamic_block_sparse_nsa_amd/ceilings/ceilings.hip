// Measured ceilings of the MI355X units the NSA kernels are bound by, for the benchmark's
// roofline (a separate library, libnsa_ceilings.so; not part of the NSA ABI).
//
//   nsa_ceiling_mfma    bf16 MFMA 16x16x32 from registers: every wave keeps 8 independent
//                       accumulators and issues a long unrolled run of products (no memory
//                       traffic), so the achieved rate is the matrix cores' own ceiling.
//   nsa_ceiling_stream  a streaming read: every thread reads 16-byte pieces a grid apart, four
//                       in flight, and folds them into one value (one store per thread): the HBM
//                       read ceiling.
//   nsa_ceiling_gather  the selected branch's access pattern: contiguous blocks of
//                       `block_bytes` at listed offsets of a buffer, one wave per block piece
//                       of 1 KB, the rate of random block gathers (L2 / memory-side cache /
//                       HBM, depending on the buffer's size).
// Each call only launches (asynchronously, on the given stream); the caller times it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nsa_ceilings.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_kernel(float* out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(0.001f * (float)(lane + i));
        b[i] = static_cast<__bf16>(0.002f * (float)(lane - i));
    }
    f32x4 c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void stream_kernel(const u32x4* __restrict__ buf, size_t n16, uint32_t* out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 v0 = buf[i], v1 = buf[i + stride], v2 = buf[i + 2 * stride], v3 = buf[i + 3 * stride];
        acc ^= v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3];
        acc ^= v2[0] ^ v2[1] ^ v2[2] ^ v2[3] ^ v3[0] ^ v3[1] ^ v3[2] ^ v3[3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = buf[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// one 256-thread workgroup per listed block; each wave reads 1 KB pieces of it, all of the
// wave's pieces requested before any is used
__global__ __launch_bounds__(256) void gather_kernel(const unsigned char* __restrict__ buf, const int64_t* offsets,
                                                     int block_bytes, uint32_t* out) {
    const unsigned char* src = buf + offsets[blockIdx.x];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int pieces = block_bytes / 1024;
    uint32_t acc = 0;
    constexpr int U = 8;
    for (int p0 = wave * U; p0 < pieces; p0 += 4 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int pc = p0 + u < pieces ? p0 + u : pieces - 1;
            v[u] = *reinterpret_cast<const u32x4*>(src + (size_t)pc * 1024 + lane * 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

int nsa_ceiling_mfma(float* out, int n_wg, int iters, void* stream) {
    if (!out || n_wg <= 0 || iters <= 0) return 1;
    mfma_kernel<<<n_wg, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int nsa_ceiling_stream(const void* buf, size_t bytes, uint32_t* out, int n_wg, void* stream) {
    if (!buf || !out || n_wg <= 0 || (bytes & 15) != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0) return 1;
    stream_kernel<<<n_wg, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(buf), bytes / 16,
                                                                           out);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int nsa_ceiling_gather(const void* buf, const int64_t* offsets, int n_blocks, int block_bytes, uint32_t* out,
                       void* stream) {
    if (!buf || !offsets || !out || n_blocks <= 0 || block_bytes <= 0 || block_bytes % 1024 != 0) return 1;
    gather_kernel<<<n_blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        static_cast<const unsigned char*>(buf), offsets, block_bytes, out);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
