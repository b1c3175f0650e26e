/*
 * nsa_ceilings.h - microbenchmarks that measure the MI355X ceilings the NSA kernels are
 * bound by (libnsa_ceilings.so, separate from the NSA library).  Each call launches one
 * kernel on `stream` (a hipStream_t; NULL = default stream) and returns at once; the caller
 * times it (HIP events) and converts to a rate.  Every pointer is a device pointer owned by
 * the caller.  Returns 0, 1 for invalid arguments (nothing launched), 5 for a launch failure.
 */
#ifndef NSA_CEILINGS_H
#define NSA_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* n_wg workgroups of 4 waves, each wave issuing iters * 32 bf16 MFMA 16x16x32 products
 * (16384 flop each) from registers; out: n_wg * 256 floats (the results, so nothing is
 * optimized away).  Rate = n_wg * 4 * iters * 32 * 16384 flop / time. */
int nsa_ceiling_mfma(float* out, int n_wg, int iters, void* stream);

/* Reads `bytes` (a multiple of 16, 16-byte aligned) once with 16-byte loads
 * spread over n_wg workgroups of 256 threads; out: n_wg * 256 words. */
int nsa_ceiling_stream(const void* buf, size_t bytes, uint32_t* out, int n_wg, void* stream);

/* Reads n_blocks blocks of block_bytes (a multiple of 1024) at byte offsets[i] (int64,
 * 16-byte aligned, offsets[i] + block_bytes within the buffer) of buf, one workgroup per
 * block; out: n_blocks * 256 words. */
int nsa_ceiling_gather(const void* buf, const int64_t* offsets, int n_blocks, int block_bytes, uint32_t* out,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NSA_CEILINGS_H */
