// Selected-block attention, sliding window and gated sum (zjai.club notes, sections 5-6
// and 10; sunshychen.top): the standalone kernel over 4-token workgroups.  The body,
// sparse_attn_tokens, and its design notes are in sparse_attn.hpp (shared with the fused
// prefill kernel).
#include "common.hpp"
#include "launch.hpp"
#include "sparse_attn.hpp"

namespace nsa {

template <int DK, int DV, int MODE = 0>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) u16 lds[sparse_lds_elems(DK, DV)];
    int unit, it;
    if (!xcd_map_tile(blockIdx.x, p.B * p.Hkv, (p.T + kTok - 1) / kTok, unit, it)) return;
    sparse_attn_tokens<DK, DV, MODE>(p, unit, it * kTok, lds);
}

bool launch_sparse_attn_stats(int DK, int DV, const AttnParams& p, hipStream_t st) {
    const int grid = xcd_grid(p.B * p.Hkv, (p.T + kTok - 1) / kTok);
    if (DK == 192 && DV == 128) sparse_attn_kernel<192, 128, 1><<<grid, 256, 0, st>>>(p);
    else if (DK == 128 && DV == 128) sparse_attn_kernel<128, 128, 1><<<grid, 256, 0, st>>>(p);
    else if (DK == 64 && DV == 64) sparse_attn_kernel<64, 64, 1><<<grid, 256, 0, st>>>(p);
    else return false;
    return true;
}

bool launch_sparse_attn(int DK, int DV, const AttnParams& p, int B, hipStream_t st) {
    (void)B;
    const int grid = xcd_grid(p.B * p.Hkv, (p.T + kTok - 1) / kTok);
    if (p.saved_o) {
        if (DK == 192 && DV == 128) sparse_attn_kernel<192, 128, 2><<<grid, 256, 0, st>>>(p);
        else if (DK == 128 && DV == 128) sparse_attn_kernel<128, 128, 2><<<grid, 256, 0, st>>>(p);
        else if (DK == 64 && DV == 64) sparse_attn_kernel<64, 64, 2><<<grid, 256, 0, st>>>(p);
        else return false;
        return true;
    }
    if (DK == 192 && DV == 128) sparse_attn_kernel<192, 128><<<grid, 256, 0, st>>>(p);
    else if (DK == 128 && DV == 128) sparse_attn_kernel<128, 128><<<grid, 256, 0, st>>>(p);
    else if (DK == 64 && DV == 64) sparse_attn_kernel<64, 64><<<grid, 256, 0, st>>>(p);
    else return false;
    return true;
}

}  // namespace nsa
