// The prefill forward in one launch: compressed attention and block scores, the
// group-shared selection, selected-block and sliding-window attention and the gated sum,
// for one workgroup tile of tokens of one KV group (zjai.club notes, sections 5, 6, 8 and
// 10; sunshychen.top: compressed scores reused as selection scores).
//
// Each workgroup runs, for its TQ = 128 / G tokens:
//   1. cmp_attn_tile (cmp_attn.hpp): the compressed branch's LSE and o_cmp, and the block
//      scores of its rows;
//   2. the selection of those rows, one wave per row (select.hpp), from the score rows the
//      workgroup has just written (still in L2);
//   3. sparse_attn_tokens (sparse_attn.hpp) for the tokens four at a time: the selected
//      blocks gathered per token, the window range shared through LDS, and the gated sum
//      with the o_cmp rows written in step 1.
// The steps are the same code as the three-call path (nsa_score_select, then
// nsa_sparse_attn_fwd), so the results are identical bit for bit.  What the fusion changes
// is the schedule: the compressed branch is bound by the MFMA and LDS pipes and moves few
// bytes, the selected branch waits on gathers from the memory fabric; as separate launches
// each runs alone on the whole chip, while here the two workgroups sharing a CU are
// usually in different steps, so one's gathers are in flight under the other's products.
// Rows are handed out longest first (the compressed branch's cost grows with the position).
#include "cmp_attn.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"
#include "sparse_attn.hpp"

namespace nsa {

template <int DK, int DV, int G, int NU>
__global__ __launch_bounds__(256, 2) void prefill_fused_kernel(SelParams sp, AttnParams ap) {
    constexpr int NQ = G == 1 ? 1 : 2;
    constexpr int TQ = cmp_tile_tokens(G);
    static_assert(TQ % kTok == 0, "the tile must split into four-token groups");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int T = sp.T;
    const int n_tiles = (T + TQ - 1) / TQ;
    int unit, it;
    if (!xcd_map_tile(blockIdx.x, sp.B * sp.Hkv, n_tiles, unit, it)) return;
    // longest rows first, and neighbouring tiles at the same time: their window ranges and
    // local blocks overlap, so those keys are read from L2 (alternating long and short tiles
    // for more even phase mixing measured 29.2 against 23.3 ms at 64K tokens)
    const int tok0 = (n_tiles - 1 - it) * TQ;
    // 1. compressed branch and block scores
    cmp_attn_tile<DK, DV, G, NQ, true>(sp, unit, tok0, smem);
    __syncthreads();   // every score row of the tile is stored
    // 2. selection, one wave per token row
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = unit / sp.Hkv, g = unit % sp.Hkv;
    for (int r = wave; r < TQ; r += 4) {
        const int t = tok0 + r;
        if (t >= T) break;
        const size_t row = ((size_t)b * T + t) * sp.Hkv + g;
        select_blocks_wave<NU>(sp.scores + row * sp.n_slc, t / sp.lp, sp.top_n, sp.n_init, sp.n_local,
                               sp.sel + row * sp.top_n);
    }
    __syncthreads();   // every list and o_cmp row of the tile is stored
    // 3. selected + window branches and the gated sum, four tokens at a time
    for (int r0 = 0; r0 < TQ && tok0 + r0 < T; r0 += kTok)
        sparse_attn_tokens<DK, DV, 0>(ap, unit, tok0 + r0, reinterpret_cast<u16*>(smem));
}

namespace {

template <int DK, int DV, int G, int NU>
void prefill_g(const SelParams& sp, const AttnParams& ap, hipStream_t st) {
    constexpr int TQ = cmp_tile_tokens(G);
    const int n_tiles = (sp.T + TQ - 1) / TQ;
    const size_t lds = prefill_lds_bytes(DK, DV, G);
    const void* fn = reinterpret_cast<const void*>(prefill_fused_kernel<DK, DV, G, NU>);
    if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    prefill_fused_kernel<DK, DV, G, NU><<<xcd_grid(sp.B * sp.Hkv, n_tiles), 256, lds, st>>>(sp, ap);
}

// candidates per lane of the selection: n_slc <= 256, 1024 or 2048 blocks
constexpr int prefill_nu(int n_slc) { return n_slc <= 256 ? 4 : n_slc <= 1024 ? 16 : 32; }

template <int DK, int DV, int G>
void prefill_nu_switch(const SelParams& sp, const AttnParams& ap, hipStream_t st) {
    switch (prefill_nu(sp.n_slc)) {
        case 4: prefill_g<DK, DV, G, 4>(sp, ap, st); break;
        case 16: prefill_g<DK, DV, G, 16>(sp, ap, st); break;
        default: prefill_g<DK, DV, G, 32>(sp, ap, st); break;
    }
}

template <int DK, int DV>
bool prefill_dk(int G, const SelParams& sp, const AttnParams& ap, hipStream_t st) {
    switch (G) {
        case 1: prefill_nu_switch<DK, DV, 1>(sp, ap, st); break;
        case 2: prefill_nu_switch<DK, DV, 2>(sp, ap, st); break;
        case 4: prefill_nu_switch<DK, DV, 4>(sp, ap, st); break;
        case 8: prefill_nu_switch<DK, DV, 8>(sp, ap, st); break;
        case 16: prefill_nu_switch<DK, DV, 16>(sp, ap, st); break;
        default: return false;
    }
    return true;
}

}  // namespace

size_t prefill_lds_bytes(int DK, int DV, int G) {
    const size_t a = cmp_attn_lds_bytes(DK, DV, G, true);
    const size_t b = (size_t)sparse_lds_elems(DK, DV) * 2;
    return a > b ? a : b;
}

bool launch_prefill_fused(int DK, int DV, int G, const SelParams& sp, const AttnParams& ap, hipStream_t st) {
    if (DK == 192 && DV == 128) return prefill_dk<192, 128>(G, sp, ap, st);
    if (DK == 128 && DV == 128) return prefill_dk<128, 128>(G, sp, ap, st);
    if (DK == 64 && DV == 64) return prefill_dk<64, 64>(G, sp, ap, st);
    return false;
}

}  // namespace nsa
