// Internal host-side entry points of the kernels (called by the C ABI in api.cpp).
// Every launcher assumes the arguments were validated by the API layer; launchers that
// return bool report whether the shape has a compiled kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nsa {

typedef uint16_t u16;

constexpr float kLog2eHost = 1.4426950408889634f;

// ---- compression and layout ----
void launch_transpose_w(const u16* W, u16* Wt, int KD, int dout, hipStream_t st);
void launch_pe_bias(const u16* pe, const u16* Wt, float* bias, int KD, int dout, hipStream_t st);
void launch_compress_linear(const u16* X, const u16* Wt, const float* bias, u16* out, int BG, int T, int d,
                            int dout, int l, int s, int N, hipStream_t st);
void launch_compress_mean(const u16* X, u16* out, int BG, int T, int d, int l, int s, int N, hipStream_t st);

// ---- compressed attention + selection ----
struct SelParams {
    const u16* Q;          // [B,T,H,DK]
    const u16* Kc;         // [B,Hkv,N,DK] (mode 1)
    const u16* Kf;         // compressed keys in fragment order, Npad keys per unit (mode 0)
    const u16* Vf;         // compressed values in fragment order, fp16 scaled by 2^-vexp (mode 0 with o_cmp)
    const int* vexp;       // [B*Hkv] scaling exponent of Vf
    float* lse;            // [B,T,H] natural-log LSE of the compressed branch, or null
    float* o_cmp;          // [B,T,H,DV] or null
    float* scores;         // [B,T,Hkv,n_slc] block scores (workspace)
    int32_t* sel;          // [B,T,Hkv,top_n] selection (written by the fused mean-score selection)
    int top_n, n_init, n_local;
    int B, T, Hkv, N, Npad, l, s, lp, n_slc;
    float scale_log2;
};
int cmp_vmax_parts();
bool launch_tile_cmp(int DK, int DV, const u16* K, const u16* V, uint32_t* vmax_part, int* vexp, u16* Kf, u16* Vf,
                     int BG, int N, int Npad, hipStream_t st);
bool launch_cmp_attn(bool with_o, int DK, int DV, int G, const SelParams& p, hipStream_t st);
size_t cmp_attn_lds_bytes(int DK, int DV, int G, bool with_o);
bool launch_mean_scores(int DK, int G, const SelParams& p, hipStream_t st);
// Mean-key scores with the selection fused (no scores workspace): G = 1 and at most
// kFusedMaxPicks blocks picked besides the forced ones (top_n - n_local).
constexpr int kFusedMaxPicks = 4;
bool launch_mean_select(int DK, const SelParams& p, hipStream_t st);
void launch_select_from_scores(const float* scores, int32_t* sel, int B, int T, int Hkv, int n_slc, int lp,
                               int top_n, int n_init, int n_local, hipStream_t st);

// ---- selected + window attention, gated sum ----
// K and V in MFMA fragment order (written by launch_tile_cmp; V as scaled fp16): for every 16-key group kt
// and contraction step ds, the 64 lanes' K operands are 1 KB contiguous
// (Kf[bg][kt][ds][lane][8]); for every 32-key chunk c and 16-wide value slice dt, the
// lanes' V^T operands likewise (Vf[bg][c][dt][lane][8]).  Keys >= T are zero.
struct AttnParams {
    const u16* Q;        // [B,T,H,DK]
    const u16* Kf;       // [B,Hkv,Tpad/16,DK/32,64,8]
    const u16* Vf;       // [B,Hkv,Tpad/32,DV/16,64,8] fp16, V * 2^-vexp[b*Hkv+g] (launch_tile_cmp)
    const int* vexp;     // [B*Hkv]
    const int32_t* sel;  // [B,T,Hkv,top_n]
    const float* o_cmp;  // [B,T,H,DV] (branch CMP)
    const float* gates;  // [B,T,H,3] or null
    u16* O;              // [B,T,H,DV]
    // backward statistics mode (launch_sparse_attn_stats): instead of O, per (token, head)
    // and branch c (cmp, slc, win) the base-2 LSE, D_c = sigma_c <dO, o_c> and sigma_c
    const float* lse_cmp;  // [B,T,H] natural-log LSE of the compressed branch
    const u16* dO;         // [B,T,H,DV]
    float* stats;          // [B,T,H,3,4]: lse2, D, sigma, 0
    float* dgates;         // [B,T,H,3] or null
    // training forward (forward mode, both non-null): the selected and window branches'
    // base-2 LSE and normalized outputs, saved for the backward
    float* saved_lse;      // [B,T,H,2]
    float* saved_o;        // [B,T,H,2,DV]
    int B, T, Tpad, Hkv, G, lp, top_n, window, branches;
    float scale_log2;
};
bool launch_sparse_attn(int DK, int DV, const AttnParams& p, int B, hipStream_t st);
bool launch_sparse_attn_stats(int DK, int DV, const AttnParams& p, hipStream_t st);
// the backward statistics from a training forward's saved LSE and outputs (no recompute)
void launch_stats_from_saved(int DV, const AttnParams& p, hipStream_t st);

// ---- the fused prefill (prefill.hip): cmp_attn_tile, selection, sparse_attn_tokens per tile ----
// sp as for launch_cmp_attn (with o_cmp, scores, sel, top_n, n_init, n_local set), ap as for
// launch_sparse_attn (ap.sel = sp.sel, ap.o_cmp = sp.o_cmp: both read back after being written)
size_t prefill_lds_bytes(int DK, int DV, int G);
bool launch_prefill_fused(int DK, int DV, int G, const SelParams& sp, const AttnParams& ap, hipStream_t st);

// ---- G = 1 selected-only attention (MoBA): inverted, block-major schedule ----
constexpr int kMobaChunk = 1024;   // tokens per histogram / scatter workgroup
struct MobaParams {
    const u16* Q;              // [B,T,H,DK] (H = Hkv)
    const u16* K;              // [B,Hkv,T,DK] row-major (tiles gathered into fragment order)
    const u16* Vf;             // fragment-order V, fp16 scaled by 2^-vexp (launch_tile_cmp)
    const int* vexp;           // [B*Hkv]
    const int32_t* sel;        // [B,T,Hkv,top_n]
    const float* gates;        // [B,T,H,3] or null (slot 1 is used)
    u16* O;                    // [B,T,H,DV]
    // workspace
    int* hist;                 // [B*Hkv, n_chunk, n_slc] counts, then prefix over chunks
    int* bucket_cnt;           // [n_bucket]
    int* bucket_start;         // [n_bucket + 1]
    int* tile_start;           // [n_bucket + 1]
    int* tile_bucket;          // [moba_max_tiles] the bucket of every 128-entry list tile
    int* entries;              // [B*Hkv*T*top_n] (token << 5 | slot), grouped by bucket
    float* part_m;             // [B,T,Hkv,top_n]
    float* part_l;             // [B,T,Hkv,top_n]
    u16* part_o;               // [B,T,Hkv,top_n,DV] fp16, normalized by the slot's own sum
    int B, T, Tpad, Hkv, lp, n_slc, top_n, n_chunk, n_bucket, n_own;
    int keep_own;              // 1: the query's own block is listed too (backward lists)
    float scale_log2;
};
// the bucket lists alone (hist, prefix, scan, tiles, scatter); uses sel, T, Hkv, lp, n_slc,
// top_n, n_chunk, n_bucket, keep_own and the list buffers
void launch_block_lists(const MobaParams& p, hipStream_t st);
int moba_n_chunk(int T);
int moba_n_own(int BH, int n_slc, int lp);
int moba_max_tiles(int BH, int T, int top_n, int n_slc);
bool launch_moba_attn(int DK, int DV, const MobaParams& p, hipStream_t st);

// ---- backward ----
constexpr int kBwdTile = 128;   // query tokens per dK/dV work item (= the block lists' tile)
constexpr int kBwdCmpTile = 512;   // query tokens per compressed-branch dK/dV work item
constexpr int kDkvWavesDense = 8;  // compressed / window items: 8 waves x 1 key tile = 128 keys
constexpr int kDkvTilesDense = 1;  // (4 waves x 2 tiles halves the LDS reads per key but runs
                                   // one wave per SIMD: 34 ms against 24.5 ms at 64K)
constexpr int kDkvWavesSlc = 4;    // selected items: 64 keys per workgroup
struct BwdParams {
    const u16* Q;              // [B,T,H,DK]
    const u16* K;              // [B,Hkv,T,DK] row-major
    const u16* V;              // [B,Hkv,T,DV]
    const u16* Kc;             // [B,Hkv,N,DK] (compressed branch)
    const u16* Vc;             // [B,Hkv,N,DV]
    const int32_t* sel;        // [B,T,Hkv,top_n]
    const u16* dO;             // [B,T,H,DV]
    const float* stats;        // [B,T,H,3,4] lse2, D, sigma (see AttnParams)
    float* dQ;                 // [B,T,H,DK], written
    float* dK;                 // [B,Hkv,T,DK], accumulated
    float* dV;
    float* dKc;                // [B,Hkv,N,DK], accumulated
    float* dVc;
    const int* bucket_start;   // block lists of the selected branch (launch_block_lists)
    const int* tile_start;
    const int* tile_bucket;
    const int* entries;
    int B, T, Hkv, G, N, l, s, lp, top_n, window, branches, n_slc, n_bucket;
    int nsb;                   // 64-key sub-blocks per selection block
    int n_kb_cmp, n_qt, qt_cmp;   // compressed key blocks, query tiles, tokens per tile
    int n_kb_win, n_qt_win;    // window key blocks, query tiles per window key block
    int n_cmp_items, n_win_items;
    float scale, scale_log2;
};
void launch_fill_zero(float* x, size_t n, hipStream_t st);   // x 16-byte aligned
void launch_fill_f32(float* x, size_t n, float v, hipStream_t st);
bool launch_bwd_dq(int DK, int DV, const BwdParams& p, hipStream_t st);
bool launch_bwd_dkv(int DK, int DV, const BwdParams& p, int n_slc_items, hipStream_t st);
// linear block map backward for one of K / V: dX += dY.W^T scattered to tokens, dW and dpe
// overwritten; colsum: d floats of scratch
void launch_compress_bwd(const u16* X, const u16* W, const u16* pe, const float* dY, float* dX, float* dW, float* dpe,
                         float* colsum, int BG, int T, int N, int d, int l, int s, hipStream_t st);

// ---- dense causal attention ----
struct FullParams {
    const u16* Q;        // [B,T,H,DK]
    const u16* Kf;       // keys in fragment order (tile_cmp layout), Tpad per unit
    const u16* Vf;       // values in fragment order, fp16 scaled by 2^-vexp
    const int* vexp;     // [B*Hkv]
    u16* O;              // [B,T,H,DV]
    int B, T, Tpad, Hkv;
    float scale_log2;
};
size_t full_attn_lds_bytes(int DK, int DV);
bool launch_full_attn(int DK, int DV, int G, const FullParams& p, hipStream_t st);

// ---- decode ----
struct DecodeParams {
    const u16* q;              // [B,H,DK]
    const u16* K;              // [B,Hkv,L,DK]
    const u16* V;              // [B,Hkv,L,DV]
    const int32_t* cache_len;  // [B]
    const u16* Kc;             // [B,Hkv,Nc,DK]
    const u16* Vc;             // [B,Hkv,Nc,DV]
    const float* gates;        // [B,H,3] or null
    u16* O;                    // [B,H,DV]
    int32_t* sel_out;          // [B,Hkv,top_n] or null
    // workspace
    float* part_m;             // [B,Hkv,n_split,16]
    float* part_l;             // [B,Hkv,n_split,16]
    u16* part_o;               // [B,Hkv,n_split,16,DV] fp16
    float* part_a;             // [B,Hkv,n_split,jb,16]
    int32_t* sel_ws;           // [B,Hkv,top_n]
    float* cmp_w;              // [B,Hkv,n_split,16] weight 2^(m_split - lse) of each split
    float* att_m;              // [B,Hkv,n_items,16]
    float* att_l;              // [B,Hkv,n_items,16]
    u16* att_o;                // [B,Hkv,n_items,16,DV] fp16
    int B, L, Hkv, G, Nc, l, s, lp, n_slc, top_n, n_init, n_local, window, branches;
    int n_split, jb, n_items;
    float scale_log2;
};
constexpr int kDecodeSplitKeys = 256;
constexpr int kDecodeMaxSplits = 32;   // compressed keys per decode call <= 256 * 32
constexpr int kDecodeMaxItems = 32;    // work items per branch (top_n <= 32, window <= 1920)
int decode_jb(int l, int s, int lp);
int decode_items(int top_n, int window);
bool launch_decode(int DK, int DV, const DecodeParams& p, hipStream_t st);

// ---- decode cache maintenance ----
struct AppendParams {
    const u16* K_new;          // [B,Hkv,n_new,dk]
    const u16* V_new;          // [B,Hkv,n_new,dv]
    u16* K_cache;              // [B,Hkv,L,dk]
    u16* V_cache;              // [B,Hkv,L,dv]
    int32_t* cache_len;        // [B], advanced by n_new
    const u16* wt_k;           // prepared weights: W_k^T [dk, l*dk], W_v^T [dv, l*dv]
    const u16* wt_v;
    const float* bias_k;       // vec(pe_k) . W_k [dk], vec(pe_v) . W_v [dv]
    const float* bias_v;
    u16* K_cmp;                // [B,Hkv,N,dk]
    u16* V_cmp;                // [B,Hkv,N,dv]
    int B, Hkv, L, dk, dv, l, s, N, n_new;
    int R;                     // candidate blocks per group: append_rows_per_group(n_new, s)
};
int append_rows_per_group(int n_new, int s);
void launch_cache_append(const AppendParams& p, hipStream_t st);

// ---- fixed device scratch (scratch.hip) ----
size_t static_scratch_bytes();
void* static_scratch(hipError_t* err);

}  // namespace nsa
