// C ABI of the NSA library (declared in include/nsa.h): argument validation, workspace
// layout and kernel dispatch.  Nothing here allocates device memory or synchronizes.
#include "nsa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <string>

#include "launch.hpp"

namespace {

thread_local std::string g_detail;

nsa_status fail(nsa_status st, const std::string& msg) {
    g_detail = msg;
    return st;
}

struct Shape {
    int B, T, Hkv, G, H, dk, dv, l, s, lp, n, n_init, n_local, w, phi, mode, br;
    int n_cmp, n_slc;
    float scale;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int round_up(int x, int a) { return (x + a - 1) / a * a; }

nsa_status check_config(const nsa_config* c, Shape* sh) {
    if (!c) return fail(NSA_ERR_NULL, "config is NULL");
    if (c->struct_size < sizeof(nsa_config)) return fail(NSA_ERR_SHAPE, "config.struct_size too small");
    Shape s{};
    s.B = c->batch; s.T = c->seq_len; s.Hkv = c->num_kv_heads; s.G = c->heads_per_group;
    s.dk = c->d_k; s.dv = c->d_v; s.l = c->cmp_block; s.s = c->cmp_stride; s.lp = c->slc_block;
    s.n = c->top_n; s.n_init = c->n_init; s.n_local = c->n_local; s.w = c->window;
    s.phi = c->phi; s.mode = c->score_mode; s.br = c->branches;
    if (s.B <= 0 || s.T <= 0 || s.Hkv <= 0 || s.G <= 0 || s.dk <= 0 || s.dv <= 0 || s.l <= 0 || s.s <= 0 || s.lp <= 0)
        return fail(NSA_ERR_SHAPE, "sizes must be positive");
    if (s.n < 0 || s.n_init < 0 || s.n_local < 0 || s.w < 0) return fail(NSA_ERR_SHAPE, "negative count");
    if (s.G != 1 && s.G != 2 && s.G != 4 && s.G != 8 && s.G != 16)
        return fail(NSA_ERR_UNSUPPORTED, "heads_per_group must be 1, 2, 4, 8 or 16");
    if (!((s.dk == 192 && s.dv == 128) || (s.dk == 128 && s.dv == 128) || (s.dk == 64 && s.dv == 64)))
        return fail(NSA_ERR_UNSUPPORTED, "(d_k, d_v) must be (192,128), (128,128) or (64,64)");
    if (s.l % s.s != 0 || s.lp % s.s != 0) return fail(NSA_ERR_UNSUPPORTED, "cmp_stride must divide cmp_block and slc_block");
    if (s.lp % 32 != 0) return fail(NSA_ERR_UNSUPPORTED, "slc_block must be a multiple of 32");
    if (s.n > 32) return fail(NSA_ERR_UNSUPPORTED, "top_n must be <= 32");
    if (s.n < s.n_init + s.n_local) return fail(NSA_ERR_UNSUPPORTED, "top_n smaller than the forced blocks");
    if (s.phi != NSA_PHI_LINEAR && s.phi != NSA_PHI_MEAN) return fail(NSA_ERR_SHAPE, "unknown phi");
    if (s.mode != NSA_SCORE_CMP_OVERLAP && s.mode != NSA_SCORE_MEAN_DOT) return fail(NSA_ERR_SHAPE, "unknown score_mode");
    if (s.br <= 0 || s.br > 7) return fail(NSA_ERR_SHAPE, "branches must be a non-empty OR of NSA_BR_*");
    if (s.mode == NSA_SCORE_MEAN_DOT) {
        if (s.l != s.s || s.l != s.lp) return fail(NSA_ERR_UNSUPPORTED, "MEAN_DOT needs cmp_block == cmp_stride == slc_block");
        if (s.n_local < 1) return fail(NSA_ERR_UNSUPPORTED, "MEAN_DOT needs n_local >= 1 (the own block is incomplete)");
        if (s.br & NSA_BR_CMP) return fail(NSA_ERR_UNSUPPORTED, "MEAN_DOT has no compressed-branch output");
    }
    if ((double)s.B * s.T * s.Hkv * s.G * std::max(s.dk, s.dv) > 4.0e12) return fail(NSA_ERR_SHAPE, "problem too large");
    s.H = s.Hkv * s.G;
    s.n_cmp = s.T >= s.l ? (s.T - s.l) / s.s + 1 : 0;
    s.n_slc = (s.T + s.lp - 1) / s.lp;
    s.scale = c->softmax_scale > 0.f ? c->softmax_scale : 1.0f / std::sqrt((float)s.dk);
    *sh = s;
    return NSA_OK;
}

nsa_status hip_check(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(NSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return NSA_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---- workspace layouts ----
struct CompressWs { size_t wt_k, wt_v, bias_k, bias_v, total; };
CompressWs compress_ws(const Shape& s) {
    CompressWs w{};
    if (s.phi != NSA_PHI_LINEAR) return w;
    size_t off = 0;
    w.wt_k = off; off = align_up(off + (size_t)s.l * s.dk * s.dk * 2, 256);
    w.wt_v = off; off = align_up(off + (size_t)s.l * s.dv * s.dv * 2, 256);
    w.bias_k = off; off = align_up(off + (size_t)s.dk * 4, 256);
    w.bias_v = off; off = align_up(off + (size_t)s.dv * 4, 256);
    w.total = off;
    return w;
}

// compressed keys and values in fragment order with the values' scaling (mode 0), block scores
// MEAN_DOT scoring with one query head per KV head and few picks selects inside the
// scoring kernel: no scores workspace.
bool fused_mean_select(const Shape& s) {
    return s.mode == NSA_SCORE_MEAN_DOT && s.G == 1 && s.n - s.n_local <= nsa::kFusedMaxPicks;
}

struct SelectWs { size_t kf, vf, vmax, vexp, scores, total; int npad; };
SelectWs select_ws(const Shape& s) {
    SelectWs w{};
    size_t off = 0;
    w.npad = round_up(std::max(s.n_cmp, 1), 64);
    if (s.mode == NSA_SCORE_CMP_OVERLAP) {
        const size_t bg = (size_t)s.B * s.Hkv;
        w.kf = off; off = align_up(off + bg * w.npad * s.dk * 2, 256);
        w.vf = off; off = align_up(off + bg * w.npad * s.dv * 2, 256);
        w.vmax = off; off = align_up(off + bg * nsa::cmp_vmax_parts() * 4, 256);
        w.vexp = off; off = align_up(off + bg * 4, 256);
    }
    w.scores = off;
    // (with no complete compressed block the selection runs on a zero score row)
    if (!fused_mean_select(s) || s.n_cmp == 0) off = align_up(off + (size_t)s.B * s.T * s.Hkv * s.n_slc * 4, 256);
    w.total = off;
    return w;
}

// dense causal attention: keys in fragment order, values as a scaled fp16 copy
struct FullWs { size_t kf, vf, vmax, vexp, total; int tpad; };
FullWs full_ws(const Shape& s) {
    FullWs w{};
    w.tpad = round_up(s.T, 64);
    const size_t bg = (size_t)s.B * s.Hkv;
    size_t off = 0;
    w.kf = off; off = align_up(off + bg * w.tpad * s.dk * 2, 256);
    w.vf = off; off = align_up(off + bg * w.tpad * s.dv * 2, 256);
    w.vmax = off; off = align_up(off + bg * nsa::cmp_vmax_parts() * 4, 256);
    w.vexp = off; off = align_up(off + bg * 4, 256);
    w.total = off;
    return w;
}

// One query head per KV head with only the selected branch (the MoBA configuration) runs
// the block-major schedule of moba.hip.
bool use_block_major(const Shape& s) { return s.G == 1 && s.br == NSA_BR_SLC; }

// V (and K) copied into MFMA fragment order, padded with 64 zero keys past a multiple of 64,
// V's fp16 scaling; then either the K copy or, for the block-major schedule (which gathers K
// from the row-major keys), the bucket lists and the per-slot partial results, over the same
// bytes (the training forward runs the query-centric kernel on the K copy even for those
// shapes).
struct AttnWs {
    size_t kf, vf, vmax, vexp, hist, bcnt, bstart, tstart, tbk, entries, pm, pl, po, total;
    int tpad, n_chunk, n_bucket;
};
AttnWs attn_ws(const Shape& s) {
    AttnWs w{};
    w.tpad = round_up(s.T, 64) + 64;   // a 64-key tile may start at any multiple of 32 below T
    const size_t bg = (size_t)s.B * s.Hkv;
    size_t off = 0;
    w.vf = off; off = align_up(off + bg * w.tpad * s.dv * 2, 256);
    w.vmax = off; off = align_up(off + bg * nsa::cmp_vmax_parts() * 4, 256);   // V's fp16 scaling
    w.vexp = off; off = align_up(off + bg * 4, 256);
    const size_t u0 = off;
    w.kf = u0;
    const size_t kf_end = align_up(u0 + bg * w.tpad * s.dk * 2, 256);
    off = u0;
    if (use_block_major(s)) {
        w.n_chunk = nsa::moba_n_chunk(s.T);
        w.n_bucket = (int)(bg * s.n_slc);
        const size_t rows = bg * s.T * s.n;   // (b, t, h, slot)
        w.hist = off; off = align_up(off + bg * w.n_chunk * s.n_slc * 4, 256);
        w.bcnt = off; off = align_up(off + (size_t)w.n_bucket * 4, 256);
        w.bstart = off; off = align_up(off + (size_t)(w.n_bucket + 1) * 4, 256);
        w.tstart = off; off = align_up(off + (size_t)(w.n_bucket + 1) * 4, 256);
        w.tbk = off; off = align_up(off + (size_t)nsa::moba_max_tiles((int)bg, s.T, s.n, s.n_slc) * 4, 256);
        w.entries = off; off = align_up(off + rows * 4, 256);
        w.pm = off; off = align_up(off + rows * 4, 256);
        w.pl = off; off = align_up(off + rows * 4, 256);
        w.po = off; off = align_up(off + rows * s.dv * 2, 256);
    }
    w.total = std::max(off, kf_end);
    return w;
}

struct DecodeWs { size_t pm, pl, po, pa, sel, cw, am, al, ao, total; int n_split, jb, n_items; };
DecodeWs decode_ws(const Shape& s) {
    DecodeWs w{};
    w.n_split = std::max(1, (s.n_cmp + nsa::kDecodeSplitKeys - 1) / nsa::kDecodeSplitKeys);
    w.jb = nsa::decode_jb(s.l, s.s, s.lp);
    w.n_items = nsa::decode_items(s.n, s.w);
    const size_t bg = (size_t)s.B * s.Hkv;
    size_t off = 0;
    w.pm = off; off = align_up(off + bg * w.n_split * 16 * 4, 256);
    w.pl = off; off = align_up(off + bg * w.n_split * 16 * 4, 256);
    w.po = off; off = align_up(off + bg * w.n_split * s.dv * 16 * 2, 256);
    w.pa = off; off = align_up(off + bg * w.n_split * 16 * w.jb * 4, 256);
    w.sel = off; off = align_up(off + bg * std::max(s.n, 1) * 4, 256);
    w.cw = off; off = align_up(off + bg * w.n_split * 16 * 4, 256);
    w.am = off; off = align_up(off + bg * w.n_items * 16 * 4, 256);
    w.al = off; off = align_up(off + bg * w.n_items * 16 * 4, 256);
    w.ao = off; off = align_up(off + bg * w.n_items * s.dv * 16 * 2, 256);
    w.total = off;
    return w;
}

// the fused prefill: the scoring call's and the attention call's workspaces side by side,
// plus room for the lists and o_cmp when the caller does not take them
struct PrefillWs { SelectWs sel; AttnWs attn; size_t attn_off, sel_out, ocmp_out, total; };
PrefillWs prefill_ws(const Shape& s) {
    PrefillWs w{};
    w.sel = select_ws(s);
    w.attn = attn_ws(s);
    size_t off = w.sel.total;
    w.attn_off = off; off = align_up(off + w.attn.total, 256);
    w.sel_out = off; off = align_up(off + (size_t)s.B * s.T * s.Hkv * std::max(s.n, 1) * 4, 256);
    w.ocmp_out = off; off = align_up(off + (size_t)s.B * s.T * s.H * s.dv * 4, 256);
    w.total = off;
    return w;
}

// backward of the branches: K, V in fragment order for the statistics pass, the per-row
// statistics, and the selected branch's block lists (own block included)
struct BwdWs {
    size_t kf, vf, vmax, vexp, stats, hist, bcnt, bstart, tstart, tbk, entries, total;
    int tpad, n_chunk, n_bucket;
};
BwdWs bwd_ws(const Shape& s) {
    BwdWs w{};
    w.tpad = round_up(s.T, 64) + 64;
    const size_t bg = (size_t)s.B * s.Hkv;
    size_t off = 0;
    w.kf = off; off = align_up(off + bg * w.tpad * s.dk * 2, 256);
    w.vf = off; off = align_up(off + bg * w.tpad * s.dv * 2, 256);
    w.vmax = off; off = align_up(off + bg * nsa::cmp_vmax_parts() * 4, 256);
    w.vexp = off; off = align_up(off + bg * 4, 256);
    w.stats = off; off = align_up(off + (size_t)s.B * s.T * s.H * 12 * 4, 256);
    if (s.br & NSA_BR_SLC) {
        w.n_chunk = nsa::moba_n_chunk(s.T);
        w.n_bucket = (int)(bg * s.n_slc);
        w.hist = off; off = align_up(off + bg * w.n_chunk * s.n_slc * 4, 256);
        w.bcnt = off; off = align_up(off + (size_t)w.n_bucket * 4, 256);
        w.bstart = off; off = align_up(off + (size_t)(w.n_bucket + 1) * 4, 256);
        w.tstart = off; off = align_up(off + (size_t)(w.n_bucket + 1) * 4, 256);
        w.tbk = off; off = align_up(off + (size_t)nsa::moba_max_tiles((int)bg, s.T, s.n, s.n_slc) * 4, 256);
        w.entries = off; off = align_up(off + bg * s.T * s.n * 4, 256);
    }
    w.total = off;
    return w;
}

// backward of the linear block map: one column-sum vector per map
size_t compress_bwd_ws(const Shape& s) { return align_up((size_t)s.dk * 4, 256) + align_up((size_t)s.dv * 4, 256); }

nsa_status check_ws(void* ws, size_t have, size_t need) {
    if (need == 0) return NSA_OK;
    if (!ws) return fail(NSA_ERR_WORKSPACE, "workspace is NULL");
    if (have < need) return fail(NSA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(NSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    return NSA_OK;
}

nsa_status check_align16(const void* p, const char* name) {
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return fail(NSA_ERR_SHAPE, std::string(name) + " must be 16-byte aligned");
    return NSA_OK;
}

template <typename T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }

}  // namespace

extern "C" {

nsa_status nsa_workspace_size(const nsa_config* cfg, int op, size_t* bytes) {
    g_detail.clear();
    if (!bytes) return fail(NSA_ERR_NULL, "bytes is NULL");
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    switch (op) {
        case NSA_OP_COMPRESS: *bytes = compress_ws(s).total; break;
        case NSA_OP_SCORE_SELECT: *bytes = select_ws(s).total; break;
        case NSA_OP_SPARSE_ATTN: *bytes = attn_ws(s).total; break;
        case NSA_OP_DECODE: *bytes = decode_ws(s).total; break;
        case NSA_OP_FULL_ATTN: *bytes = full_ws(s).total; break;
        case NSA_OP_SPARSE_BWD: *bytes = bwd_ws(s).total; break;
        case NSA_OP_COMPRESS_BWD: *bytes = compress_bwd_ws(s); break;
        case NSA_OP_PREFILL: *bytes = prefill_ws(s).total; break;
        default: return fail(NSA_ERR_SHAPE, "unknown op");
    }
    return NSA_OK;
}

// W^T and the position-embedding bias vec(pe) . W of both linear maps, into a buffer laid
// out as compress_ws.
void prepare_weights(const Shape& s, const CompressWs& w, const void* W_k, const void* W_v, const void* pe_k,
                     const void* pe_v, void* ws, hipStream_t hs) {
    using nsa::u16;
    const int KDk = s.l * s.dk, KDv = s.l * s.dv;
    u16* wtk = at<u16>(ws, w.wt_k);
    u16* wtv = at<u16>(ws, w.wt_v);
    nsa::launch_transpose_w(static_cast<const u16*>(W_k), wtk, KDk, s.dk, hs);
    nsa::launch_transpose_w(static_cast<const u16*>(W_v), wtv, KDv, s.dv, hs);
    nsa::launch_pe_bias(static_cast<const u16*>(pe_k), wtk, at<float>(ws, w.bias_k), KDk, s.dk, hs);
    nsa::launch_pe_bias(static_cast<const u16*>(pe_v), wtv, at<float>(ws, w.bias_v), KDv, s.dv, hs);
}

nsa_status nsa_compress(const nsa_config* cfg, const void* K, const void* V, const void* W_k, const void* W_v,
                        const void* pe_k, const void* pe_v, void* K_cmp, void* V_cmp, void* ws, size_t ws_bytes,
                        void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    if (s.n_cmp == 0) return NSA_OK;   // shorter than one block: nothing to compress
    if (!K || !K_cmp) return fail(NSA_ERR_NULL, "K and K_cmp are required");
    const int BG = s.B * s.Hkv;
    const hipStream_t hs = as_stream(stream);
    using nsa::u16;
    if (s.phi == NSA_PHI_MEAN) {
        if (s.dk > 1024) return fail(NSA_ERR_UNSUPPORTED, "d_k too large");
        nsa::launch_compress_mean(static_cast<const u16*>(K), static_cast<u16*>(K_cmp), BG, s.T, s.dk, s.l, s.s,
                                  s.n_cmp, hs);
        return hip_check("compress_mean");
    }
    if (!V || !W_k || !W_v || !pe_k || !pe_v || !V_cmp)
        return fail(NSA_ERR_NULL, "linear phi needs V, W_k, W_v, pe_k, pe_v and V_cmp");
    const CompressWs w = compress_ws(s);
    if ((st = check_ws(ws, ws_bytes, w.total)) != NSA_OK) return st;
    if ((st = check_align16(K, "K")) != NSA_OK || (st = check_align16(V, "V")) != NSA_OK) return st;
    prepare_weights(s, w, W_k, W_v, pe_k, pe_v, ws, hs);
    u16* wtk = at<u16>(ws, w.wt_k);
    u16* wtv = at<u16>(ws, w.wt_v);
    float* bk = at<float>(ws, w.bias_k);
    float* bv = at<float>(ws, w.bias_v);
    nsa::launch_compress_linear(static_cast<const u16*>(K), wtk, bk, static_cast<u16*>(K_cmp), BG, s.T, s.dk, s.dk,
                                s.l, s.s, s.n_cmp, hs);
    nsa::launch_compress_linear(static_cast<const u16*>(V), wtv, bv, static_cast<u16*>(V_cmp), BG, s.T, s.dv, s.dv,
                                s.l, s.s, s.n_cmp, hs);
    return hip_check("compress_linear");
}

namespace {
// Steps a2-a4 when the sequence is shorter than one compressed block (no compressed key is
// visible to any query): o_cmp = 0, LSE = -inf, every block score 0, so the selection keeps
// the forced blocks and fills any other slot by the lowest eligible index.
nsa_status no_block_select(const Shape& s, float* scores, int32_t* sel_idx, float* lse_cmp, float* o_cmp,
                           hipStream_t hs) {
    nsa::launch_fill_f32(scores, (size_t)s.B * s.T * s.Hkv * s.n_slc, 0.f, hs);
    if (lse_cmp) nsa::launch_fill_f32(lse_cmp, (size_t)s.B * s.T * s.H, -INFINITY, hs);
    if (o_cmp) nsa::launch_fill_f32(o_cmp, (size_t)s.B * s.T * s.H * s.dv, 0.f, hs);
    nsa::launch_select_from_scores(scores, sel_idx, s.B, s.T, s.Hkv, s.n_slc, s.lp, s.n, s.n_init, s.n_local, hs);
    return hip_check("score_select");
}
}  // namespace

nsa_status nsa_score_select(const nsa_config* cfg, const void* Q, const void* K_cmp, const void* V_cmp,
                            int32_t* sel_idx, float* lse_cmp, float* o_cmp, void* ws, size_t ws_bytes,
                            void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    if (!Q || !sel_idx || (!K_cmp && s.n_cmp > 0)) return fail(NSA_ERR_NULL, "Q, K_cmp and sel_idx are required");
    if (s.n_slc > 64 * 32) return fail(NSA_ERR_UNSUPPORTED, "at most 2048 selection blocks");
    if (s.mode == NSA_SCORE_MEAN_DOT && (lse_cmp || o_cmp))
        return fail(NSA_ERR_SHAPE, "MEAN_DOT mode produces no lse_cmp / o_cmp");
    const bool with_o = o_cmp != nullptr;
    if (with_o && !V_cmp && s.n_cmp > 0) return fail(NSA_ERR_NULL, "o_cmp needs V_cmp");
    if (s.mode == NSA_SCORE_CMP_OVERLAP && nsa::cmp_attn_lds_bytes(s.dk, s.dv, s.G, with_o) > 160 * 1024)
        return fail(NSA_ERR_UNSUPPORTED, "tile too large for one workgroup's LDS");
    if (s.mode == NSA_SCORE_CMP_OVERLAP) {
        const int R = s.lp / s.s, L = s.l / s.s;
        if (64 % R != 0 || L > 64)
            return fail(NSA_ERR_UNSUPPORTED, "slc_block / cmp_stride must divide 64 and cmp_block / cmp_stride <= 64");
    }
    const SelectWs w = select_ws(s);
    if ((st = check_ws(ws, ws_bytes, w.total)) != NSA_OK) return st;
    const hipStream_t hs = as_stream(stream);
    if (s.n_cmp == 0) return no_block_select(s, at<float>(ws, w.scores), sel_idx, lse_cmp, o_cmp, hs);
    using nsa::u16;
    nsa::SelParams p{};
    p.Q = static_cast<const u16*>(Q);
    p.Kc = static_cast<const u16*>(K_cmp);
    p.scores = at<float>(ws, w.scores);
    p.B = s.B; p.T = s.T; p.Hkv = s.Hkv; p.N = s.n_cmp; p.Npad = w.npad; p.l = s.l; p.s = s.s; p.lp = s.lp;
    p.n_slc = s.n_slc;
    p.scale_log2 = s.scale * nsa::kLog2eHost;
    if (s.mode == NSA_SCORE_CMP_OVERLAP) {
        u16* kf = at<u16>(ws, w.kf);
        u16* vf = with_o ? at<u16>(ws, w.vf) : nullptr;
        if (!nsa::launch_tile_cmp(s.dk, s.dv, p.Kc, with_o ? static_cast<const u16*>(V_cmp) : nullptr,
                                  at<uint32_t>(ws, w.vmax), at<int>(ws, w.vexp), kf, vf, s.B * s.Hkv, s.n_cmp, w.npad,
                                  hs))
            return fail(NSA_ERR_UNSUPPORTED, "no layout kernel for this shape");
        p.Kf = kf;
        p.Vf = vf;
        p.vexp = at<int>(ws, w.vexp);
        p.lse = lse_cmp;
        p.o_cmp = o_cmp;
        if (!nsa::launch_cmp_attn(with_o, s.dk, s.dv, s.G, p, hs))
            return fail(NSA_ERR_UNSUPPORTED, "no compressed-attention kernel for this shape");
    } else if (fused_mean_select(s)) {
        p.sel = sel_idx;
        p.top_n = s.n; p.n_init = s.n_init; p.n_local = s.n_local;
        if (!nsa::launch_mean_select(s.dk, p, hs)) return fail(NSA_ERR_UNSUPPORTED, "no score kernel for this shape");
        return hip_check("score_select");
    } else if (!nsa::launch_mean_scores(s.dk, s.G, p, hs)) {
        return fail(NSA_ERR_UNSUPPORTED, "no score kernel for this shape");
    }
    nsa::launch_select_from_scores(p.scores, sel_idx, s.B, s.T, s.Hkv, s.n_slc, s.lp, s.n, s.n_init, s.n_local, hs);
    return hip_check("score_select");
}

nsa_status nsa_select_from_scores(const nsa_config* cfg, const float* scores, int32_t* sel_idx, void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    if (!scores || !sel_idx) return fail(NSA_ERR_NULL, "scores and sel_idx are required");
    if (s.n_slc > 64 * 32) return fail(NSA_ERR_UNSUPPORTED, "at most 2048 selection blocks");
    nsa::launch_select_from_scores(scores, sel_idx, s.B, s.T, s.Hkv, s.n_slc, s.lp, s.n, s.n_init, s.n_local,
                                   as_stream(stream));
    return hip_check("select_from_scores");
}

namespace {
nsa_status sparse_attn_fwd_impl(const nsa_config* cfg, const void* Q, const void* K, const void* V,
                                const int32_t* sel_idx, const float* o_cmp, const float* gate_logits, void* O,
                                float* saved_lse, float* saved_o, void* ws, size_t ws_bytes, void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    const bool train = saved_lse != nullptr || saved_o != nullptr;
    if (train && (!saved_lse || !saved_o)) return fail(NSA_ERR_NULL, "saved_lse and saved_o go together");
    if (!Q || !K || !V || !O) return fail(NSA_ERR_NULL, "Q, K, V and O are required");
    if ((s.br & NSA_BR_SLC) && !sel_idx) return fail(NSA_ERR_NULL, "sel_idx is required for the selected branch");
    if ((s.br & NSA_BR_CMP) && !o_cmp) return fail(NSA_ERR_NULL, "o_cmp is required for the compressed branch");
    if ((s.br & NSA_BR_WIN) && s.w <= 0) return fail(NSA_ERR_SHAPE, "window branch with window = 0");
    const AttnWs w = attn_ws(s);
    if ((st = check_ws(ws, ws_bytes, w.total)) != NSA_OK) return st;
    const hipStream_t hs = as_stream(stream);
    using nsa::u16;
    const bool block_major = use_block_major(s) && !train;
    if (block_major && (long long)s.T >= (1LL << 26))
        return fail(NSA_ERR_UNSUPPORTED, "sequence too long for the block lists");
    // the block-major kernel gathers K from the row-major keys: only V is copied for it
    u16* kf = block_major ? nullptr : at<u16>(ws, w.kf);
    u16* vf = at<u16>(ws, w.vf);
    // fragment order, V as fp16 scaled by a power of two per (sequence, group)
    if (!nsa::launch_tile_cmp(s.dk, s.dv, static_cast<const u16*>(K), static_cast<const u16*>(V),
                              at<uint32_t>(ws, w.vmax), at<int>(ws, w.vexp), kf, vf, s.B * s.Hkv, s.T, w.tpad, hs))
        return fail(NSA_ERR_UNSUPPORTED, "no layout kernel");
    if (block_major) {
        nsa::MobaParams m{};
        m.Q = static_cast<const u16*>(Q);
        m.K = static_cast<const u16*>(K);
        m.Vf = vf;
        m.vexp = at<int>(ws, w.vexp);
        m.sel = sel_idx;
        m.gates = gate_logits;
        m.O = static_cast<u16*>(O);
        m.hist = at<int>(ws, w.hist);
        m.bucket_cnt = at<int>(ws, w.bcnt);
        m.bucket_start = at<int>(ws, w.bstart);
        m.tile_start = at<int>(ws, w.tstart);
        m.tile_bucket = at<int>(ws, w.tbk);
        m.entries = at<int>(ws, w.entries);
        m.part_m = at<float>(ws, w.pm);
        m.part_l = at<float>(ws, w.pl);
        m.part_o = at<u16>(ws, w.po);
        m.B = s.B; m.T = s.T; m.Tpad = w.tpad; m.Hkv = s.Hkv; m.lp = s.lp; m.n_slc = s.n_slc; m.top_n = s.n;
        m.n_chunk = w.n_chunk; m.n_bucket = w.n_bucket; m.n_own = nsa::moba_n_own(s.B * s.Hkv, s.n_slc, s.lp);
        m.scale_log2 = s.scale * nsa::kLog2eHost;
        if (!nsa::launch_moba_attn(s.dk, s.dv, m, hs)) return fail(NSA_ERR_UNSUPPORTED, "no block-major kernel");
        return hip_check("sparse_attn");
    }
    nsa::AttnParams p{};
    p.Q = static_cast<const u16*>(Q);
    p.Kf = kf;
    p.Vf = vf;
    p.vexp = at<int>(ws, w.vexp);
    p.sel = sel_idx;
    p.o_cmp = o_cmp;
    p.gates = gate_logits;
    p.O = static_cast<u16*>(O);
    p.saved_lse = saved_lse;
    p.saved_o = saved_o;
    p.B = s.B; p.T = s.T; p.Tpad = w.tpad; p.Hkv = s.Hkv; p.G = s.G; p.lp = s.lp; p.top_n = s.n; p.window = s.w;
    p.branches = s.br;
    p.scale_log2 = s.scale * nsa::kLog2eHost;
    if (!nsa::launch_sparse_attn(s.dk, s.dv, p, s.B, hs)) return fail(NSA_ERR_UNSUPPORTED, "no attention kernel");
    return hip_check("sparse_attn");
}
}  // namespace

nsa_status nsa_sparse_attn_fwd(const nsa_config* cfg, const void* Q, const void* K, const void* V,
                               const int32_t* sel_idx, const float* o_cmp, const float* gate_logits, void* O,
                               void* ws, size_t ws_bytes, void* stream) {
    return sparse_attn_fwd_impl(cfg, Q, K, V, sel_idx, o_cmp, gate_logits, O, nullptr, nullptr, ws, ws_bytes,
                                stream);
}

nsa_status nsa_sparse_attn_fwd_train(const nsa_config* cfg, const void* Q, const void* K, const void* V,
                                     const int32_t* sel_idx, const float* o_cmp, const float* gate_logits, void* O,
                                     float* saved_lse, float* saved_o, void* ws, size_t ws_bytes, void* stream) {
    if (!saved_lse || !saved_o) {
        g_detail.clear();
        return fail(NSA_ERR_NULL, "saved_lse and saved_o are required");
    }
    if ((reinterpret_cast<uintptr_t>(saved_o) & 15u) != 0 || (reinterpret_cast<uintptr_t>(saved_lse) & 7u) != 0) {
        g_detail.clear();
        return fail(NSA_ERR_SHAPE, "saved_o must be 16-byte and saved_lse 8-byte aligned");
    }
    return sparse_attn_fwd_impl(cfg, Q, K, V, sel_idx, o_cmp, gate_logits, O, saved_lse, saved_o, ws, ws_bytes,
                                stream);
}

nsa_status nsa_prefill_fwd(const nsa_config* cfg, const void* Q, const void* K, const void* V, const void* K_cmp,
                           const void* V_cmp, const float* gate_logits, void* O, int32_t* sel_idx, float* lse_cmp,
                           float* o_cmp, void* ws, size_t ws_bytes, void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    if (!Q || !K || !V || !O || ((!K_cmp || !V_cmp) && s.n_cmp > 0))
        return fail(NSA_ERR_NULL, "Q, K, V, K_cmp, V_cmp and O are required");
    if (s.mode != NSA_SCORE_CMP_OVERLAP)
        return fail(NSA_ERR_UNSUPPORTED, "the fused prefill scores blocks by compressed attention (CMP_OVERLAP)");
    if (s.n_slc > 64 * 32) return fail(NSA_ERR_UNSUPPORTED, "at most 2048 selection blocks");
    {
        const int R = s.lp / s.s, L = s.l / s.s;
        if (64 % R != 0 || L > 64)
            return fail(NSA_ERR_UNSUPPORTED, "slc_block / cmp_stride must divide 64 and cmp_block / cmp_stride <= 64");
    }
    if (nsa::prefill_lds_bytes(s.dk, s.dv, s.G) > 160 * 1024)
        return fail(NSA_ERR_UNSUPPORTED, "tile too large for one workgroup's LDS");
    if ((s.br & NSA_BR_WIN) && s.w <= 0) return fail(NSA_ERR_SHAPE, "window branch with window = 0");
    const PrefillWs w = prefill_ws(s);
    if ((st = check_ws(ws, ws_bytes, w.total)) != NSA_OK) return st;
    if (o_cmp && (reinterpret_cast<uintptr_t>(o_cmp) & 15u) != 0) return fail(NSA_ERR_SHAPE, "o_cmp must be 16-byte aligned");
    const hipStream_t hs = as_stream(stream);
    using nsa::u16;
    int32_t* sel = sel_idx ? sel_idx : at<int32_t>(ws, w.sel_out);
    float* oc = o_cmp ? o_cmp : at<float>(ws, w.ocmp_out);
    // compressed keys/values in fragment order (V as scaled fp16)
    nsa::SelParams sp{};
    if (s.n_cmp == 0) {   // no complete compressed block: steps a2-a4 without the scoring kernel
        if ((st = no_block_select(s, at<float>(ws, w.sel.scores), sel, lse_cmp, oc, hs)) != NSA_OK) return st;
    } else {
        sp.Q = static_cast<const u16*>(Q);
        sp.Kc = static_cast<const u16*>(K_cmp);
        sp.scores = at<float>(ws, w.sel.scores);
        sp.sel = sel;
        sp.top_n = s.n; sp.n_init = s.n_init; sp.n_local = s.n_local;
        sp.B = s.B; sp.T = s.T; sp.Hkv = s.Hkv; sp.N = s.n_cmp; sp.Npad = w.sel.npad; sp.l = s.l; sp.s = s.s; sp.lp = s.lp;
        sp.n_slc = s.n_slc;
        sp.scale_log2 = s.scale * nsa::kLog2eHost;
        u16* ckf = at<u16>(ws, w.sel.kf);
        u16* cvf = at<u16>(ws, w.sel.vf);
        if (!nsa::launch_tile_cmp(s.dk, s.dv, sp.Kc, static_cast<const u16*>(V_cmp), at<uint32_t>(ws, w.sel.vmax),
                                  at<int>(ws, w.sel.vexp), ckf, cvf, s.B * s.Hkv, s.n_cmp, w.sel.npad, hs))
            return fail(NSA_ERR_UNSUPPORTED, "no layout kernel for this shape");
        sp.Kf = ckf;
        sp.Vf = cvf;
        sp.vexp = at<int>(ws, w.sel.vexp);
        sp.lse = lse_cmp;
        sp.o_cmp = oc;
    }
    // K and V in fragment order (V as scaled fp16)
    void* aws = at<void>(ws, w.attn_off);
    u16* kf = at<u16>(aws, w.attn.kf);
    u16* vf = at<u16>(aws, w.attn.vf);
    if (!nsa::launch_tile_cmp(s.dk, s.dv, static_cast<const u16*>(K), static_cast<const u16*>(V),
                              at<uint32_t>(aws, w.attn.vmax), at<int>(aws, w.attn.vexp), kf, vf, s.B * s.Hkv, s.T,
                              w.attn.tpad, hs))
        return fail(NSA_ERR_UNSUPPORTED, "no layout kernel");
    nsa::AttnParams ap{};
    ap.Q = static_cast<const u16*>(Q);
    ap.Kf = kf;
    ap.Vf = vf;
    ap.vexp = at<int>(aws, w.attn.vexp);
    ap.sel = sel;
    ap.o_cmp = oc;
    ap.gates = gate_logits;
    ap.O = static_cast<u16*>(O);
    ap.B = s.B; ap.T = s.T; ap.Tpad = w.attn.tpad; ap.Hkv = s.Hkv; ap.G = s.G; ap.lp = s.lp; ap.top_n = s.n;
    ap.window = s.w; ap.branches = s.br;
    ap.scale_log2 = s.scale * nsa::kLog2eHost;
    if (s.n_cmp == 0) {   // the lists are ready: steps a5-a7 alone
        if (!nsa::launch_sparse_attn(s.dk, s.dv, ap, s.B, hs)) return fail(NSA_ERR_UNSUPPORTED, "no attention kernel");
    } else if (!nsa::launch_prefill_fused(s.dk, s.dv, s.G, sp, ap, hs)) {
        return fail(NSA_ERR_UNSUPPORTED, "no fused prefill kernel for this shape");
    }
    return hip_check("prefill_fwd");
}

nsa_status nsa_compress_prepare(const nsa_config* cfg, const void* W_k, const void* W_v, const void* pe_k,
                                const void* pe_v, void* prep, size_t prep_bytes, void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    if (s.phi != NSA_PHI_LINEAR) return fail(NSA_ERR_UNSUPPORTED, "prepared weights exist for the linear phi only");
    if (!W_k || !W_v || !pe_k || !pe_v) return fail(NSA_ERR_NULL, "W_k, W_v, pe_k and pe_v are required");
    const CompressWs w = compress_ws(s);
    if ((st = check_ws(prep, prep_bytes, w.total)) != NSA_OK) return st;
    prepare_weights(s, w, W_k, W_v, pe_k, pe_v, prep, as_stream(stream));
    return hip_check("compress_prepare");
}

nsa_status nsa_cache_append(const nsa_config* cfg, const void* K_new, const void* V_new, int32_t n_new,
                            void* K_cache, void* V_cache, int32_t* cache_len, void* K_cmp_cache, void* V_cmp_cache,
                            const void* prep, size_t prep_bytes, void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    if (s.phi != NSA_PHI_LINEAR) return fail(NSA_ERR_UNSUPPORTED, "cache maintenance implements the linear phi");
    if (!K_new || !V_new || !K_cache || !V_cache || !cache_len || !prep)
        return fail(NSA_ERR_NULL, "new tokens, caches, cache_len and the prepared weights are required");
    if (s.n_cmp > 0 && (!K_cmp_cache || !V_cmp_cache)) return fail(NSA_ERR_NULL, "compressed caches are required");
    if (n_new < 1 || n_new > s.T) return fail(NSA_ERR_SHAPE, "n_new must be in [1, capacity]");
    const CompressWs w = compress_ws(s);
    if ((st = check_ws(const_cast<void*>(prep), prep_bytes, w.total)) != NSA_OK) return st;
    if ((st = check_align16(K_new, "K_new")) != NSA_OK || (st = check_align16(V_new, "V_new")) != NSA_OK ||
        (st = check_align16(K_cache, "K_cache")) != NSA_OK || (st = check_align16(V_cache, "V_cache")) != NSA_OK)
        return st;
    using nsa::u16;
    nsa::AppendParams p{};
    p.K_new = static_cast<const u16*>(K_new);
    p.V_new = static_cast<const u16*>(V_new);
    p.K_cache = static_cast<u16*>(K_cache);
    p.V_cache = static_cast<u16*>(V_cache);
    p.cache_len = cache_len;
    p.wt_k = at<const u16>(const_cast<void*>(prep), w.wt_k);
    p.wt_v = at<const u16>(const_cast<void*>(prep), w.wt_v);
    p.bias_k = at<const float>(const_cast<void*>(prep), w.bias_k);
    p.bias_v = at<const float>(const_cast<void*>(prep), w.bias_v);
    p.K_cmp = static_cast<u16*>(K_cmp_cache);
    p.V_cmp = static_cast<u16*>(V_cmp_cache);
    p.B = s.B; p.Hkv = s.Hkv; p.L = s.T; p.dk = s.dk; p.dv = s.dv; p.l = s.l; p.s = s.s; p.N = s.n_cmp;
    p.n_new = n_new;
    p.R = nsa::append_rows_per_group(n_new, s.s);
    nsa::launch_cache_append(p, as_stream(stream));
    return hip_check("cache_append");
}

nsa_status nsa_full_attn_fwd(const nsa_config* cfg, const void* Q, const void* K, const void* V, void* O, void* ws,
                             size_t ws_bytes, void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    if (!Q || !K || !V || !O) return fail(NSA_ERR_NULL, "Q, K, V and O are required");
    const FullWs w = full_ws(s);
    if ((st = check_ws(ws, ws_bytes, w.total)) != NSA_OK) return st;
    const hipStream_t hs = as_stream(stream);
    using nsa::u16;
    u16* kf = at<u16>(ws, w.kf);
    u16* vf = at<u16>(ws, w.vf);
    if (!nsa::launch_tile_cmp(s.dk, s.dv, static_cast<const u16*>(K), static_cast<const u16*>(V),
                              at<uint32_t>(ws, w.vmax), at<int>(ws, w.vexp), kf, vf, s.B * s.Hkv, s.T, w.tpad, hs))
        return fail(NSA_ERR_UNSUPPORTED, "no layout kernel for this shape");
    nsa::FullParams p{};
    p.Q = static_cast<const u16*>(Q);
    p.Kf = kf;
    p.Vf = vf;
    p.vexp = at<int>(ws, w.vexp);
    p.O = static_cast<u16*>(O);
    p.B = s.B; p.T = s.T; p.Tpad = w.tpad; p.Hkv = s.Hkv;
    p.scale_log2 = s.scale * nsa::kLog2eHost;
    if (!nsa::launch_full_attn(s.dk, s.dv, s.G, p, hs)) return fail(NSA_ERR_UNSUPPORTED, "no dense attention kernel");
    return hip_check("full_attn");
}

}  // extern "C"

namespace {
// nsa_decode with its scratch either from the caller's workspace or, with ws == nullptr and
// use_static, from the library's fixed per-device scratch array.
nsa_status decode_impl(const nsa_config* cfg, const void* q, const void* K_cache, const void* V_cache,
                       const int32_t* cache_len, const void* K_cmp_cache, const void* V_cmp_cache,
                       const float* gate_logits, void* O, int32_t* sel_idx_out, void* ws, size_t ws_bytes,
                       bool use_static, void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    if (!q || !K_cache || !V_cache || !cache_len || !O) return fail(NSA_ERR_NULL, "q, caches, cache_len and O are required");
    if (s.mode != NSA_SCORE_CMP_OVERLAP || s.phi != NSA_PHI_LINEAR)
        return fail(NSA_ERR_UNSUPPORTED, "decode implements the NSA (linear phi, compressed-overlap) mode");
    if (s.n_cmp == 0) return fail(NSA_ERR_UNSUPPORTED, "cache capacity shorter than cmp_block");
    if (!K_cmp_cache || !V_cmp_cache) return fail(NSA_ERR_NULL, "compressed caches are required");
    if ((s.br & NSA_BR_WIN) && s.w <= 0) return fail(NSA_ERR_SHAPE, "window branch with window = 0");
    if (s.n_slc > 64 * 32) return fail(NSA_ERR_UNSUPPORTED, "at most 2048 selection blocks");
    const DecodeWs w = decode_ws(s);
    if (w.n_items - s.n > nsa::kDecodeMaxItems)
        return fail(NSA_ERR_UNSUPPORTED, "decode supports windows up to " +
                                             std::to_string(64 * (nsa::kDecodeMaxItems - 2)) + " tokens");
    if (s.lp / s.s + s.l / s.s - 1 > nsa::kDecodeSplitKeys)
        return fail(NSA_ERR_UNSUPPORTED, "decode needs (slc_block + cmp_block) / cmp_stride - 1 <= " +
                                             std::to_string(nsa::kDecodeSplitKeys));
    if (w.n_split > nsa::kDecodeMaxSplits)
        return fail(NSA_ERR_UNSUPPORTED, "decode supports at most " +
                                             std::to_string(nsa::kDecodeMaxSplits * nsa::kDecodeSplitKeys) +
                                             " compressed keys");
    if (use_static) {
        if (w.total > nsa::static_scratch_bytes())
            return fail(NSA_ERR_WORKSPACE, "decode needs " + std::to_string(w.total) +
                                               " bytes of scratch; the allocation-free entry point has " +
                                               std::to_string(nsa::static_scratch_bytes()));
        hipError_t e = hipSuccess;
        ws = nsa::static_scratch(&e);
        if (!ws) return fail(NSA_ERR_HIP, std::string("scratch address: ") + hipGetErrorString(e));
        ws_bytes = nsa::static_scratch_bytes();
    }
    if ((st = check_ws(ws, ws_bytes, w.total)) != NSA_OK) return st;
    using nsa::u16;
    nsa::DecodeParams p{};
    p.q = static_cast<const u16*>(q);
    p.K = static_cast<const u16*>(K_cache);
    p.V = static_cast<const u16*>(V_cache);
    p.cache_len = cache_len;
    p.Kc = static_cast<const u16*>(K_cmp_cache);
    p.Vc = static_cast<const u16*>(V_cmp_cache);
    p.gates = gate_logits;
    p.O = static_cast<u16*>(O);
    p.sel_out = sel_idx_out;
    p.part_m = at<float>(ws, w.pm);
    p.part_l = at<float>(ws, w.pl);
    p.part_o = at<nsa::u16>(ws, w.po);
    p.part_a = at<float>(ws, w.pa);
    p.sel_ws = at<int32_t>(ws, w.sel);
    p.cmp_w = at<float>(ws, w.cw);
    p.att_m = at<float>(ws, w.am);
    p.att_l = at<float>(ws, w.al);
    p.att_o = at<nsa::u16>(ws, w.ao);
    p.B = s.B; p.L = s.T; p.Hkv = s.Hkv; p.G = s.G; p.Nc = s.n_cmp; p.l = s.l; p.s = s.s; p.lp = s.lp;
    p.n_slc = s.n_slc; p.top_n = s.n; p.n_init = s.n_init; p.n_local = s.n_local; p.window = s.w;
    p.branches = s.br; p.n_split = w.n_split; p.jb = w.jb; p.n_items = w.n_items;
    p.scale_log2 = s.scale * nsa::kLog2eHost;
    if (!nsa::launch_decode(s.dk, s.dv, p, as_stream(stream))) return fail(NSA_ERR_UNSUPPORTED, "no decode kernel");
    return hip_check("decode");
}
}  // namespace

extern "C" {

nsa_status nsa_decode(const nsa_config* cfg, const void* q, const void* K_cache, const void* V_cache,
                      const int32_t* cache_len, const void* K_cmp_cache, const void* V_cmp_cache,
                      const float* gate_logits, void* O, int32_t* sel_idx_out, void* ws, size_t ws_bytes,
                      void* stream) {
    return decode_impl(cfg, q, K_cache, V_cache, cache_len, K_cmp_cache, V_cmp_cache, gate_logits, O, sel_idx_out,
                       ws, ws_bytes, false, stream);
}

nsa_status nsa_decode_noalloc(const nsa_config* cfg, const void* q, const void* K_cache, const void* V_cache,
                              const int32_t* cache_len, const void* K_cmp_cache, const void* V_cmp_cache,
                              const float* gate_logits, void* O, int32_t* sel_idx_out, void* stream) {
    return decode_impl(cfg, q, K_cache, V_cache, cache_len, K_cmp_cache, V_cmp_cache, gate_logits, O, sel_idx_out,
                       nullptr, 0, true, stream);
}

nsa_status nsa_sparse_attn_bwd(const nsa_config* cfg, const void* Q, const void* K, const void* V,
                               const void* K_cmp, const void* V_cmp, const int32_t* sel_idx, const float* lse_cmp,
                               const float* o_cmp, const float* gate_logits, const float* saved_lse,
                               const float* saved_o, const void* dO, float* dQ, float* dK, float* dV,
                               float* dK_cmp, float* dV_cmp, float* d_gate_logits, void* ws, size_t ws_bytes,
                               void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    if (!Q || !K || !V || !dO || !dQ || !dK || !dV) return fail(NSA_ERR_NULL, "Q, K, V, dO, dQ, dK and dV are required");
    if ((s.br & NSA_BR_SLC) && !sel_idx) return fail(NSA_ERR_NULL, "sel_idx is required for the selected branch");
    if ((s.br & NSA_BR_CMP) && (!K_cmp || !V_cmp || !lse_cmp || !o_cmp || !dK_cmp || !dV_cmp))
        return fail(NSA_ERR_NULL, "the compressed branch needs K_cmp, V_cmp, lse_cmp, o_cmp, dK_cmp and dV_cmp");
    if (d_gate_logits && !gate_logits) return fail(NSA_ERR_NULL, "d_gate_logits needs gate_logits");
    if ((saved_lse == nullptr) != (saved_o == nullptr)) return fail(NSA_ERR_NULL, "saved_lse and saved_o go together");
    if (saved_o && ((reinterpret_cast<uintptr_t>(saved_o) & 15u) != 0 || (reinterpret_cast<uintptr_t>(saved_lse) & 7u) != 0))
        return fail(NSA_ERR_SHAPE, "saved_o must be 16-byte and saved_lse 8-byte aligned");
    if ((s.br & NSA_BR_CMP) && (reinterpret_cast<uintptr_t>(o_cmp) & 15u) != 0)
        return fail(NSA_ERR_SHAPE, "o_cmp must be 16-byte aligned");
    if ((s.br & NSA_BR_WIN) && s.w <= 0) return fail(NSA_ERR_SHAPE, "window branch with window = 0");
    if ((long long)s.T >= (1LL << 26)) return fail(NSA_ERR_UNSUPPORTED, "sequence too long for the block lists");
    const BwdWs w = bwd_ws(s);
    if ((st = check_ws(ws, ws_bytes, w.total)) != NSA_OK) return st;
    const void* ptrs[] = {Q, K, V, dO, dQ, dK, dV};
    const char* names[] = {"Q", "K", "V", "dO", "dQ", "dK", "dV"};
    for (int i = 0; i < 7; ++i)
        if ((st = check_align16(ptrs[i], names[i])) != NSA_OK) return st;
    if ((s.br & NSA_BR_CMP) &&
        ((st = check_align16(dK_cmp, "dK_cmp")) != NSA_OK || (st = check_align16(dV_cmp, "dV_cmp")) != NSA_OK))
        return st;
    const hipStream_t hs = as_stream(stream);
    using nsa::u16;
    const size_t bg = (size_t)s.B * s.Hkv;
    const bool cmp = (s.br & NSA_BR_CMP) != 0;
    nsa::launch_fill_zero(dK, bg * s.T * s.dk, hs);
    nsa::launch_fill_zero(dV, bg * s.T * s.dv, hs);
    if (cmp) {
        nsa::launch_fill_zero(dK_cmp, bg * s.n_cmp * s.dk, hs);
        nsa::launch_fill_zero(dV_cmp, bg * s.n_cmp * s.dv, hs);
    }
    // 1. per-row statistics: from the training forward's saved outputs, or the forward's
    //    selected and window branches recomputed
    u16* kf = at<u16>(ws, w.kf);
    u16* vf = at<u16>(ws, w.vf);
    if (!saved_o && !nsa::launch_tile_cmp(s.dk, s.dv, static_cast<const u16*>(K), static_cast<const u16*>(V),
                                          at<uint32_t>(ws, w.vmax), at<int>(ws, w.vexp), kf, vf, (int)bg, s.T, w.tpad,
                                          hs))
        return fail(NSA_ERR_UNSUPPORTED, "no layout kernel");
    nsa::AttnParams a{};
    a.Q = static_cast<const u16*>(Q);
    a.Kf = kf;
    a.Vf = vf;
    a.vexp = at<int>(ws, w.vexp);
    a.sel = sel_idx;
    a.o_cmp = o_cmp;
    a.gates = gate_logits;
    a.lse_cmp = lse_cmp;
    a.dO = static_cast<const u16*>(dO);
    a.stats = at<float>(ws, w.stats);
    a.dgates = d_gate_logits;
    a.B = s.B; a.T = s.T; a.Tpad = w.tpad; a.Hkv = s.Hkv; a.G = s.G; a.lp = s.lp; a.top_n = s.n; a.window = s.w;
    a.branches = s.br;
    a.scale_log2 = s.scale * nsa::kLog2eHost;
    a.saved_lse = const_cast<float*>(saved_lse);
    a.saved_o = const_cast<float*>(saved_o);
    if (saved_o) nsa::launch_stats_from_saved(s.dv, a, hs);
    else if (!nsa::launch_sparse_attn_stats(s.dk, s.dv, a, hs))
        return fail(NSA_ERR_UNSUPPORTED, "no statistics kernel");
    // 2. dQ
    nsa::BwdParams p{};
    p.Q = static_cast<const u16*>(Q);
    p.K = static_cast<const u16*>(K);
    p.V = static_cast<const u16*>(V);
    p.Kc = static_cast<const u16*>(K_cmp);
    p.Vc = static_cast<const u16*>(V_cmp);
    p.sel = sel_idx;
    p.dO = static_cast<const u16*>(dO);
    p.stats = a.stats;
    p.dQ = dQ; p.dK = dK; p.dV = dV; p.dKc = dK_cmp; p.dVc = dV_cmp;
    p.B = s.B; p.T = s.T; p.Hkv = s.Hkv; p.G = s.G; p.N = s.n_cmp; p.l = s.l; p.s = s.s; p.lp = s.lp; p.top_n = s.n;
    p.window = s.w; p.branches = s.br; p.n_slc = s.n_slc;
    p.scale = s.scale;
    p.scale_log2 = s.scale * nsa::kLog2eHost;
    if (!nsa::launch_bwd_dq(s.dk, s.dv, p, hs)) return fail(NSA_ERR_UNSUPPORTED, "no dQ kernel");
    // 3. block lists of the selected branch
    long long n_slc_items = 0;
    if (s.br & NSA_BR_SLC) {
        nsa::MobaParams m{};
        m.sel = sel_idx;
        m.hist = at<int>(ws, w.hist);
        m.bucket_cnt = at<int>(ws, w.bcnt);
        m.bucket_start = at<int>(ws, w.bstart);
        m.tile_start = at<int>(ws, w.tstart);
        m.tile_bucket = at<int>(ws, w.tbk);
        m.entries = at<int>(ws, w.entries);
        m.B = s.B; m.T = s.T; m.Hkv = s.Hkv; m.lp = s.lp; m.n_slc = s.n_slc; m.top_n = s.n;
        m.n_chunk = w.n_chunk; m.n_bucket = w.n_bucket; m.keep_own = 1;
        nsa::launch_block_lists(m, hs);
        p.bucket_start = m.bucket_start;
        p.tile_start = m.tile_start;
        p.tile_bucket = m.tile_bucket;
        p.entries = m.entries;
        p.n_bucket = w.n_bucket;
        p.nsb = (s.lp + 16 * nsa::kDkvWavesSlc - 1) / (16 * nsa::kDkvWavesSlc);
        n_slc_items = (long long)nsa::moba_max_tiles((int)bg, s.T, s.n, s.n_slc) * p.nsb;
    }
    // 4. dK, dV, dK_cmp, dV_cmp
    const int dense_keys = 16 * nsa::kDkvWavesDense * nsa::kDkvTilesDense;
    p.qt_cmp = nsa::kBwdCmpTile;
    p.n_qt = (s.T + p.qt_cmp - 1) / p.qt_cmp;
    p.n_kb_cmp = cmp ? (s.n_cmp + dense_keys - 1) / dense_keys : 0;
    p.n_kb_win = (s.br & NSA_BR_WIN) ? (s.T + dense_keys - 1) / dense_keys : 0;
    p.n_qt_win = (dense_keys + s.w - 1 + nsa::kBwdTile - 1) / nsa::kBwdTile;
    const long long n_dense = (long long)bg * p.n_kb_cmp * p.n_qt + (long long)bg * p.n_kb_win * p.n_qt_win;
    if (n_dense + n_slc_items >= (1LL << 31)) return fail(NSA_ERR_SHAPE, "problem too large");
    p.n_cmp_items = (int)(bg * p.n_kb_cmp * p.n_qt);
    p.n_win_items = (int)(bg * p.n_kb_win * p.n_qt_win);
    if (!nsa::launch_bwd_dkv(s.dk, s.dv, p, (int)n_slc_items, hs)) return fail(NSA_ERR_UNSUPPORTED, "no dK/dV kernel");
    return hip_check("sparse_attn_bwd");
}

nsa_status nsa_compress_bwd(const nsa_config* cfg, const void* K, const void* V, const void* W_k, const void* W_v,
                            const void* pe_k, const void* pe_v, const float* dK_cmp, const float* dV_cmp, float* dK,
                            float* dV, float* dW_k, float* dW_v, float* dpe_k, float* dpe_v, void* ws,
                            size_t ws_bytes, void* stream) {
    g_detail.clear();
    Shape s;
    nsa_status st = check_config(cfg, &s);
    if (st != NSA_OK) return st;
    if (s.phi != NSA_PHI_LINEAR) return fail(NSA_ERR_UNSUPPORTED, "the block-map backward implements the linear phi");
    if (!K || !V || !W_k || !W_v || !pe_k || !pe_v || !dK_cmp || !dV_cmp || !dK || !dV || !dW_k || !dW_v || !dpe_k ||
        !dpe_v)
        return fail(NSA_ERR_NULL, "every argument is required");
    if ((st = check_ws(ws, ws_bytes, compress_bwd_ws(s))) != NSA_OK) return st;
    const void* ptrs[] = {dW_k, dW_v, dpe_k, dpe_v};
    const char* names[] = {"dW_k", "dW_v", "dpe_k", "dpe_v"};
    for (int i = 0; i < 4; ++i)
        if ((st = check_align16(ptrs[i], names[i])) != NSA_OK) return st;
    const hipStream_t hs = as_stream(stream);
    using nsa::u16;
    const int BG = s.B * s.Hkv;
    float* ck = at<float>(ws, 0);
    float* cv = at<float>(ws, align_up((size_t)s.dk * 4, 256));
    nsa::launch_compress_bwd(static_cast<const u16*>(K), static_cast<const u16*>(W_k), static_cast<const u16*>(pe_k),
                             dK_cmp, dK, dW_k, dpe_k, ck, BG, s.T, s.n_cmp, s.dk, s.l, s.s, hs);
    nsa::launch_compress_bwd(static_cast<const u16*>(V), static_cast<const u16*>(W_v), static_cast<const u16*>(pe_v),
                             dV_cmp, dV, dW_v, dpe_v, cv, BG, s.T, s.n_cmp, s.dv, s.l, s.s, hs);
    return hip_check("compress_bwd");
}

const char* nsa_status_string(nsa_status status) {
    switch (status) {
        case NSA_OK: return "ok";
        case NSA_ERR_NULL: return "required pointer is NULL";
        case NSA_ERR_SHAPE: return "inconsistent or invalid sizes";
        case NSA_ERR_UNSUPPORTED: return "shape not implemented by the library's kernels";
        case NSA_ERR_WORKSPACE: return "workspace missing or too small";
        case NSA_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

const char* nsa_last_error_detail(void) { return g_detail.c_str(); }

}  // extern "C"
