/*
 * nsa.h - C ABI of an MI355X (gfx950) library for the forward pass of Native Sparse
 * Attention (NSA) and of the MoBA-style mean-pooled block selection.
 *
 * What the operations compute (the pages give the method in prose only):
 *   - youtublog.net, "Songlin Yang explains attention mechanisms from DeepSeek, Kimi and
 *     MiniMax" (English page): attention weights the values by a softmax of query/key
 *     scores over the keys a query may access, with a causal mask; NSA has three
 *     branches - coarse attention over compressed blocks, fine attention over a few
 *     selected blocks, a sliding window - mixed by learned gates; the heads of a GQA
 *     group aggregate their scores and share one selection; MoBA represents a block by
 *     mean pooling and lets each head select its own blocks.
 *   - zjai.club episode notes, section 5 (each contiguous KV block compressed to one key
 *     and one value; block scores pick the top-k blocks, whose tokens get token-level
 *     attention; the window attends to nearby tokens), section 6 (a gate computed from
 *     the current token scales each branch output, and the three are added), section 8
 *     (scores summed over the group's heads, then one top-k), section 13 (decoding is
 *     memory-bound: its cost is the KV bytes read per step), sections 16-17 (MoBA:
 *     mean-pooled block keys, query-mean inner product as the score, 512-token blocks,
 *     top 3).
 *   - sunshychen.top MoBA/NSA comparison: the query's own block is always attended and
 *     causally masked; with fixed block sizes the compressed attention scores serve
 *     directly as selection scores; the NSA window crosses block boundaries.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers.  bf16 tensors are raw 16-bit patterns.
 *   - Layouts (row-major, last index fastest), with H = num_kv_heads * heads_per_group
 *     and query head h = g * heads_per_group + i belonging to KV group g:
 *       Q, O            [B, T, H, d]           (prefill)
 *       K, V            [B, H_kv, T, d]        (also the decode caches, T = capacity)
 *       K_cmp, V_cmp    [B, H_kv, N_cmp, d]    N_cmp = floor((T - l)/s) + 1
 *       sel_idx         [B, T, H_kv, top_n]    int32, ascending, padded with -1
 *       gate_logits     [B, T, H, 3]           fp32, order (compressed, selected, window)
 *       o_cmp, lse_cmp  [B, T, H, d_v], [B, T, H]   fp32
 *   - The caller owns every buffer.  The library never allocates device memory; calls
 *     that need scratch take a caller workspace whose size nsa_workspace_size reports
 *     (nsa_decode_noalloc instead uses a fixed device array the library holds).
 *   - Calls are asynchronous on the given stream (a hipStream_t; NULL = default stream)
 *     and never synchronize.  Inputs are read-only; outputs are fully overwritten.
 *   - Arguments are validated on the host before anything is launched; a failing call
 *     launches nothing and returns a status (details: nsa_last_error_detail).
 *   - Calls on different streams with disjoint outputs and workspaces may overlap.
 */
#ifndef NSA_H
#define NSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NSA_OK = 0,
    NSA_ERR_NULL = 1,          /* a required pointer is NULL */
    NSA_ERR_SHAPE = 2,         /* sizes are inconsistent or non-positive */
    NSA_ERR_UNSUPPORTED = 3,   /* a shape the library's kernels do not implement */
    NSA_ERR_WORKSPACE = 4,     /* workspace NULL or smaller than nsa_workspace_size */
    NSA_ERR_HIP = 5            /* a HIP launch failed (see nsa_last_error_detail) */
} nsa_status;

/* Block representation (step "compress"). */
typedef enum {
    NSA_PHI_LINEAR = 0,   /* cmp[i] = vec(X[i*s : i*s+l] + PE) . W  (NSA) */
    NSA_PHI_MEAN = 1      /* cmp[i] = mean of X[i*s : i*s+l]         (MoBA) */
} nsa_phi;

/* Block score used for selection. */
typedef enum {
    NSA_SCORE_CMP_OVERLAP = 0, /* sum over the group's heads and over the compressed blocks
                                  overlapping the block of the compressed attention
                                  probabilities (NSA) */
    NSA_SCORE_MEAN_DOT = 1     /* sum over the group's heads of <q, mean key of the block>
                                  over complete earlier blocks (MoBA; needs l = s = l') */
} nsa_score_mode;

/* Branch bits for nsa_config.branches. */
enum { NSA_BR_CMP = 1, NSA_BR_SLC = 2, NSA_BR_WIN = 4 };

/* Work items for nsa_workspace_size. */
enum { NSA_OP_COMPRESS = 0, NSA_OP_SCORE_SELECT = 1, NSA_OP_SPARSE_ATTN = 2, NSA_OP_DECODE = 3,
       NSA_OP_FULL_ATTN = 4, NSA_OP_SPARSE_BWD = 5, NSA_OP_COMPRESS_BWD = 6, NSA_OP_PREFILL = 7 };

typedef struct nsa_config {
    uint32_t struct_size;      /* sizeof(nsa_config) */
    int32_t batch;             /* B */
    int32_t seq_len;           /* T (prefill) or cache capacity L (decode) */
    int32_t num_kv_heads;      /* H_kv: KV heads = GQA groups */
    int32_t heads_per_group;   /* G: query heads sharing one KV head (1, 2, 4, 8 or 16) */
    int32_t d_k;               /* query/key head dim (64, 128 or 192) */
    int32_t d_v;               /* value head dim (64 or 128) */
    int32_t cmp_block;         /* l: tokens per compressed block */
    int32_t cmp_stride;        /* s: stride between compressed blocks (s | l, s | l') */
    int32_t slc_block;         /* l': tokens per selection block (multiple of 32) */
    int32_t top_n;             /* n: selected blocks per (query, group), forced ones included (<= 32) */
    int32_t n_init;            /* blocks 0 .. n_init-1 are always selected */
    int32_t n_local;           /* the n_local blocks ending at the query's own block are always selected */
    int32_t window;            /* w: sliding-window length including the query (0 = no window) */
    int32_t phi;               /* nsa_phi */
    int32_t score_mode;        /* nsa_score_mode */
    int32_t branches;          /* OR of NSA_BR_* */
    float softmax_scale;       /* <= 0 selects 1/sqrt(d_k) (MEAN_DOT scores are never scaled) */
} nsa_config;

/* Bytes of workspace `op` needs for this configuration (0 is possible). */
nsa_status nsa_workspace_size(const nsa_config* cfg, int op, size_t* bytes);

/* Step "compress": one key (and, for NSA_PHI_LINEAR, one value) per block of l tokens
 * taken every s tokens (zjai.club notes, section 5; MoBA mean pooling, section 16).
 *   NSA_PHI_LINEAR: K_cmp[b,g,i,:] = sum_{r<l, e<d_k} (K[b,g,i*s+r,e] + pe_k[r,e]) * W_k[r*d_k+e, :]
 *                   and the same for V with W_v [l*d_v, d_v] and pe_v [l, d_v].
 *                   W_k [l*d_k, d_k] and pe_k [l, d_k] are bf16 and shared by all KV heads.
 *   NSA_PHI_MEAN:   K_cmp[b,g,i,:] = (1/l) * sum_{r<l} K[b,g,i*s+r,:]; V, W_*, pe_*, V_cmp unused.
 * Accumulates in fp32 and rounds once to bf16.  Works for the decode caches too (T = L).
 * With T < l there is no block: nothing is written and every pointer may be NULL. */
nsa_status nsa_compress(const nsa_config* cfg, const void* K, const void* V,
                        const void* W_k, const void* W_v, const void* pe_k, const void* pe_v,
                        void* K_cmp, void* V_cmp, void* ws, size_t ws_bytes, void* stream);

/* Steps "compressed attention, block scores, selection" (zjai.club notes, sections 5 and 8;
 * sunshychen.top: compressed scores reused as selection scores).
 * NSA_SCORE_CMP_OVERLAP: for query t and head h, compressed block i is visible when
 *   i*s + l - 1 <= t; p = softmax(scale * q . K_cmp) over visible blocks;
 *   lse_cmp = log sum exp (-inf when nothing is visible);
 *   o_cmp = sum_i p_i V_cmp[i] (0 when nothing is visible);
 *   score[j] = sum over the group's heads and visible i whose tokens intersect block j of p_i.
 * NSA_SCORE_MEAN_DOT: score[j] = sum over the group's heads of q . K_cmp[j] for j < t / l'.
 * Selection (both modes): with jc = t / l', the forced blocks are 0..n_init-1 and
 *   jc-n_local+1..jc (within 0..jc); the other blocks 0..jc are taken by descending score,
 *   ties to the lower index, until min(top_n, jc+1) blocks are chosen.
 * Outputs: sel_idx (required); lse_cmp and o_cmp optional (NULL = not produced; o_cmp
 *   needs V_cmp; both must be NULL in MEAN_DOT mode).  Scores are fp32.
 * With T < l no compressed block exists (K_cmp / V_cmp may be NULL): o_cmp = 0, lse_cmp =
 *   -inf, every score 0, so the rows hold the forced blocks and, in any other slot, the
 *   lowest eligible indices. */
nsa_status nsa_score_select(const nsa_config* cfg, const void* Q, const void* K_cmp,
                            const void* V_cmp, int32_t* sel_idx, float* lse_cmp, float* o_cmp,
                            void* ws, size_t ws_bytes, void* stream);

/* Selection alone, from caller scores [B, T, H_kv, N_slc] fp32 (N_slc = ceil(T / l')),
 * with the rule of nsa_score_select.  For custom block scores; also exercises the top-n
 * stage in isolation. */
nsa_status nsa_select_from_scores(const nsa_config* cfg, const float* scores, int32_t* sel_idx,
                                  void* stream);

/* Steps "selected attention, sliding window, gated sum" (zjai.club notes, sections 5-6;
 * sunshychen.top: the window crosses block boundaries, the query's own block is causal).
 *   o_slc = softmax(scale * q . K) . V over tokens of the listed blocks that are <= t;
 *   o_win = the same over tokens max(0, t-w+1) .. t;
 *   O = sum over enabled branches of sigmoid(z_branch) * o_branch, with o_cmp taken from the
 *   caller (as produced by nsa_score_select) when NSA_BR_CMP is set.
 * sel_idx rows must list distinct blocks <= t / l' in ascending order, padded with -1 at the
 * end (as nsa_score_select writes them).  gate_logits NULL = weight 1.
 * O is bf16 [B, T, H, d_v].  Values: any bf16 magnitude (V's fp16 copy is scaled per
 * sequence and group by a power of two; the MoBA schedule's fp16 partials stay in those
 * scaled units). */
nsa_status nsa_sparse_attn_fwd(const nsa_config* cfg, const void* Q, const void* K, const void* V,
                               const int32_t* sel_idx, const float* o_cmp, const float* gate_logits,
                               void* O, void* ws, size_t ws_bytes, void* stream);

/* Steps "compressed attention, block scores, selection, selected attention, sliding window,
 * gated sum" in one call: nsa_score_select followed by nsa_sparse_attn_fwd (zjai.club notes,
 * sections 5, 6 and 8; sunshychen.top: compressed scores reused as selection scores), run as
 * one fused launch whose workgroups each score, select and attend their own tile of tokens.
 * Same arithmetic and results as the two calls, bit for bit.
 *   Inputs: Q [B,T,H,d_k], K [B,H_kv,T,d_k], V [B,H_kv,T,d_v], K_cmp / V_cmp [B,H_kv,N_cmp,d]
 *   (from nsa_compress) bf16; gate_logits [B,T,H,3] fp32 (NULL = weight 1).
 *   Outputs: O [B,T,H,d_v] bf16 (required); sel_idx [B,T,H_kv,top_n] int32, lse_cmp [B,T,H]
 *   and o_cmp [B,T,H,d_v] fp32 are optional (NULL = kept in the workspace / not written).
 *   Workspace: nsa_workspace_size(cfg, NSA_OP_PREFILL).
 * Needs the compressed-overlap scores (NSA_SCORE_CMP_OVERLAP); every branch mask is allowed
 * (the compressed branch's output is formed in any case: the scores need it).  With T < l
 * (no compressed block; K_cmp / V_cmp may be NULL) the call runs the two calls' no-block
 * path.  Errors as for the two calls; NSA_ERR_UNSUPPORTED for the MEAN_DOT scores. */
nsa_status nsa_prefill_fwd(const nsa_config* cfg, const void* Q, const void* K, const void* V, const void* K_cmp,
                           const void* V_cmp, const float* gate_logits, void* O, int32_t* sel_idx, float* lse_cmp,
                           float* o_cmp, void* ws, size_t ws_bytes, void* stream);

/* One decode step (zjai.club notes, section 13): every sequence b has one new query at
 * position t_b = cache_len[b] - 1 whose K/V are already in the caches; K_cmp_cache /
 * V_cmp_cache hold the compressed blocks of the cache (nsa_compress over the cache).
 * Computes exactly the prefill result for row t_b: compressed branch, scores, selection,
 * selected and window branches, gated sum.
 *   q [B, H, d_k] bf16; caches [B, H_kv, L, d] bf16; compressed caches [B, H_kv, N_cmp(L), d];
 *   cache_len [B] int32 device array (1 <= cache_len <= L); gate_logits [B, H, 3] (NULL = 1);
 *   O [B, H, d_v] bf16; sel_idx_out [B, H_kv, top_n] (optional).
 * Partial outputs pass through fp16 normalized by their softmax sums: |V| and |V_cmp| must
 * stay below 65504.
 * NSA_ERR_UNSUPPORTED for a mode other than linear phi with compressed-overlap scores, more
 * than 8192 compressed keys, top_n > 32, windows over 1920 tokens, or
 * (slc_block + cmp_block) / cmp_stride - 1 > 256. */
nsa_status nsa_decode(const nsa_config* cfg, const void* q, const void* K_cache, const void* V_cache,
                      const int32_t* cache_len, const void* K_cmp_cache, const void* V_cmp_cache,
                      const float* gate_logits, void* O, int32_t* sel_idx_out,
                      void* ws, size_t ws_bytes, void* stream);

/* nsa_decode without a workspace, for callers that cannot allocate device memory (work
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, kernels and results as nsa_decode, minus ws / ws_bytes: the scratch comes from
 * a fixed 64 MiB array in device memory that the library holds on every GPU it runs on
 * until the process ends (the B = 32, 65536-token decode step uses 30 MiB; nsa_workspace_size
 * with NSA_OP_DECODE gives any configuration's need).  The call allocates and frees nothing.
 * Errors: those of nsa_decode, NSA_ERR_WORKSPACE when the configuration needs more scratch
 * than the array holds, NSA_ERR_HIP when the array's device address cannot be obtained.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must be serialized by the caller.
 * Nothing in the array needs clearing between calls (every value read is written earlier in
 * the same call). */
nsa_status nsa_decode_noalloc(const nsa_config* cfg, const void* q, const void* K_cache, const void* V_cache,
                              const int32_t* cache_len, const void* K_cmp_cache, const void* V_cmp_cache,
                              const float* gate_logits, void* O, int32_t* sel_idx_out, void* stream);

/* Decode cache maintenance (zjai.club notes, section 5: the compressed cache gains one entry
 * every s tokens; section 13: decoding runs against these caches).
 *
 * nsa_compress_prepare writes the transposed linear maps and the position-embedding biases
 * vec(pe) . W of both maps into `prep` (nsa_workspace_size(cfg, NSA_OP_COMPRESS) bytes,
 * 256-byte aligned, caller-owned); prepare once per set of weights, reuse for every append.
 * NSA_PHI_LINEAR only.
 *
 * nsa_cache_append appends n_new tokens per sequence: K_new [B, H_kv, n_new, d_k] and V_new
 * [B, H_kv, n_new, d_v] (bf16) go to K_cache / V_cache [B, H_kv, L, d] at positions
 * cache_len[b] .. cache_len[b] + n_new - 1, and every compressed block whose last token is
 * one of them is written to K_cmp_cache / V_cmp_cache [B, H_kv, N_cmp(L), d] with the
 * arithmetic of nsa_compress (the result equals nsa_compress over the grown cache, bit for
 * bit).  Then cache_len[b] += n_new on the device, so a following nsa_decode on the same
 * stream sees the new lengths.  Tokens that would land at or past L are dropped (cache_len
 * saturates at L); the caller keeps cache_len[b] + n_new <= L.  Raw caches and new tokens
 * must be 16-byte aligned.  Errors: NSA_ERR_SHAPE for n_new outside [1, L] or a misaligned array,
 * NSA_ERR_UNSUPPORTED for a non-linear phi, NSA_ERR_WORKSPACE for a short or unaligned prep. */
nsa_status nsa_compress_prepare(const nsa_config* cfg, const void* W_k, const void* W_v, const void* pe_k,
                                const void* pe_v, void* prep, size_t prep_bytes, void* stream);
nsa_status nsa_cache_append(const nsa_config* cfg, const void* K_new, const void* V_new, int32_t n_new,
                            void* K_cache, void* V_cache, int32_t* cache_len, void* K_cmp_cache, void* V_cmp_cache,
                            const void* prep, size_t prep_bytes, void* stream);

/* Dense causal attention, the computation NSA is compared against (zjai.club notes, summary
 * bullets and section 13: a full-attention kernel written the same way as the NSA kernel):
 *   O[b,t,h,:] = softmax(scale * q . K[b,g,x,:] over x = 0..t) . V[b,g,x,:],  g = h / G.
 * cfg must be a valid configuration; only batch, seq_len, num_kv_heads, heads_per_group, d_k,
 * d_v and softmax_scale are used (workspace: nsa_workspace_size with NSA_OP_FULL_ATTN).
 * Q [B, T, H, d_k], K [B, H_kv, T, d_k], V [B, H_kv, T, d_v] bf16; O bf16 [B, T, H, d_v].
 * Probabilities enter the value product in fp16 against an fp16 copy of V scaled by a power
 * of two per (b, g) (workspace). */
nsa_status nsa_full_attn_fwd(const nsa_config* cfg, const void* Q, const void* K, const void* V, void* O,
                             void* ws, size_t ws_bytes, void* stream);

/* Backward of the three branches and the gated sum (zjai.club notes, section 4: the method
 * is trained natively, forward and backward; section 14: the top-k choice has no derivative,
 * so sel_idx is held fixed and the compressed branch's output carries the gradient into the
 * compressed keys and values).  For the upstream gradient dO of O (the gated sum returned by
 * nsa_sparse_attn_fwd for the same inputs), with sigma_c = sigmoid(gate logit c) (1 without
 * gates) and, per branch, p = softmax(scale q.k) over that branch's keys and o_c its output:
 *   dq += scale sum_k p_k (sigma_c <dO, v_k> - sigma_c <dO, o_c>) k_k   (the same factor times q
 *   goes to dk_k), dv_k += sigma_c p_k dO, d_gate_c = sigma_c (1 - sigma_c) <dO, o_c>.
 * Keys per branch are those of the forward: compressed blocks i with i*s + l - 1 <= t, tokens
 * <= t of the listed blocks, tokens t-w+1 .. t.
 * Inputs as for the forward (bf16 Q [B,T,H,d_k], K/V [B,H_kv,T,d], K_cmp/V_cmp [B,H_kv,N,d],
 * sel_idx [B,T,H_kv,top_n], gate_logits [B,T,H,3] fp32 or NULL) plus lse_cmp [B,T,H] and o_cmp
 * [B,T,H,d_v] fp32 as written by nsa_score_select, optionally saved_lse / saved_o from
 * nsa_sparse_attn_fwd_train (NULL: the two branches' statistics are recomputed), and dO bf16
 * [B,T,H,d_v].
 * Outputs, fp32, overwritten: dQ [B,T,H,d_k], dK [B,H_kv,T,d_k], dV [B,H_kv,T,d_v], dK_cmp
 * [B,H_kv,N,d_k], dV_cmp [B,H_kv,N,d_v] (compressed branch only, else unused and may be NULL),
 * d_gate_logits [B,T,H,3] (may be NULL; zero for a disabled branch).  dK/dV hold the selected
 * and window branches' share; nsa_compress_bwd adds the compressed branch's share through the
 * block map.  Workspace: nsa_workspace_size(cfg, NSA_OP_SPARSE_BWD).  Q, K, V, dO, dQ, dK and
 * dV must be 16-byte aligned.  Key-side gradients are summed with fp32 atomics, so their
 * rounding depends on the order of the sums.  Errors: NSA_ERR_NULL for a missing required
 * pointer; NSA_ERR_SHAPE / NSA_ERR_UNSUPPORTED as for the forward, or seq_len >= 2^26. */
nsa_status nsa_sparse_attn_bwd(const nsa_config* cfg, const void* Q, const void* K, const void* V,
                               const void* K_cmp, const void* V_cmp, const int32_t* sel_idx,
                               const float* lse_cmp, const float* o_cmp, const float* gate_logits,
                               const float* saved_lse, const float* saved_o, const void* dO,
                               float* dQ, float* dK, float* dV, float* dK_cmp, float* dV_cmp,
                               float* d_gate_logits, void* ws, size_t ws_bytes, void* stream);

/* Training forward: nsa_sparse_attn_fwd (same inputs, same O) that also saves, for
 * nsa_sparse_attn_bwd, the selected and window branches' base-2 log-sum-exp
 * (saved_lse [B,T,H,2] fp32: log2 of the sum over the branch's keys of
 * 2^(scale*log2(e)*q.k), order slc, win) and normalized outputs (saved_o [B,T,H,2,d_v] fp32,
 * same order); a disabled branch saves zeros.  Both are required (NSA_ERR_NULL otherwise);
 * saved_o 16-byte and saved_lse 8-byte aligned (NSA_ERR_SHAPE).  Every configuration runs the
 * query-centric kernel here (also G = 1 with the selected branch only).  Passing both to
 * nsa_sparse_attn_bwd replaces its recompute of the two branches by a pass over the saved
 * values; either both or neither (NSA_ERR_NULL). */
nsa_status nsa_sparse_attn_fwd_train(const nsa_config* cfg, const void* Q, const void* K, const void* V,
                                     const int32_t* sel_idx, const float* o_cmp,
                                     const float* gate_logits, void* O, float* saved_lse,
                                     float* saved_o, void* ws, size_t ws_bytes, void* stream);

/* Backward of the linear block map of nsa_compress (NSA_PHI_LINEAR; zjai.club notes,
 * section 14: the loss reaches the block representations through the compressed branch).
 * For the gradients dK_cmp, dV_cmp (fp32 [B,H_kv,N,d]) of its outputs:
 *   dK[b,g,i*s+r,e] += sum_o W_k[r*d_k+e,o] dK_cmp[b,g,i,o]     (accumulated into dK; a token
 *                                                                 in several blocks sums them)
 *   dpe_k[r,e]       = sum_{b,g,i,o} W_k[r*d_k+e,o] dK_cmp[b,g,i,o]
 *   dW_k[r*d_k+e,o]  = sum_{b,g,i} (K[b,g,i*s+r,e] + pe_k[r,e]) dK_cmp[b,g,i,o]
 * and the same for V.  K, V, W_*, pe_* bf16 as for nsa_compress; dK, dV fp32 [B,H_kv,T,d]
 * (accumulated); dW_k [l*d_k,d_k], dW_v [l*d_v,d_v], dpe_k [l,d_k], dpe_v [l,d_v] fp32,
 * overwritten.  fp32 arithmetic.  dK and dV get one add per element, with no atomics (each
 * element's terms are summed by one thread); dW and dpe sum row ranges with fp32 atomics,
 * so their rounding depends on the order of those sums.  Workspace:
 * nsa_workspace_size(cfg, NSA_OP_COMPRESS_BWD).  Errors: NSA_ERR_NULL for any missing
 * pointer, NSA_ERR_UNSUPPORTED for NSA_PHI_MEAN. */
nsa_status nsa_compress_bwd(const nsa_config* cfg, const void* K, const void* V, const void* W_k,
                            const void* W_v, const void* pe_k, const void* pe_v,
                            const float* dK_cmp, const float* dV_cmp, float* dK, float* dV,
                            float* dW_k, float* dW_v, float* dpe_k, float* dpe_v, void* ws,
                            size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* nsa_status_string(nsa_status status);

/* Detail of the last failing call on this thread ("" if none). */
const char* nsa_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* NSA_H */
