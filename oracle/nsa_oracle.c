/*
 * nsa_oracle.c - plain, slow, fp64 CPU oracle of the Native Sparse Attention (NSA)
 * forward pass, its backward pass (gradients through the compression and the three
 * branches, the selection held fixed) and the MoBA-style mean-pooled block selection.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU-baseline
 * leg may load this library.  It shares no code, header, table or helper with the
 * GPU library; neither includes or links the other.
 *
 * Every function takes fp64 host arrays, works on one batch element, and loops in the
 * plainest order: no tiling, no fusion, no online softmax.  Row-parallel loops use
 * OpenMP (each row is computed independently, so threading does not change results).
 *
 * Sources, by page and section (the pages print no formulas; the steps below follow
 * their prose, and where the prose is silent the plainest reading is taken):
 *   [A] youtublog.net "Songlin Yang explains attention mechanisms..." (English page):
 *       attention = softmax of query/key scores over the keys a query may access,
 *       weighting the values; causal masking; NSA's three branches (compressed blocks,
 *       selected blocks, sliding window) mixed by learned gates; a GQA group shares
 *       one selection made from group-aggregated scores; MoBA mean-pools block keys.
 *   [B] zjai.club episode notes, section 5 (one key and one value per contiguous
 *       block; top-k blocks by block score, token-level attention inside them;
 *       sliding window over nearby tokens), section 6 (each branch output scaled by a
 *       gate computed from the current token, then summed), section 8 (scores summed
 *       over the heads of a group, then one top-k), section 16 (MoBA: mean pooling,
 *       query-mean dot product as the block score).
 *   [C] sunshychen.top MoBA/NSA comparison: the current block is always attended and
 *       causally masked; selecting every block gives full attention, selecting none
 *       gives sliding-window attention; with fixed block sizes the compressed
 *       attention scores are reused directly as selection scores; the NSA window
 *       crosses block boundaries.
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *   - phi is a linear map of the flattened block plus a learned intra-block position
 *     embedding: cmp[i] = sum_{r<l, e<d} (X[i*s + r][e] + PE[r][e]) * W[r*d + e][:].
 *   - compressed block i (tokens i*s .. i*s+l-1) is visible to query t only when all
 *     its tokens are <= t; a query with no visible block has a zero compressed output.
 *   - the selection score of block j is the sum, over the group's heads and over the
 *     compressed blocks whose token span intersects block j, of the compressed
 *     attention probabilities.
 *   - top_n counts the forced blocks: the first n_init blocks and the n_local blocks
 *     ending at the query's own block; the free slots take the highest-scoring other
 *     eligible blocks, ties to the lower block index.
 *   - the window holds the w most recent tokens including the query itself.
 *   - the gated combination is a sum sigma(z_c)*o_c over the enabled branches.
 *   - MoBA scores are the unscaled inner product of the query with the block's mean
 *     key, over the complete blocks before the query's own block.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------- */
/* Step 1: block compression                                                 */
/* ------------------------------------------------------------------------- */

/* Linear phi over each listed block i:
 *   out[b][o] = sum_{r<l} sum_{e<d} (X[(i*s + r)*d + e] + pe[r*d + e]) * W[(r*d + e)*d_out + o]
 * X: [n_tok, d] token rows of one KV head; pe: [l, d] or NULL (zero); W: [l*d, d_out].
 * blocks: block indices (must satisfy i*s + l <= n_tok); out: [nblk, d_out]. */
ORACLE_API void oracle_compress_linear(int n_tok, int d, int d_out, int l, int s,
                                       const double* X, const double* pe, const double* W,
                                       const int* blocks, int nblk, double* out)
{
    (void)n_tok;
#pragma omp parallel for schedule(dynamic)
    for (int bi = 0; bi < nblk; ++bi) {
        const int i = blocks[bi];
        double* acc = out + (size_t)bi * d_out;
        for (int o = 0; o < d_out; ++o) acc[o] = 0.0;
        for (int r = 0; r < l; ++r) {
            for (int e = 0; e < d; ++e) {
                double x = X[(size_t)(i * s + r) * d + e];
                if (pe) x += pe[r * d + e];
                const double* wrow = W + (size_t)(r * d + e) * d_out;
                for (int o = 0; o < d_out; ++o) acc[o] += x * wrow[o];
            }
        }
    }
}

/* Mean-pooled block key (MoBA): out[b][e] = (1/l) * sum_{r<l} X[(i*s + r)*d + e]. */
ORACLE_API void oracle_compress_mean(int d, int l, int s, const double* X,
                                     const int* blocks, int nblk, double* out)
{
#pragma omp parallel for schedule(static)
    for (int bi = 0; bi < nblk; ++bi) {
        const int i = blocks[bi];
        for (int e = 0; e < d; ++e) {
            double sum = 0.0;
            for (int r = 0; r < l; ++r) sum += X[(size_t)(i * s + r) * d + e];
            out[(size_t)bi * d + e] = sum / (double)l;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* helpers                                                                   */
/* ------------------------------------------------------------------------- */

static double dot(const double* a, const double* b, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/* Softmax of logits[0..n) into p, returning log(sum exp(logits)).  n >= 1. */
static double softmax(const double* logits, int n, double* p)
{
    double mx = logits[0];
    for (int i = 1; i < n; ++i) if (logits[i] > mx) mx = logits[i];
    double sum = 0.0;
    for (int i = 0; i < n; ++i) { p[i] = exp(logits[i] - mx); sum += p[i]; }
    for (int i = 0; i < n; ++i) p[i] /= sum;
    return mx + log(sum);
}

/* Number of compressed blocks whose whole span lies at or before token t. */
static int visible_cmp(int t, int l, int s, int n_cmp)
{
    if (t < l - 1) return 0;
    int n = (t - l + 1) / s + 1;
    return n < n_cmp ? n : n_cmp;
}


typedef struct { double score; int j; } cand_t;

/* Descending score; equal scores: ascending block index. */
static int cand_cmp(const void* x, const void* y)
{
    const cand_t* a = (const cand_t*)x;
    const cand_t* b = (const cand_t*)y;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int int_cmp(const void* x, const void* y)
{
    int a = *(const int*)x, b = *(const int*)y;
    return (a > b) - (a < b);
}

/* Forced blocks for a query whose own block is jc: {0..n_init-1} U {jc-n_local+1..jc},
 * restricted to 0..jc.  Writes a 0/1 flag per block 0..jc; returns the count. */
static int forced_blocks(int jc, int n_init, int n_local, unsigned char* flag)
{
    int cnt = 0;
    for (int j = 0; j <= jc; ++j) {
        flag[j] = (unsigned char)((j < n_init) || (j > jc - n_local));
        cnt += flag[j];
    }
    return cnt;
}

/* Step 4: pick blocks for one (query, group) from the scores of blocks 0..jc.
 * sel: top_n entries, ascending, -1 padded.  Returns the score gap between the last
 * chosen free block and the first rejected one (+inf when no free choice was cut). */
static double select_blocks(int jc, int top_n, int n_init, int n_local, const double* score,
                            int* sel, unsigned char* flag, cand_t* cand)
{
    const int n_elig = jc + 1;
    const int n_forced = forced_blocks(jc, n_init, n_local, flag);
    const int m = top_n < n_elig ? top_n : n_elig;
    const int k = m - n_forced;           /* free slots (validated >= 0 by the caller) */
    int nc = 0;
    for (int j = 0; j <= jc; ++j)
        if (!flag[j]) { cand[nc].score = score[j]; cand[nc].j = j; ++nc; }
    qsort(cand, (size_t)nc, sizeof(cand_t), cand_cmp);
    int cnt = 0;
    for (int j = 0; j <= jc; ++j) if (flag[j]) sel[cnt++] = j;
    for (int c = 0; c < k && c < nc; ++c) sel[cnt++] = cand[c].j;
    qsort(sel, (size_t)cnt, sizeof(int), int_cmp);
    for (int c = cnt; c < top_n; ++c) sel[c] = -1;
    if (k > 0 && k < nc) return cand[k - 1].score - cand[k].score;
    return INFINITY;
}

/* ------------------------------------------------------------------------- */
/* Steps 2-4: compressed attention, block scores, group-shared selection      */
/* ------------------------------------------------------------------------- */

/* For each listed query row (position rows[r]) and each KV group g:
 *   mode 0 (compressed-overlap scores):
 *     per head h of the group: logits a_i = scale * <q_h, Kc[g][i]> over the visible
 *     compressed blocks, p = softmax(a), lse = log sum exp(a), o_cmp = sum_i p_i Vc[g][i];
 *     score[j] = sum_h sum_{visible i intersecting block j} p_i.
 *   mode 1 (MoBA mean-key scores):
 *     score[j] = sum_h <q_h, Kc[g][j]> (unscaled) for complete blocks j before the
 *     query's own block (Kc holds the mean-pooled block keys); no compressed output.
 *   then the selection of step 4 over blocks 0 .. rows[r]/lp.
 *
 * Q_rows: [nrows, H_kv*G, dk]; Kc: [H_kv, n_cmp, dk]; Vc: [H_kv, n_cmp, dv] (mode 0 only,
 * may be NULL when o_cmp is not wanted).
 * Outputs (NULL = not wanted, except sel): lse [nrows, H] (-inf for an empty row),
 * o_cmp [nrows, H, dv], scores [nrows, H_kv, n_slc] (0 for blocks past the query's own),
 * sel [nrows, H_kv, top_n], gap [nrows, H_kv].
 * Returns 0, or -1 when top_n is smaller than the number of forced blocks. */
ORACLE_API int oracle_score_select(int mode, int H_kv, int G, int dk, int dv,
                                   int l, int s, int n_cmp, int lp, int n_slc,
                                   int top_n, int n_init, int n_local, double scale,
                                   const double* Q_rows, const int* rows, int nrows,
                                   const double* Kc, const double* Vc,
                                   double* lse_out, double* ocmp_out, double* scores_out,
                                   int* sel_out, double* gap_out)
{
    const int H = H_kv * G;
    if (top_n < n_init + n_local) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(|: bad)
    for (int rg = 0; rg < nrows * H_kv; ++rg) {
        const int r = rg / H_kv, g = rg % H_kv;
        const int t = rows[r];
        const int jc = t / lp;
        double* score = (double*)calloc((size_t)n_slc, sizeof(double));
        double* logit = (double*)malloc(sizeof(double) * (size_t)(n_cmp > 0 ? n_cmp : 1));
        double* p = (double*)malloc(sizeof(double) * (size_t)(n_cmp > 0 ? n_cmp : 1));
        unsigned char* flag = (unsigned char*)malloc((size_t)n_slc);
        cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)n_slc);
        if (!score || !logit || !p || !flag || !cand) { bad = 1; goto done; }

        for (int hh = 0; hh < G; ++hh) {
            const int h = g * G + hh;
            const double* q = Q_rows + ((size_t)r * H + h) * dk;
            if (mode == 0) {
                const int nv = visible_cmp(t, l, s, n_cmp);
                if (lse_out) lse_out[(size_t)r * H + h] = -INFINITY;
                if (ocmp_out) for (int e = 0; e < dv; ++e) ocmp_out[((size_t)r * H + h) * dv + e] = 0.0;
                if (nv == 0) continue;
                for (int i = 0; i < nv; ++i)
                    logit[i] = scale * dot(q, Kc + ((size_t)g * n_cmp + i) * dk, dk);
                const double lse = softmax(logit, nv, p);
                if (lse_out) lse_out[(size_t)r * H + h] = lse;
                if (ocmp_out && Vc) {
                    double* o = ocmp_out + ((size_t)r * H + h) * dv;
                    for (int i = 0; i < nv; ++i)
                        for (int e = 0; e < dv; ++e)
                            o[e] += p[i] * Vc[((size_t)g * n_cmp + i) * dv + e];
                }
                /* compressed block i spans tokens i*s .. i*s+l-1; it counts toward every
                 * selection block holding one of those tokens */
                for (int i = 0; i < nv; ++i)
                    for (int j = (i * s) / lp; j <= (i * s + l - 1) / lp && j < n_slc; ++j)
                        score[j] += p[i];
            } else {
                for (int j = 0; j < jc && j < n_cmp; ++j)
                    score[j] += dot(q, Kc + ((size_t)g * n_cmp + j) * dk, dk);
            }
        }
        {
            const double gap = select_blocks(jc, top_n, n_init, n_local, score,
                                             sel_out + ((size_t)r * H_kv + g) * top_n, flag, cand);
            if (gap_out) gap_out[(size_t)r * H_kv + g] = gap;
            if (scores_out) {
                double* so = scores_out + ((size_t)r * H_kv + g) * n_slc;
                for (int j = 0; j < n_slc; ++j) so[j] = (j <= jc) ? score[j] : 0.0;
            }
        }
    done:
        free(score); free(logit); free(p); free(flag); free(cand);
    }
    return bad ? -2 : 0;
}

/* Step 4 alone, from given scores: sel[r][.] for a query whose own block is jc[r].
 * scores: [nrows, n_slc]; sel: [nrows, top_n]; gap: [nrows] or NULL. */
ORACLE_API int oracle_select_from_scores(int nrows, int n_slc, int top_n, int n_init, int n_local,
                                         const int* jc, const double* scores, int* sel, double* gap)
{
    if (top_n < n_init + n_local) return -1;
    unsigned char* flag = (unsigned char*)malloc((size_t)n_slc);
    cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)n_slc);
    for (int r = 0; r < nrows; ++r) {
        const double gp = select_blocks(jc[r], top_n, n_init, n_local, scores + (size_t)r * n_slc,
                                        sel + (size_t)r * top_n, flag, cand);
        if (gap) gap[r] = gp;
    }
    free(flag); free(cand);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Steps 5-7: selected attention, sliding window, gated sum                  */
/* ------------------------------------------------------------------------- */

/* Softmax attention of q over an explicit key list: o = sum_k softmax(scale*<q,K[k]>) V[k]. */
static void attend_list(const double* q, const double* K, const double* V, int dk, int dv,
                        double scale, const int* keys, int nk, double* logit, double* p, double* o)
{
    for (int e = 0; e < dv; ++e) o[e] = 0.0;
    if (nk == 0) return;
    for (int c = 0; c < nk; ++c) logit[c] = scale * dot(q, K + (size_t)keys[c] * dk, dk);
    softmax(logit, nk, p);
    for (int c = 0; c < nk; ++c)
        for (int e = 0; e < dv; ++e) o[e] += p[c] * V[(size_t)keys[c] * dv + e];
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* For each listed query row and head h (group g = h / G):
 *   o_slc: attention over the tokens of the listed blocks of (row, g) that are <= t;
 *   o_win: attention over tokens max(0, t-w+1) .. t;
 *   out = sum over enabled branches of sigmoid(gate) * o_branch
 *         (branch bits: 1 compressed, 2 selected, 4 window; gate order cmp, slc, win;
 *          gates NULL -> every gate weight is 1).
 * Q_rows [nrows, H, dk]; K [H_kv, n_tok, dk]; V [H_kv, n_tok, dv]; sel [nrows, H_kv, top_n]
 * (entries < 0 ignored); ocmp [nrows, H, dv] (needed when branch 1 is on); gates
 * [nrows, H, 3]; out, oslc, owin [nrows, H, dv] (oslc/owin may be NULL). */
ORACLE_API int oracle_attend(int H_kv, int G, int dk, int dv, int n_tok, int lp, int top_n,
                             int window, double scale, int branches,
                             const double* Q_rows, const int* rows, int nrows,
                             const double* K, const double* V, const int* sel,
                             const double* ocmp, const double* gates,
                             double* out, double* oslc_out, double* owin_out)
{
    const int H = H_kv * G;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(|: bad)
    for (int rh = 0; rh < nrows * H; ++rh) {
        const int r = rh / H, h = rh % H, g = h / G;
        const int t = rows[r];
        const double* q = Q_rows + ((size_t)r * H + h) * dk;
        const double* Kg = K + (size_t)g * n_tok * dk;
        const double* Vg = V + (size_t)g * n_tok * dv;
        const int cap = top_n * lp + window + 1;
        int* keys = (int*)malloc(sizeof(int) * (size_t)cap);
        double* logit = (double*)malloc(sizeof(double) * (size_t)cap);
        double* p = (double*)malloc(sizeof(double) * (size_t)cap);
        double* os = (double*)malloc(sizeof(double) * (size_t)dv);
        double* ow = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!keys || !logit || !p || !os || !ow) { bad = 1; goto done; }

        /* selected tokens: the union of the listed blocks, restricted to <= t */
        {
            int nk = 0;
            const int* sl = sel + ((size_t)r * H_kv + g) * top_n;
            for (int c = 0; c < top_n; ++c) {
                const int j = sl[c];
                if (j < 0) continue;
                int dup = 0;
                for (int c2 = 0; c2 < c; ++c2) dup |= (sl[c2] == j);
                if (dup) continue;
                for (int x = j * lp; x < (j + 1) * lp && x <= t; ++x) keys[nk++] = x;
            }
            attend_list(q, Kg, Vg, dk, dv, scale, keys, nk, logit, p, os);
        }
        /* window tokens */
        {
            int nk = 0;
            const int t0 = (t - window + 1) > 0 ? (t - window + 1) : 0;
            for (int x = t0; x <= t && window > 0; ++x) keys[nk++] = x;
            attend_list(q, Kg, Vg, dk, dv, scale, keys, nk, logit, p, ow);
        }
        {
            const double* z = gates ? gates + ((size_t)r * H + h) * 3 : NULL;
            const double gc = z ? sigmoid(z[0]) : 1.0;
            const double gs = z ? sigmoid(z[1]) : 1.0;
            const double gw = z ? sigmoid(z[2]) : 1.0;
            double* o = out + ((size_t)r * H + h) * dv;
            for (int e = 0; e < dv; ++e) {
                double acc = 0.0;
                if (branches & 1) acc += gc * ocmp[((size_t)r * H + h) * dv + e];
                if (branches & 2) acc += gs * os[e];
                if (branches & 4) acc += gw * ow[e];
                o[e] = acc;
            }
            if (oslc_out) memcpy(oslc_out + ((size_t)r * H + h) * dv, os, sizeof(double) * dv);
            if (owin_out) memcpy(owin_out + ((size_t)r * H + h) * dv, ow, sizeof(double) * dv);
        }
    done:
        free(keys); free(logit); free(p); free(os); free(ow);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------- */
/* Textbook references used by the oracle's own pins                         */
/* ------------------------------------------------------------------------- */

/* Causal attention of one head, restricted to keys t-w+1 .. t when w > 0 (w <= 0: all
 * keys 0 .. t).  Q [n, dk], K [n, dk], V [n, dv], out [n, dv]. */
ORACLE_API void oracle_causal_attention(int n, int dk, int dv, int w, double scale,
                                        const double* Q, const double* K, const double* V,
                                        double* out)
{
#pragma omp parallel for schedule(dynamic)
    for (int t = 0; t < n; ++t) {
        const int t0 = (w > 0 && t - w + 1 > 0) ? t - w + 1 : 0;
        const int nk = t - t0 + 1;
        double* logit = (double*)malloc(sizeof(double) * (size_t)nk);
        double mx = -INFINITY, sum = 0.0;
        for (int x = t0; x <= t; ++x) {
            double a = 0.0;
            for (int e = 0; e < dk; ++e) a += Q[(size_t)t * dk + e] * K[(size_t)x * dk + e];
            logit[x - t0] = a * scale;
            if (logit[x - t0] > mx) mx = logit[x - t0];
        }
        for (int c = 0; c < nk; ++c) { logit[c] = exp(logit[c] - mx); sum += logit[c]; }
        for (int e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int x = t0; x <= t; ++x) acc += logit[x - t0] * V[(size_t)x * dv + e];
            out[(size_t)t * dv + e] = acc / sum;
        }
        free(logit);
    }
}

/* Causal attention of listed query rows (row rows[k] attends keys 0 .. rows[k]): the same
 * textbook softmax as oracle_causal_attention, for rows taken from a long sequence. */
ORACLE_API void oracle_causal_attention_rows(int nrows, const int* rows, int dk, int dv, double scale,
                                             const double* Qrows, const double* K, const double* V,
                                             double* out)
{
#pragma omp parallel for schedule(dynamic)
    for (int k = 0; k < nrows; ++k) {
        const int t = rows[k];
        double* logit = (double*)malloc(sizeof(double) * (size_t)(t + 1));
        double mx = -INFINITY, sum = 0.0;
        for (int x = 0; x <= t; ++x) {
            double a = 0.0;
            for (int e = 0; e < dk; ++e) a += Qrows[(size_t)k * dk + e] * K[(size_t)x * dk + e];
            logit[x] = a * scale;
            if (logit[x] > mx) mx = logit[x];
        }
        for (int x = 0; x <= t; ++x) { logit[x] = exp(logit[x] - mx); sum += logit[x]; }
        for (int e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int x = 0; x <= t; ++x) acc += logit[x] * V[(size_t)x * dv + e];
            out[(size_t)k * dv + e] = acc / sum;
        }
        free(logit);
    }
}

/* ------------------------------------------------------------------------- */
/* Backward pass (gradients of the output, the selection held fixed)         */
/* ------------------------------------------------------------------------- */
/*
 * zjai.club [B], section 4 (the method is trained natively, forward and backward),
 * section 13 (its speed claims cover the backward pass too) and section 14 (the top-k
 * choice has no derivative; the compressed branch's output is what carries the loss's
 * gradient into the block representations): the backward pass is the chain rule through
 * steps 1, 2 and 5-7.  The block choice of steps 3-4 is a discrete function of the scores
 * and passes no gradient; the listed blocks are an input here.
 *
 * For one softmax attention o = sum_k p_k v_k, p = softmax(a), a_k = scale <q, k_k>, and an
 * upstream gradient go of o (the textbook derivative of a softmax-weighted sum):
 *   dv_k += p_k go
 *   dp_k  = <go, v_k>
 *   da_k  = p_k (dp_k - sum_j p_j dp_j)
 *   dq   += scale sum_k da_k k_k
 *   dk_k += scale da_k q
 * For the gated sum out = sum_c sigma(z_c) o_c: go_c = sigma(z_c) dout and
 * dz_c = sigma(z_c) (1 - sigma(z_c)) <dout, o_c>.
 */

/* Backward of one attention over an explicit key list (indices into K / V).  Adds into
 * dq [dk], dK, dV (rows indexed like K, V; both NULL: the key side is skipped).  Returns
 * <dout, o>, o recomputed here. */
static double attend_list_bwd(const double* q, const double* K, const double* V, int dk, int dv, double scale,
                              const int* keys, int nk, const double* dout, double sig,
                              double* logit, double* p, double* o,
                              double* dq, double* dK, double* dV)
{
    if (nk == 0) return 0.0;
    for (int c = 0; c < nk; ++c) logit[c] = scale * dot(q, K + (size_t)keys[c] * dk, dk);
    softmax(logit, nk, p);
    for (int e = 0; e < dv; ++e) o[e] = 0.0;
    for (int c = 0; c < nk; ++c)
        for (int e = 0; e < dv; ++e) o[e] += p[c] * V[(size_t)keys[c] * dv + e];
    /* dp_k = <sig * dout, v_k>; logit[] is reused to hold dp */
    double pdp = 0.0;
    for (int c = 0; c < nk; ++c) {
        logit[c] = sig * dot(dout, V + (size_t)keys[c] * dv, dv);
        pdp += p[c] * logit[c];
    }
    for (int c = 0; c < nk; ++c) {
        const int x = keys[c];
        const double da = p[c] * (logit[c] - pdp);
        for (int e = 0; e < dk; ++e) dq[e] += scale * da * K[(size_t)x * dk + e];
        if (!dK) continue;
        for (int e = 0; e < dk; ++e) dK[(size_t)x * dk + e] += scale * da * q[e];
        for (int e = 0; e < dv; ++e) dV[(size_t)x * dv + e] += p[c] * sig * dout[e];
    }
    return dot(dout, o, dv);
}

/* Gradients of the gated output of every row t = 0 .. n_tok-1 of one batch element with
 * respect to Q, K, V (selected and window branches), the compressed keys and values Kc, Vc
 * (compressed branch) and the gate logits, for the upstream gradient dO.  The branches
 * and visibility rules are those of the forward functions above: compressed blocks i with
 * i*s + l - 1 <= t; the tokens <= t of the listed blocks; tokens max(0, t-w+1) .. t.
 * Q [n_tok, H, dk]; K [H_kv, n_tok, dk]; V [H_kv, n_tok, dv]; Kc [H_kv, n_cmp, dk];
 * Vc [H_kv, n_cmp, dv]; sel [n_tok, H_kv, top_n]; gates [n_tok, H, 3] or NULL (weights 1,
 * dgates not written); dO [n_tok, H, dv].  Every output is overwritten (dKc, dVc and
 * dgates may be NULL when unused).  Returns 0, or -2 when memory runs out. */
ORACLE_API int oracle_nsa_bwd(int H_kv, int G, int dk, int dv, int n_tok, int n_cmp, int l, int s, int lp,
                              int top_n, int window, double scale, int branches,
                              const double* Q, const double* K, const double* V,
                              const double* Kc, const double* Vc, const int* sel,
                              const double* gates, const double* dO,
                              double* dQ, double* dK, double* dV, double* dKc, double* dVc, double* dgates)
{
    const int H = H_kv * G;
    const size_t nK = (size_t)H_kv * n_tok, nC = (size_t)H_kv * n_cmp;
    memset(dQ, 0, sizeof(double) * (size_t)n_tok * H * dk);
    memset(dK, 0, sizeof(double) * nK * dk);
    memset(dV, 0, sizeof(double) * nK * dv);
    if (dKc) memset(dKc, 0, sizeof(double) * nC * dk);
    if (dVc) memset(dVc, 0, sizeof(double) * nC * dv);
    if (dgates) memset(dgates, 0, sizeof(double) * (size_t)n_tok * H * 3);
    int bad = 0;
#pragma omp parallel reduction(|: bad)
    {
        /* per-thread sums of the key-side gradients, added up once at the end */
        double* tK = (double*)calloc(nK * dk, sizeof(double));
        double* tV = (double*)calloc(nK * dv, sizeof(double));
        double* tKc = (double*)calloc(nC * dk + 1, sizeof(double));
        double* tVc = (double*)calloc(nC * dv + 1, sizeof(double));
        const int cap = n_cmp + top_n * lp + window + 1;
        int* keys = (int*)malloc(sizeof(int) * (size_t)cap);
        double* logit = (double*)malloc(sizeof(double) * (size_t)cap);
        double* p = (double*)malloc(sizeof(double) * (size_t)cap);
        double* o = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!tK || !tV || !tKc || !tVc || !keys || !logit || !p || !o) bad = 1;
        else {
#pragma omp for schedule(dynamic)
            for (int th = 0; th < n_tok * H; ++th) {
                const int t = th / H, h = th % H, g = h / G;
                const double* q = Q + (size_t)th * dk;
                const double* dout = dO + (size_t)th * dv;
                double* dq = dQ + (size_t)th * dk;
                const double* z = gates ? gates + (size_t)th * 3 : NULL;
                double sig[3];
                for (int c = 0; c < 3; ++c) sig[c] = z ? sigmoid(z[c]) : 1.0;
                double od[3] = {0.0, 0.0, 0.0};
                const size_t kg = (size_t)g * n_tok, cg = (size_t)g * n_cmp;
                if (branches & 1) {
                    const int nk = visible_cmp(t, l, s, n_cmp);
                    for (int i = 0; i < nk; ++i) keys[i] = i;
                    od[0] = attend_list_bwd(q, Kc + cg * dk, Vc + cg * dv, dk, dv, scale, keys, nk, dout, sig[0],
                                            logit, p, o, dq, tKc + cg * dk, tVc + cg * dv);
                }
                if (branches & 2) {
                    int nk = 0;
                    const int* sl = sel + ((size_t)t * H_kv + g) * top_n;
                    for (int c = 0; c < top_n; ++c) {
                        const int j = sl[c];
                        if (j < 0) continue;
                        int dup = 0;
                        for (int c2 = 0; c2 < c; ++c2) dup |= (sl[c2] == j);
                        if (dup) continue;
                        for (int x = j * lp; x < (j + 1) * lp && x <= t; ++x) keys[nk++] = x;
                    }
                    od[1] = attend_list_bwd(q, K + kg * dk, V + kg * dv, dk, dv, scale, keys, nk, dout, sig[1],
                                            logit, p, o, dq, tK + kg * dk, tV + kg * dv);
                }
                if (branches & 4) {
                    int nk = 0;
                    const int t0 = (t - window + 1) > 0 ? (t - window + 1) : 0;
                    for (int x = t0; x <= t && window > 0; ++x) keys[nk++] = x;
                    od[2] = attend_list_bwd(q, K + kg * dk, V + kg * dv, dk, dv, scale, keys, nk, dout, sig[2],
                                            logit, p, o, dq, tK + kg * dk, tV + kg * dv);
                }
                if (dgates)
                    for (int c = 0; c < 3; ++c)
                        if (branches & (1 << c)) dgates[(size_t)th * 3 + c] = sig[c] * (1.0 - sig[c]) * od[c];
            }
#pragma omp critical
            {
                for (size_t i = 0; i < nK * dk; ++i) dK[i] += tK[i];
                for (size_t i = 0; i < nK * dv; ++i) dV[i] += tV[i];
                if (dKc) for (size_t i = 0; i < nC * dk; ++i) dKc[i] += tKc[i];
                if (dVc) for (size_t i = 0; i < nC * dv; ++i) dVc[i] += tVc[i];
            }
        }
        free(tK); free(tV); free(tKc); free(tVc); free(keys); free(logit); free(p); free(o);
    }
    return bad ? -2 : 0;
}

/* The query-side part of oracle_nsa_bwd for listed rows only (dq and the gate-logit
 * gradients; the key side is not formed), so that rows of a long sequence can be checked one
 * by one.  Q_rows [nrows, H, dk], sel_rows [nrows, H_kv, top_n], gates_rows [nrows, H, 3] or
 * NULL, dO_rows [nrows, H, dv]; K, V, Kc, Vc as for oracle_nsa_bwd; dQ_rows [nrows, H, dk],
 * dgates_rows [nrows, H, 3] or NULL (overwritten).  Returns 0, or -2 when memory runs out. */
ORACLE_API int oracle_nsa_bwd_rows(int H_kv, int G, int dk, int dv, int n_tok, int n_cmp, int l, int s, int lp,
                                   int top_n, int window, double scale, int branches,
                                   const double* Q_rows, const int* rows, int nrows,
                                   const double* K, const double* V, const double* Kc, const double* Vc,
                                   const int* sel_rows, const double* gates_rows, const double* dO_rows,
                                   double* dQ_rows, double* dgates_rows)
{
    const int H = H_kv * G;
    int bad = 0;
    memset(dQ_rows, 0, sizeof(double) * (size_t)nrows * H * dk);
    if (dgates_rows) memset(dgates_rows, 0, sizeof(double) * (size_t)nrows * H * 3);
#pragma omp parallel for schedule(dynamic) reduction(|: bad)
    for (int rh = 0; rh < nrows * H; ++rh) {
        const int r = rh / H, h = rh % H, g = h / G, t = rows[r];
        const int cap = n_cmp + top_n * lp + window + 1;
        int* keys = (int*)malloc(sizeof(int) * (size_t)cap);
        double* logit = (double*)malloc(sizeof(double) * (size_t)cap);
        double* p = (double*)malloc(sizeof(double) * (size_t)cap);
        double* o = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!keys || !logit || !p || !o) { bad = 1; goto done; }
        {
            const double* q = Q_rows + (size_t)rh * dk;
            const double* dout = dO_rows + (size_t)rh * dv;
            double* dq = dQ_rows + (size_t)rh * dk;
            const double* z = gates_rows ? gates_rows + (size_t)rh * 3 : NULL;
            double sig[3], od[3] = {0.0, 0.0, 0.0};
            for (int c = 0; c < 3; ++c) sig[c] = z ? sigmoid(z[c]) : 1.0;
            const size_t kg = (size_t)g * n_tok, cg = (size_t)g * n_cmp;
            if (branches & 1) {
                const int nk = visible_cmp(t, l, s, n_cmp);
                for (int i = 0; i < nk; ++i) keys[i] = i;
                od[0] = attend_list_bwd(q, Kc + cg * dk, Vc + cg * dv, dk, dv, scale, keys, nk, dout, sig[0],
                                        logit, p, o, dq, NULL, NULL);
            }
            if (branches & 2) {
                int nk = 0;
                const int* sl = sel_rows + ((size_t)r * H_kv + g) * top_n;
                for (int c = 0; c < top_n; ++c) {
                    const int j = sl[c];
                    if (j < 0) continue;
                    int dup = 0;
                    for (int c2 = 0; c2 < c; ++c2) dup |= (sl[c2] == j);
                    if (dup) continue;
                    for (int x = j * lp; x < (j + 1) * lp && x <= t; ++x) keys[nk++] = x;
                }
                od[1] = attend_list_bwd(q, K + kg * dk, V + kg * dv, dk, dv, scale, keys, nk, dout, sig[1],
                                        logit, p, o, dq, NULL, NULL);
            }
            if (branches & 4) {
                int nk = 0;
                const int t0 = (t - window + 1) > 0 ? (t - window + 1) : 0;
                for (int x = t0; x <= t && window > 0; ++x) keys[nk++] = x;
                od[2] = attend_list_bwd(q, K + kg * dk, V + kg * dv, dk, dv, scale, keys, nk, dout, sig[2],
                                        logit, p, o, dq, NULL, NULL);
            }
            if (dgates_rows)
                for (int c = 0; c < 3; ++c)
                    if (branches & (1 << c)) dgates_rows[(size_t)rh * 3 + c] = sig[c] * (1.0 - sig[c]) * od[c];
        }
    done:
        free(keys); free(logit); free(p); free(o);
    }
    return bad ? -2 : 0;
}

/* The key-side part of oracle_nsa_bwd for listed keys only, so that keys of a long
 * sequence can be checked without forming every gradient.  raw_keys [n_raw] are token
 * indices and cmp_keys [n_ck] compressed-block indices (each ascending, no repeats); both
 * lists apply to every KV group.  Outputs (overwritten): dK_l [H_kv, n_raw, dk], dV_l
 * [H_kv, n_raw, dv], dKc_l [H_kv, n_ck, dk], dVc_l [H_kv, n_ck, dv] (the last two may be NULL
 * when n_ck = 0) hold exactly the sums oracle_nsa_bwd forms for those keys: over every
 * (token, head) row whose branch sees the key, dk += scale * da * q and dv += sigma * p * dO,
 * with that row's softmax taken over all of the branch's keys.  Rows that see no listed key
 * are skipped.  Other arguments as for oracle_nsa_bwd.  Returns 0, or -2 when memory runs
 * out. */
static void list_bwd_keys(const double* q, const double* K, const double* V, int dk, int dv, double scale,
                          const int* keys, int nk, const double* dout, double sig, const int* slot,
                          double* logit, double* p, double* dK_l, double* dV_l)
{
    for (int c = 0; c < nk; ++c) logit[c] = scale * dot(q, K + (size_t)keys[c] * dk, dk);
    softmax(logit, nk, p);
    double pdp = 0.0;
    for (int c = 0; c < nk; ++c) {
        logit[c] = sig * dot(dout, V + (size_t)keys[c] * dv, dv);   /* dp_k */
        pdp += p[c] * logit[c];
    }
    for (int c = 0; c < nk; ++c) {
        const int sl = slot[keys[c]];
        if (sl < 0) continue;
        const double da = p[c] * (logit[c] - pdp);
        for (int e = 0; e < dk; ++e) dK_l[(size_t)sl * dk + e] += scale * da * q[e];
        for (int e = 0; e < dv; ++e) dV_l[(size_t)sl * dv + e] += p[c] * sig * dout[e];
    }
}

ORACLE_API int oracle_nsa_bwd_keys(int H_kv, int G, int dk, int dv, int n_tok, int n_cmp, int l, int s, int lp,
                                   int top_n, int window, double scale, int branches,
                                   const double* Q, const double* K, const double* V,
                                   const double* Kc, const double* Vc, const int* sel,
                                   const double* gates, const double* dO,
                                   const int* raw_keys, int n_raw, const int* cmp_keys, int n_ck,
                                   double* dK_l, double* dV_l, double* dKc_l, double* dVc_l)
{
    const int H = H_kv * G;
    const size_t nRk = (size_t)H_kv * n_raw * dk, nRv = (size_t)H_kv * n_raw * dv;
    const size_t nCk = (size_t)H_kv * n_ck * dk, nCv = (size_t)H_kv * n_ck * dv;
    memset(dK_l, 0, sizeof(double) * nRk);
    memset(dV_l, 0, sizeof(double) * nRv);
    if (dKc_l) memset(dKc_l, 0, sizeof(double) * nCk);
    if (dVc_l) memset(dVc_l, 0, sizeof(double) * nCv);
    /* slot of every token / compressed block in the lists (-1: not listed), and the number
     * of listed tokens before each position (a row sees a listed token of [a, b] exactly when
     * before[b + 1] > before[a]) */
    int* rslot = (int*)malloc(sizeof(int) * (size_t)(n_tok + 1));
    int* before = (int*)malloc(sizeof(int) * (size_t)(n_tok + 1));
    int* cslot = (int*)malloc(sizeof(int) * (size_t)(n_cmp + 1));
    if (!rslot || !before || !cslot) { free(rslot); free(before); free(cslot); return -2; }
    for (int x = 0; x < n_tok; ++x) rslot[x] = -1;
    for (int i = 0; i < n_cmp; ++i) cslot[i] = -1;
    for (int c = 0; c < n_raw; ++c) rslot[raw_keys[c]] = c;
    for (int c = 0; c < n_ck; ++c) cslot[cmp_keys[c]] = c;
    before[0] = 0;
    for (int x = 0; x < n_tok; ++x) before[x + 1] = before[x] + (rslot[x] >= 0);
    const int first_ck = n_ck > 0 ? cmp_keys[0] : n_cmp;
    int bad = 0;
#pragma omp parallel reduction(|: bad)
    {
        double* tK = (double*)calloc(nRk + 1, sizeof(double));
        double* tV = (double*)calloc(nRv + 1, sizeof(double));
        double* tKc = (double*)calloc(nCk + 1, sizeof(double));
        double* tVc = (double*)calloc(nCv + 1, sizeof(double));
        const int cap = n_cmp + top_n * lp + window + 1;
        int* keys = (int*)malloc(sizeof(int) * (size_t)cap);
        double* logit = (double*)malloc(sizeof(double) * (size_t)cap);
        double* p = (double*)malloc(sizeof(double) * (size_t)cap);
        if (!tK || !tV || !tKc || !tVc || !keys || !logit || !p) bad = 1;
        else {
#pragma omp for schedule(dynamic, 16)
            for (int th = 0; th < n_tok * H; ++th) {
                const int t = th / H, h = th % H, g = h / G;
                const double* q = Q + (size_t)th * dk;
                const double* dout = dO + (size_t)th * dv;
                const double* z = gates ? gates + (size_t)th * 3 : NULL;
                double sig[3];
                for (int c = 0; c < 3; ++c) sig[c] = z ? sigmoid(z[c]) : 1.0;
                const size_t kg = (size_t)g * n_tok, cg = (size_t)g * n_cmp;
                if ((branches & 1) && n_ck > 0) {
                    const int nk = visible_cmp(t, l, s, n_cmp);
                    if (nk > first_ck) {
                        for (int i = 0; i < nk; ++i) keys[i] = i;
                        list_bwd_keys(q, Kc + cg * dk, Vc + cg * dv, dk, dv, scale, keys, nk, dout, sig[0], cslot,
                                      logit, p, tKc + (size_t)g * n_ck * dk, tVc + (size_t)g * n_ck * dv);
                    }
                }
                if ((branches & 2) && n_raw > 0) {
                    int nk = 0, hit = 0;
                    const int* sl = sel + ((size_t)t * H_kv + g) * top_n;
                    for (int c = 0; c < top_n; ++c) {
                        const int j = sl[c];
                        if (j < 0) continue;
                        int dup = 0;
                        for (int c2 = 0; c2 < c; ++c2) dup |= (sl[c2] == j);
                        if (dup) continue;
                        const int a = j * lp, b = ((j + 1) * lp - 1 < t ? (j + 1) * lp - 1 : t);
                        if (a > b) continue;
                        hit |= before[b + 1] > before[a];
                        for (int x = a; x <= b; ++x) keys[nk++] = x;
                    }
                    if (hit)
                        list_bwd_keys(q, K + kg * dk, V + kg * dv, dk, dv, scale, keys, nk, dout, sig[1], rslot,
                                      logit, p, tK + (size_t)g * n_raw * dk, tV + (size_t)g * n_raw * dv);
                }
                if ((branches & 4) && n_raw > 0 && window > 0) {
                    const int t0 = (t - window + 1) > 0 ? (t - window + 1) : 0;
                    if (before[t + 1] > before[t0]) {
                        int nk = 0;
                        for (int x = t0; x <= t; ++x) keys[nk++] = x;
                        list_bwd_keys(q, K + kg * dk, V + kg * dv, dk, dv, scale, keys, nk, dout, sig[2], rslot,
                                      logit, p, tK + (size_t)g * n_raw * dk, tV + (size_t)g * n_raw * dv);
                    }
                }
            }
#pragma omp critical
            {
                for (size_t i = 0; i < nRk; ++i) dK_l[i] += tK[i];
                for (size_t i = 0; i < nRv; ++i) dV_l[i] += tV[i];
                if (dKc_l) for (size_t i = 0; i < nCk; ++i) dKc_l[i] += tKc[i];
                if (dVc_l) for (size_t i = 0; i < nCv; ++i) dVc_l[i] += tVc[i];
            }
        }
        free(tK); free(tV); free(tKc); free(tVc); free(keys); free(logit); free(p);
    }
    free(rslot); free(before); free(cslot);
    return bad ? -2 : 0;
}

/* Backward of the linear block map of step 1 over blocks 0 .. nblk-1 (block i covers
 * tokens i*s .. i*s+l-1), for the gradient dY [nblk, d_out] of its output.  Since
 * Y[i][o] = sum_{r,e} (X[i*s+r][e] + pe[r][e]) W[r*d+e][o]:
 *   dX[i*s+r][e] += sum_o W[r*d+e][o] dY[i][o]     (a token in several blocks sums them)
 *   dpe[r][e]    += the same sum
 *   dW[r*d+e][o] += (X[i*s+r][e] + pe[r][e]) dY[i][o]
 * X [n_tok, d]; pe [l, d] or NULL; W [l*d, d_out]; dX [n_tok, d]; dW [l*d, d_out]; dpe
 * [l, d] or NULL.  Accumulates (the caller zeroes), so heads and sequences can be summed. */
ORACLE_API void oracle_compress_linear_bwd(int n_tok, int d, int d_out, int l, int s, int nblk,
                                           const double* X, const double* pe, const double* W,
                                           const double* dY, double* dX, double* dW, double* dpe)
{
    (void)n_tok;
    for (int i = 0; i < nblk; ++i) {
        const double* dy = dY + (size_t)i * d_out;
        for (int r = 0; r < l; ++r) {
            for (int e = 0; e < d; ++e) {
                const double* wrow = W + (size_t)(r * d + e) * d_out;
                double x = X[(size_t)(i * s + r) * d + e];
                if (pe) x += pe[r * d + e];
                double gx = 0.0;
                for (int o = 0; o < d_out; ++o) {
                    gx += wrow[o] * dy[o];
                    dW[(size_t)(r * d + e) * d_out + o] += x * dy[o];
                }
                dX[(size_t)(i * s + r) * d + e] += gx;
                if (dpe) dpe[r * d + e] += gx;
            }
        }
    }
}

ORACLE_API int oracle_num_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp master
        n = omp_get_num_threads();
    }
#endif
    return n;
}
