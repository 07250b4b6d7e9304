/*
 * attn_oracle.c -- plain, slow, obviously correct fp64 CPU attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the bench's
 * CPU-baseline leg use it.  It shares no code, header or constant with the HIP
 * library; its mask codes are its own (ORACLE_MASK_* below).
 *
 * What it computes.  The attention that the paper "A Modern Multimodal
 * Assistant on a 6 GB 2011 GPU" speeds up is exact scaled-dot-product
 * attention: its abstract, result (iii), replaces a naive attention kernel by
 * per-head GEMMs that give the same scores, so the faster path is the same
 * function, computed faster.  The gist.science technical summary of the same
 * paper (Metodologia, attention rewrite) names two forms of it: causal
 * attention in the language model and bidirectional attention in the vision
 * tower; the abstract names a window-attention merger as a third stage.  For
 * every query row i of a sequence, with J(i) its visible keys:
 *
 *     s_j  = scale * <q_i, k_j>                      j in J(i)
 *     out_i = sum_j softmax(s)_j * v_j
 *
 * Where the pages leave a step open this file takes the plain reading:
 *   - no dropout, bias, cap or sink; the softmax is the textbook one;
 *   - causal: J(i) = {0..i} (diagonal included), positions local to the
 *     sequence;
 *   - full (bidirectional): J(i) = every key of the same sequence;
 *   - window W: non-overlapping blocks of W tokens aligned to the sequence
 *     start, bidirectional inside a block, last block may be partial;
 *   - sequences in a packed batch never see each other;
 *   - grouped-query heads: query head h reads key/value head h / (Hq/Hkv).
 *
 * Arithmetic is fp64 throughout, in the order of the definition: scores,
 * their maximum, the shifted exponentials, their sum, then the weighted sum
 * of values.  Rows are independent; OpenMP splits the list of requested rows
 * and nothing else.
 *
 * Layout: q[T][Hq][d], k[T][Hkv][d], v[T][Hkv][d], row-major fp64, T the
 * total number of packed tokens; cu_seqlens[n_seqs+1] gives sequence b the
 * tokens cu_seqlens[b] .. cu_seqlens[b+1]-1.
 *
 * Queries against a longer key sequence (the *_kv entry points).  The
 * paper's system keeps its key/value cache resident on the GPU (gist.science
 * technical summary, Metodologia) and decodes over it after prefill (same
 * summary, Contribuciones Clave y Resultados), so a call may hold fewer new
 * queries than keys:
 * q[Tq][Hq][d] packed by cu_q, k/v[Tk][Hkv][d] packed by cu_k, with
 * Lq_b = cu_q[b+1]-cu_q[b] <= Lk_b = cu_k[b+1]-cu_k[b].  The pages do not say
 * where those queries sit; the plain reading is that they are the LAST Lq_b
 * tokens of the sequence (the newest tokens, "bottom-right" alignment), so
 * local query i has position p = i + Lk_b - Lq_b and every mask above is
 * evaluated at p over Lk_b keys.  With cu_q = cu_k this is the square case.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_MASK_CAUSAL 0
#define ORACLE_MASK_FULL 1
#define ORACLE_MASK_WINDOW 2

/* Visible keys of local query row i in a sequence of n tokens, as the
 * half-open local range [*lo, *hi).  Integer arithmetic only. */
static void visible_range(int mask, int64_t window, int64_t i, int64_t n,
                          int64_t *lo, int64_t *hi) {
    if (mask == ORACLE_MASK_CAUSAL) {
        *lo = 0;
        *hi = i + 1;
    } else if (mask == ORACLE_MASK_FULL) {
        *lo = 0;
        *hi = n;
    } else {
        int64_t start = (i / window) * window;
        int64_t end = start + window;
        *lo = start;
        *hi = end < n ? end : n;
    }
}

/* Index b of the sequence holding packed token t (cu is non-decreasing). */
static int seq_of_token(const int32_t *cu, int n_seqs, int64_t t) {
    int b = 0;
    while (b < n_seqs && (int64_t)cu[b + 1] <= t) b++;
    return b;
}

/*
 * One output row: the query row qi of query head h at position pos of a
 * sequence whose n keys/values start at kseq/vseq.  Writes d values to
 * out_row and, when lse is non-NULL, log(sum_j exp(s_j)) to *lse.  When probs
 * is non-NULL it receives the softmax weights of the visible keys, in key
 * order (the caller sizes it to the sequence length).  Returns the number of
 * visible keys.
 */
static int64_t one_row(const double *qi, const double *kseq, const double *vseq,
                       int hq, int hkv, int d, int mask, int64_t window,
                       double scale, int64_t pos, int64_t n, int h,
                       double *out_row, double *lse, double *probs,
                       double *scores) {
    int g = h / (hq / hkv);
    int64_t lo, hi;
    visible_range(mask, window, pos, n, &lo, &hi);

    /* scores of the visible keys */
    for (int64_t j = lo; j < hi; j++) {
        const double *kj = kseq + ((size_t)j * hkv + g) * d;
        double dot = 0.0;
        for (int c = 0; c < d; c++) dot += qi[c] * kj[c];
        scores[j - lo] = scale * dot;
    }
    /* softmax: maximum, shifted exponentials, their sum */
    double m = -INFINITY;
    for (int64_t j = lo; j < hi; j++)
        if (scores[j - lo] > m) m = scores[j - lo];
    double l = 0.0;
    for (int64_t j = lo; j < hi; j++) {
        scores[j - lo] = exp(scores[j - lo] - m);
        l += scores[j - lo];
    }
    /* weighted sum of the visible values */
    for (int c = 0; c < d; c++) out_row[c] = 0.0;
    for (int64_t j = lo; j < hi; j++) {
        double p = scores[j - lo] / l;
        const double *vj = vseq + ((size_t)j * hkv + g) * d;
        for (int c = 0; c < d; c++) out_row[c] += p * vj[c];
        if (probs) probs[j - lo] = p;
    }
    if (lse) *lse = m + log(l);
    return hi - lo;
}

/* Row of packed query token t (head h): locate its sequence and position. */
static int64_t token_row(const double *q, const double *k, const double *v,
                         const int32_t *cu_q, const int32_t *cu_k, int n_seqs,
                         int hq, int hkv, int d, int mask, int64_t window,
                         double scale, int64_t t, int h, double *out_row,
                         double *lse, double *probs, double *scores) {
    int b = seq_of_token(cu_q, n_seqs, t);
    int64_t lq = (int64_t)cu_q[b + 1] - cu_q[b];
    int64_t lk = (int64_t)cu_k[b + 1] - cu_k[b];
    int64_t pos = (t - cu_q[b]) + (lk - lq);
    const double *kseq = k + (size_t)cu_k[b] * hkv * d;
    const double *vseq = v + (size_t)cu_k[b] * hkv * d;
    return one_row(q + ((size_t)t * hq + h) * d, kseq, vseq, hq, hkv, d, mask,
                   window, scale, pos, lk, h, out_row, lse, probs, scores);
}

static int args_ok(const int32_t *cu_q, const int32_t *cu_k, int n_seqs,
                   int hq, int hkv, int d, int mask, int64_t window) {
    if (n_seqs < 0 || hq <= 0 || hkv <= 0 || d <= 0) return 0;
    if (hq % hkv != 0) return 0;
    if (mask != ORACLE_MASK_CAUSAL && mask != ORACLE_MASK_FULL &&
        mask != ORACLE_MASK_WINDOW)
        return 0;
    if (mask == ORACLE_MASK_WINDOW && window <= 0) return 0;
    if (n_seqs > 0 && (cu_q[0] != 0 || cu_k[0] != 0)) return 0;
    for (int b = 0; b < n_seqs; b++) {
        if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return 0;
        /* queries are the last Lq tokens of a sequence of Lk */
        if (cu_q[b + 1] - cu_q[b] > cu_k[b + 1] - cu_k[b]) return 0;
    }
    return 1;
}

static int64_t max_len(const int32_t *cu, int n_seqs) {
    int64_t m = 0;
    for (int b = 0; b < n_seqs; b++)
        if (cu[b + 1] - cu[b] > m) m = cu[b + 1] - cu[b];
    return m;
}

/*
 * Selected rows, queries against a key sequence of their own packing: row r
 * is packed query token rows[r], query head heads[r].  out is [n_rows][d];
 * lse (optional) is [n_rows].  Returns 0, or -1 on bad arguments or a row
 * index outside [0, Tq).
 */
int oracle_attention_kv_rows(const double *q, const double *k,
                             const double *v, const int32_t *cu_q,
                             const int32_t *cu_k, int32_t n_seqs, int32_t hq,
                             int32_t hkv, int32_t d, int32_t mask,
                             int32_t window, double scale, const int64_t *rows,
                             const int32_t *heads, int64_t n_rows, double *out,
                             double *lse) {
    if (!args_ok(cu_q, cu_k, n_seqs, hq, hkv, d, mask, window)) return -1;
    int64_t T = n_seqs > 0 ? cu_q[n_seqs] : 0;
    int64_t maxlen = max_len(cu_k, n_seqs);
    for (int64_t r = 0; r < n_rows; r++)
        if (rows[r] < 0 || rows[r] >= T || heads[r] < 0 || heads[r] >= hq)
            return -1;
    int bad = 0;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (maxlen + 1));
        if (!scores) {
#pragma omp atomic write
            bad = 1;
        }
        /* every thread enters the worksharing loop; one without scratch
         * skips its rows and the call reports failure */
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n_rows; r++)
            if (scores)
                token_row(q, k, v, cu_q, cu_k, n_seqs, hq, hkv, d, mask, window,
                          scale, rows[r], heads[r], out + (size_t)r * d,
                          lse ? lse + r : NULL, NULL, scores);
        free(scores);
    }
    return bad ? -1 : 0;
}

/* Every query row: out is [Tq][Hq][d], lse (optional) is [Tq][Hq]. */
int oracle_attention_kv(const double *q, const double *k, const double *v,
                        const int32_t *cu_q, const int32_t *cu_k,
                        int32_t n_seqs, int32_t hq, int32_t hkv, int32_t d,
                        int32_t mask, int32_t window, double scale,
                        double *out, double *lse) {
    if (!args_ok(cu_q, cu_k, n_seqs, hq, hkv, d, mask, window)) return -1;
    int64_t T = n_seqs > 0 ? cu_q[n_seqs] : 0;
    int64_t maxlen = max_len(cu_k, n_seqs);
    int bad = 0;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (maxlen + 1));
        if (!scores) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < T * hq; r++) {
            if (!scores) continue;
            int64_t t = r / hq;
            int h = (int)(r % hq);
            token_row(q, k, v, cu_q, cu_k, n_seqs, hq, hkv, d, mask, window,
                      scale, t, h, out + (size_t)r * d, lse ? lse + r : NULL,
                      NULL, scores);
        }
        free(scores);
    }
    return bad ? -1 : 0;
}

/* The square case (queries and keys share cu_seqlens): selected rows. */
int oracle_attention_rows(const double *q, const double *k, const double *v,
                          const int32_t *cu, int32_t n_seqs, int32_t hq,
                          int32_t hkv, int32_t d, int32_t mask, int32_t window,
                          double scale, const int64_t *rows,
                          const int32_t *heads, int64_t n_rows, double *out,
                          double *lse) {
    return oracle_attention_kv_rows(q, k, v, cu, cu, n_seqs, hq, hkv, d, mask,
                                    window, scale, rows, heads, n_rows, out,
                                    lse);
}

/* The square case: every row, out [T][Hq][d], lse (optional) [T][Hq]. */
int oracle_attention(const double *q, const double *k, const double *v,
                     const int32_t *cu, int32_t n_seqs, int32_t hq,
                     int32_t hkv, int32_t d, int32_t mask, int32_t window,
                     double scale, double *out, double *lse) {
    return oracle_attention_kv(q, k, v, cu, cu, n_seqs, hq, hkv, d, mask,
                               window, scale, out, lse);
}

/*
 * Softmax weights of one row (token t, head h) over the keys of its own
 * sequence: probs[0..n) with n the sequence length; invisible keys get 0.
 * Returns the number of visible keys, or -1 on bad arguments.
 */
int64_t oracle_attention_probs(const double *q, const double *k,
                               const double *v, const int32_t *cu,
                               int32_t n_seqs, int32_t hq, int32_t hkv,
                               int32_t d, int32_t mask, int32_t window,
                               double scale, int64_t t, int32_t h,
                               double *probs) {
    if (!args_ok(cu, cu, n_seqs, hq, hkv, d, mask, window)) return -1;
    int64_t T = n_seqs > 0 ? cu[n_seqs] : 0;
    if (t < 0 || t >= T || h < 0 || h >= hq) return -1;
    int b = seq_of_token(cu, n_seqs, t);
    int64_t n = (int64_t)cu[b + 1] - cu[b];
    int64_t lo, hi;
    visible_range(mask, window, t - cu[b], n, &lo, &hi);
    double *scores = (double *)malloc(sizeof(double) * (n + 1));
    double *row = (double *)malloc(sizeof(double) * d);
    double *vis = (double *)malloc(sizeof(double) * (n + 1));
    if (!scores || !row || !vis) {
        free(scores);
        free(row);
        free(vis);
        return -1;
    }
    int64_t cnt = token_row(q, k, v, cu, cu, n_seqs, hq, hkv, d, mask, window,
                            scale, t, h, row, NULL, vis, scores);
    for (int64_t j = 0; j < n; j++) probs[j] = 0.0;
    for (int64_t j = lo; j < hi; j++) probs[j] = vis[j - lo];
    free(scores);
    free(row);
    free(vis);
    return cnt;
}
