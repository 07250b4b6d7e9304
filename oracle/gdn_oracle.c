/*
 * gdn_oracle.c -- plain, slow, obviously correct fp64 CPU gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the bench's
 * CPU-baseline leg use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes.  The language backbone of the system in the paper "A
 * Modern Multimodal Assistant on a 6 GB 2011 GPU" is a hybrid gated-delta-net
 * (abstract; gist.science technical summary, Metodologia): its recurrent
 * layers carry, per head, a matrix state that every token decays by a gate
 * and corrects towards the token's value along the token's key (the delta
 * rule), and the paper rewrites that token-by-token scan into a chunked
 * intra-/inter-chunk form (abstract, result (i); summary, Metodologia,
 * recurrent layers).  The pages name the layer type and the rewrite but print
 * neither formula; the plain reading, that of the gated delta rule paper the
 * pages link (Gated Delta Networks, its recurrence), is, per head and token t
 * of a sequence, with state S (d_v x d_k), alpha_t = exp(g_t), beta_t:
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t (scale q_t)
 *
 * This file is that definition, written as the scan the chunked form
 * replaces: one token after the other, fp64 throughout, in the order
 *     S' = alpha_t S_{t-1};   u = beta_t (v_t - S' k_t);   S_t = S' + u k_t^T;
 *     o_t = S_t (scale q_t),
 * which is the recurrence above with the product expanded
 * (alpha S (I - beta k k^T) + beta v k^T = alpha S + beta (v - alpha S k) k^T).
 * Sequences of a packed batch and heads are independent; OpenMP splits
 * (sequence, head) pairs and nothing else.  Inputs are used as given (the
 * layer's own normalisation of q and k happens before this step).
 *
 * Layout: q[T][H][dk], k[T][H][dk], v[T][H][dv], g[T][H], beta[T][H],
 * out[T][H][dv], states [n_seqs][H][dv][dk], row-major fp64; cu_seqlens
 * [n_seqs+1] gives sequence b the tokens cu_seqlens[b] .. cu_seqlens[b+1]-1.
 * s0 may be NULL (zero initial state); s_final may be NULL.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

static int gdn_args_ok(const int32_t *cu, int32_t n_seqs, int32_t h, int32_t dk, int32_t dv) {
  if (n_seqs < 0 || h <= 0 || dk <= 0 || dv <= 0) return 0;
  if (n_seqs > 0 && cu == NULL) return 0;
  if (n_seqs > 0 && cu[0] != 0) return 0;
  for (int32_t b = 0; b < n_seqs; ++b)
    if (cu[b + 1] < cu[b]) return 0;
  return 1;
}

int oracle_gated_delta_rule(const double *q, const double *k, const double *v, const double *g,
                            const double *beta, const double *s0, const int32_t *cu,
                            int32_t n_seqs, int32_t h, int32_t dk, int32_t dv, double scale,
                            double *out, double *s_final) {
  if (!gdn_args_ok(cu, n_seqs, h, dk, dv)) return -1;
  const int64_t pairs = (int64_t)n_seqs * h;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t p = 0; p < pairs; ++p) {
    const int32_t b = (int32_t)(p / h), hh = (int32_t)(p % h);
    double *S = malloc(sizeof(double) * (size_t)dv * dk);
    double *u = malloc(sizeof(double) * (size_t)dv);
    if (S == NULL || u == NULL) {
      free(S);
      free(u);
#pragma omp atomic write
      bad = 1;
      continue;
    }
    if (s0 != NULL)
      memcpy(S, s0 + (size_t)p * dv * dk, sizeof(double) * (size_t)dv * dk);
    else
      memset(S, 0, sizeof(double) * (size_t)dv * dk);
    for (int32_t t = cu[b]; t < cu[b + 1]; ++t) {
      const size_t th = (size_t)t * h + hh;
      const double *qt = q + th * dk, *kt = k + th * dk, *vt = v + th * dv;
      const double alpha = exp(g[th]), bt = beta[th];
      /* S' = alpha S */
      for (int64_t i = 0; i < (int64_t)dv * dk; ++i) S[i] *= alpha;
      /* u = beta (v - S' k) */
      for (int32_t i = 0; i < dv; ++i) {
        double sk = 0.0;
        for (int32_t j = 0; j < dk; ++j) sk += S[(size_t)i * dk + j] * kt[j];
        u[i] = bt * (vt[i] - sk);
      }
      /* S = S' + u k^T */
      for (int32_t i = 0; i < dv; ++i)
        for (int32_t j = 0; j < dk; ++j) S[(size_t)i * dk + j] += u[i] * kt[j];
      /* o = S (scale q) */
      double *ot = out + th * dv;
      for (int32_t i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int32_t j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * (scale * qt[j]);
        ot[i] = acc;
      }
    }
    if (s_final != NULL) memcpy(s_final + (size_t)p * dv * dk, S, sizeof(double) * (size_t)dv * dk);
    free(S);
    free(u);
  }
  return bad ? -2 : 0;
}
