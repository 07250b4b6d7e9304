/*
 * gdn_prefill.h -- C ABI of the MI355X (gfx950) chunked gated-delta-rule
 * prefill.
 *
 * The language backbone of the system in the paper "A Modern Multimodal
 * Assistant on a 6 GB 2011 GPU" is a hybrid gated-delta-net: beside its
 * attention layers, recurrent layers carry per head a matrix state that each
 * token decays by a gate and corrects towards its value along its key
 * (abstract; gist.science technical summary, Metodologia).  The paper's
 * prefill rewrites that token-by-token scan into a chunked intra-/inter-chunk
 * form, 2.8x faster than the scan once its forward-substitution kernel was
 * fixed (abstract, result (i); summary, Metodologia, recurrent layers).  The
 * pages print no formula; this library computes the recurrence of the gated
 * delta rule (the paper the pages link, Gated Delta Networks), per sequence
 * and head, with state S (d_v x d_k), alpha_t = exp(g_t):
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t (scale q_t)
 *
 * S_{-1} is the sequence's initial state (zero when none is given), and the
 * state after its last token is its final state.  q and k are used as given
 * (the layer normalises them before this step; unit-norm keys keep the
 * recurrence contractive).
 *
 * Layout ("packed THD"): q, k [T][n_heads][d_k], v and out [T][n_heads][d_v],
 * bf16, contiguous; g and beta [T][n_heads] float32; states
 * [n_seqs][n_heads][d_v][d_k] float32 (row-major: S[v][k]).  T =
 * cu_seqlens[n_seqs].  Device pointers must be 16-byte aligned (g and beta:
 * 4-byte).
 *
 * Method: chunks of 64 tokens in the WY form.  A first kernel, parallel over
 * (chunk, head), builds each chunk's lower-triangular system, inverts it by
 * blocked forward substitution, and stores the chunk's key/value
 * combinations, its masked intra-chunk scores and gates in the workspace; a
 * second kernel runs the chunks of each (sequence, head, 32 value rows) in
 * order, carrying the state in fp32.  Products run on bf16 MFMA with fp32
 * accumulation (operands rounded to bf16); the state is fp32 between chunks.
 *
 * Ownership, execution, errors: as for attn_prefill (attn_prefill.h) -- the
 * caller owns every buffer, the call checks all arguments on the host before
 * any device work, enqueues on `stream` and returns; the same status codes.
 */
#ifndef GDN_PREFILL_H
#define GDN_PREFILL_H

#include <stdint.h>

#include "attn_prefill.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Chunked gated-delta-rule prefill over a packed batch.
 *
 *   q, k           device bf16 [T][n_heads][head_dim_k]
 *   v              device bf16 [T][n_heads][head_dim_v]
 *   g              device float32 [T][n_heads]: log of the decay, <= 0
 *                  (alpha = exp(g)); finite
 *   beta           device float32 [T][n_heads]: write strength, usually in
 *                  [0, 1]
 *   initial_state  NULL (zero state) or device float32
 *                  [n_seqs][n_heads][head_dim_v][head_dim_k]
 *   out            device bf16 [T][n_heads][head_dim_v]; overlaps no input
 *   final_state    NULL or device float32 [n_seqs][n_heads][head_dim_v]
 *                  [head_dim_k]; may be the same buffer as initial_state
 *                  (updated in place), overlaps nothing else
 *   cu_seqlens     host int32[n_seqs + 1], cu_seqlens[0] = 0, non-decreasing;
 *                  empty sequences pass their initial state through
 *   n_heads        > 0
 *   head_dim_k/v   128 / 128
 *   dtype          ATTN_BF16
 *   scale          multiplier of q, finite (usually 1/sqrt(head_dim_k))
 *   workspace      device scratch of at least gdn_prefill_workspace_size()
 *                  bytes, 16-byte aligned, overlapping no other buffer; may be
 *                  NULL when that size is 0.  Calls sharing one workspace must
 *                  be ordered (same stream).
 *
 * Returns ATTN_OK; ATTN_EINVAL for a NULL or misaligned pointer (pointers may
 * be NULL only when T = 0, except the states), a bad cu_seqlens, n_seqs < 0,
 * n_heads <= 0, a non-finite scale, overlapping buffers, or a missing, small
 * or misaligned workspace; ATTN_EUNSUPPORTED for other head dims or dtypes or
 * sizes whose offsets overflow; ATTN_ELAUNCH when the runtime refuses a launch.
 */
int gdn_prefill(const void *q, const void *k, const void *v, const float *g,
                const float *beta, const float *initial_state, void *out,
                float *final_state, const int32_t *cu_seqlens, int32_t n_seqs,
                int32_t n_heads, int32_t head_dim_k, int32_t head_dim_v,
                int32_t dtype, float scale, void *workspace,
                uint64_t workspace_bytes, void *stream);

/* Bytes of workspace gdn_prefill needs for this shape (host-only): per
 * 64-token chunk and head, 73984 bytes.  Returns the shape codes of
 * gdn_prefill. */
int gdn_prefill_workspace_size(const int32_t *cu_seqlens, int32_t n_seqs,
                               int32_t n_heads, int32_t head_dim_k,
                               int32_t head_dim_v, int32_t dtype,
                               uint64_t *bytes);

/* The argument checks of gdn_prefill alone (host-only, touches no device
 * memory): what gdn_prefill would return before enqueuing anything. */
int gdn_prefill_check(const void *q, const void *k, const void *v,
                      const float *g, const float *beta,
                      const float *initial_state, const void *out,
                      const float *final_state, const int32_t *cu_seqlens,
                      int32_t n_seqs, int32_t n_heads, int32_t head_dim_k,
                      int32_t head_dim_v, int32_t dtype, float scale,
                      const void *workspace, uint64_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PREFILL_H */
