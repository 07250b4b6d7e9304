/*
 * vision_block.h -- C ABI of the vision tower's attention block for MI355X
 * (gfx950): QKV projection -> exact attention -> output projection, one call.
 *
 * The paper "A Modern Multimodal Assistant on a 6 GB 2011 GPU" runs a SigLIP2
 * vision tower in FP32 whose bidirectional attention it rewrote with the same
 * GEMM method as the language model's, cutting image encoding 6x (abstract,
 * result (iii); gist.science technical summary, Metodologia, attention
 * rewrite and FP32 vision weights).  The pages give no layer formula; the
 * plain reading is the standard pre-output attention block of a transformer
 * encoder layer (its norm and MLP are other steps):
 *
 *     [q | k | v] = x W_qkv^T + b_qkv        (heads contiguous, q then k then v)
 *     a = softmax(scale q k^T) v per head    (mask: full, or blocks of `window`)
 *     out = a W_o^T + b_o
 *
 * Layout (row-major, contiguous, all of `dtype`): x [T][hidden],
 * w_qkv [3 H d][hidden], b_qkv [3 H d], w_o [hidden][H d], b_o [hidden],
 * out [T][hidden]; T = cu_seqlens[n_seqs], sequences (images) independent.
 * The projections are the vendor GEMM (hipBLASLt) with fp32 accumulation and
 * the bias added to the fp32 sums in its epilogue, so each of q, k, v and
 * out is rounded once to `dtype`; the attention (attn_prefill's kernels:
 * fp32 inputs on the fp32 matrix cores, bf16 on the bf16 ones) reads q, k
 * and v in place as the three column blocks of the [T][3 H d] projection
 * output, and its output is rounded to `dtype` before the output projection.
 *
 * Ownership and errors as for attn_prefill; the caller passes a workspace of
 * vision_attention_block_workspace_size() bytes (16-byte aligned, overlapping
 * nothing else); calls sharing one workspace must be ordered.
 */
#ifndef VISION_BLOCK_H
#define VISION_BLOCK_H

#include <stdint.h>

#include "attn_prefill.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 *   n_heads     H > 0;  head_dim d: 64, 72 or 128;  hidden > 0 (a multiple of 8)
 *   dtype       ATTN_BF16 or ATTN_F32
 *   mask_kind   ATTN_FULL or ATTN_WINDOW (with window > 0); ATTN_CAUSAL too
 *   scale       finite (usually 1/sqrt(d))
 * Returns ATTN_OK; ATTN_EINVAL for NULL or misaligned pointers (pointers may
 * be NULL only when T = 0), bad cu_seqlens, bad sizes or mask, overlap, or a
 * missing/small workspace; ATTN_EUNSUPPORTED for other head dims or dtypes or
 * sizes of 2^31 or more; ATTN_ELAUNCH when a launch fails or the vendor GEMM
 * has no algorithm for the shape or refuses the call.
 */
int vision_attention_block(const void *x, const void *w_qkv, const void *b_qkv,
                           const void *w_o, const void *b_o, void *out,
                           const int32_t *cu_seqlens, int32_t n_seqs,
                           int32_t n_heads, int32_t head_dim, int32_t hidden,
                           int32_t dtype, int32_t mask_kind, int32_t window,
                           float scale, void *workspace, uint64_t workspace_bytes,
                           void *stream);

/* Workspace bytes for T tokens (host-only): 4 T H d values of dtype, the
 * QKV projection output and the attention output (each rounded up to 256
 * bytes).  Returns ATTN_EINVAL / ATTN_EUNSUPPORTED for bad sizes, else
 * ATTN_OK. */
int vision_attention_block_workspace_size(int64_t tokens, int32_t n_heads,
                                          int32_t head_dim, int32_t hidden,
                                          int32_t dtype, uint64_t *bytes);

#ifdef __cplusplus
}
#endif

#endif /* VISION_BLOCK_H */
