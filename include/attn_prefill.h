/*
 * attn_prefill.h -- C ABI of the MI355X (gfx950) exact attention-prefill library.
 *
 * The operation is exact scaled-dot-product attention over packed
 * variable-length sequences,
 *
 *     out[t, h, :] = sum_{j in J(t)} softmax_j(scale * <q[t, h], k[j, g]>) * v[j, g, :]
 *
 * with g = h / (n_q_heads / n_kv_heads).  This is the computation the paper
 * "A Modern Multimodal Assistant on a 6 GB 2011 GPU" makes fast for long
 * contexts (abstract, result (iii): the O(N^2) attention of 2k-10k-token
 * prefill, rewritten without changing its result); its gist.science technical
 * summary (Metodologia, attention rewrite) names the causal form used by the
 * language model and the bidirectional form used by the vision tower, and the
 * abstract names the window-attention merger, the third mask kind here.
 * Unlike the paper's per-head GEMMs writing an N x N score buffer, one fused
 * kernel keeps scores on chip; the N x N matrix never exists in memory.
 *
 * Visible keys J(t) of the query at local position i of a sequence of n
 * tokens (positions local to that sequence; sequences never see each other):
 *   ATTN_CAUSAL   keys 0..i (diagonal included)
 *   ATTN_FULL     keys 0..n-1 (bidirectional)
 *   ATTN_WINDOW   the block of `window` tokens holding i, blocks aligned to the
 *                 sequence start, bidirectional inside; the last block of a
 *                 sequence may be shorter.
 *
 * Layout ("packed THD"): q and out are [T][n_q_heads][head_dim], k and v are
 * [T][n_kv_heads][head_dim], contiguous row-major, T = cu_seqlens[n_seqs].
 * All four share one element type (ATTN_BF16 or ATTN_F32).  Device pointers
 * must be 16-byte aligned.  bf16 inputs are multiplied on matrix cores with
 * fp32 accumulation and a fp32 softmax; the output is rounded to bf16 (nearest
 * even).  fp32 inputs are computed in fp32 on the fp32 matrix cores (exact
 * products, fp32 sums).
 *
 * Ownership: the caller owns every buffer.  cu_seqlens is a HOST array read
 * only during the call.  The library allocates no device memory and may be
 * called from several threads on several streams.  Its only state is a pair
 * of work counters per stream and device, in a static device array that
 * comes with the library's code (causal bf16 launches of more than two items
 * per workgroup slot hand out their later items through them; each launch
 * leaves them at zero).  Launches on a stream under capture, on the
 * per-thread default stream, or on streams beyond the array's 1024 run
 * without them.
 *
 * Execution: stream-ordered and asynchronous.  The call validates its
 * arguments on the host, enqueues its kernel(s) on `stream` (a hipStream_t;
 * NULL is the default stream) and returns; `out` is ready when the stream has
 * reached that point.  Results are deterministic: the same inputs give the
 * same bits (the work counters change which workgroup computes an item, not
 * what it computes).
 *
 * Errors: every argument is checked before any device work; on error nothing
 * is enqueued and `out` is untouched.  No C++ exception crosses the ABI.
 */
#ifndef ATTN_PREFILL_H
#define ATTN_PREFILL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define ATTN_OK 0
#define ATTN_EINVAL (-1)      /* bad argument (see attn_prefill) */
#define ATTN_EUNSUPPORTED (-2) /* valid request this build does not implement */
#define ATTN_ELAUNCH (-3)      /* the HIP runtime refused the launch */

/* element types */
#define ATTN_BF16 1
#define ATTN_F32 2

/* mask kinds */
#define ATTN_CAUSAL 0
#define ATTN_FULL 1
#define ATTN_WINDOW 2

/*
 * Exact attention prefill over a packed batch.
 *
 *   q, k, v      device inputs as laid out above (read only)
 *   out          device output [T][n_q_heads][head_dim]; must not overlap
 *                q, k or v
 *   cu_seqlens   host int32[n_seqs + 1]: cu_seqlens[0] = 0, non-decreasing;
 *                sequence b is tokens cu_seqlens[b] .. cu_seqlens[b+1]-1.
 *                Empty sequences are allowed.
 *   n_seqs       number of sequences, >= 0
 *   n_q_heads    query heads, > 0, a multiple of n_kv_heads
 *   n_kv_heads   key/value heads, > 0
 *   head_dim     64, 72 or 128
 *   dtype        ATTN_BF16 or ATTN_F32
 *   mask_kind    ATTN_CAUSAL, ATTN_FULL or ATTN_WINDOW
 *   window       block length W > 0 when mask_kind is ATTN_WINDOW, else ignored
 *   scale        logit multiplier, any finite value (usually 1/sqrt(head_dim))
 *   stream       hipStream_t or NULL
 *
 * Returns ATTN_OK; ATTN_EINVAL for a NULL or misaligned pointer (pointers may
 * be NULL only when T = 0), a bad cu_seqlens, n_seqs < 0, heads <= 0 or
 * n_q_heads % n_kv_heads != 0, an unknown mask kind, window <= 0 for
 * ATTN_WINDOW, a non-finite scale, or out overlapping an input;
 * ATTN_EUNSUPPORTED for another head_dim or dtype, or sizes whose element
 * offsets do not fit in 63 bits; ATTN_ELAUNCH when the runtime reports a
 * launch failure.  T = 0 succeeds without device work.
 */
int attn_prefill(const void *q, const void *k, const void *v, void *out,
                 const int32_t *cu_seqlens, int32_t n_seqs, int32_t n_q_heads,
                 int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                 int32_t mask_kind, int32_t window, float scale, void *stream);

/*
 * The argument checks of attn_prefill alone: same arguments, same status
 * codes, but host-only -- it touches no device and no pointed-to device
 * memory, so it can run where there is no GPU.  Returns what attn_prefill
 * would return before enqueuing anything (ATTN_OK if it would launch).
 */
int attn_prefill_check(const void *q, const void *k, const void *v,
                       const void *out, const int32_t *cu_seqlens,
                       int32_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                       int32_t head_dim, int32_t dtype, int32_t mask_kind,
                       int32_t window, float scale);

/*
 * Queries against a longer key/value sequence: chunked prefill over a
 * resident key/value cache, and decode (one query per sequence).  The
 * paper's system keeps its KV cache resident on the GPU (gist.science
 * technical summary, Metodologia) and decodes over it after prefill (same
 * summary, Contribuciones Clave y Resultados: greedy decode rate); this
 * entry point computes the same exact attention for a call that brings only
 * the newest queries.
 *
 * Sequence b holds Lq_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] queries and
 * Lk_b = cu_seqlens_k[b+1] - cu_seqlens_k[b] >= Lq_b keys/values.  The
 * queries are the LAST Lq_b positions of the sequence ("bottom-right"
 * alignment): local query i sits at position p = i + Lk_b - Lq_b and sees
 *   ATTN_CAUSAL   keys 0..p
 *   ATTN_FULL     keys 0..Lk_b-1
 *   ATTN_WINDOW   the block of `window` tokens holding p (blocks aligned to
 *                 the sequence start; the last may be shorter).
 * With cu_seqlens_q equal to cu_seqlens_k element by element this is
 * attn_prefill.
 *
 *   q, out         [Tq][n_q_heads][head_dim], Tq = cu_seqlens_q[n_seqs]
 *   k, v           [Tk][n_kv_heads][head_dim], Tk = cu_seqlens_k[n_seqs]
 *   lse            NULL, or a device float32 [Tq][n_q_heads], 4-byte aligned
 *                  and overlapping no other buffer, that receives for every
 *                  row ln(sum_j exp(scale * <q, k_j>)) over its visible keys:
 *                  with out, what merges the results of two calls over
 *                  disjoint key ranges exactly,
 *                  o = (o1 e^lse1 + o2 e^lse2) / (e^lse1 + e^lse2).
 *                  Accurate to ~2^-8 absolute for bf16 inputs (the row sum is
 *                  taken over bf16-rounded probabilities), ~1e-6 for fp32.
 *   cu_seqlens_q   host int32[n_seqs + 1], cu_seqlens_q[0] = 0, non-decreasing
 *   cu_seqlens_k   host int32[n_seqs + 1], cu_seqlens_k[0] = 0, non-decreasing
 *   other arguments as for attn_prefill.
 *
 * Returns the codes of attn_prefill, plus ATTN_EINVAL when some Lq_b > Lk_b,
 * lse is misaligned or overlaps q, k, v or out.  Tq = 0 succeeds without
 * device work.  Ownership, execution and determinism as for attn_prefill.
 */
int attn_prefill_kv(const void *q, const void *k, const void *v, void *out, float *lse,
                    const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                    int32_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                    int32_t head_dim, int32_t dtype, int32_t mask_kind,
                    int32_t window, float scale, void *stream);

/* The argument checks of attn_prefill_kv alone (host-only, like
 * attn_prefill_check). */
int attn_prefill_kv_check(const void *q, const void *k, const void *v,
                          const void *out, const float *lse,
                          const int32_t *cu_seqlens_q,
                          const int32_t *cu_seqlens_k, int32_t n_seqs,
                          int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, int32_t dtype, int32_t mask_kind,
                          int32_t window, float scale);

/*
 * Decode: the attention of each sequence's newest token over its whole
 * key/value cache -- one query per sequence, the step the paper's system
 * repeats per generated token over its GPU-resident cache (gist.science
 * technical summary, Metodologia; Contribuciones Clave y Resultados: greedy
 * decode rate).  The result is attn_prefill_kv with cu_seqlens_q = 0, 1, ...,
 * n_seqs; for bf16 with head_dim 64 or 128 the visible keys of each sequence
 * are cut into chunks computed in parallel and merged exactly through their
 * references and sums, which needs a workspace.
 *
 *   q, out         [n_seqs][n_q_heads][head_dim]: row b is sequence b's query
 *   k, v           [Tk][n_kv_heads][head_dim], Tk = cu_seqlens_k[n_seqs]
 *   lse            NULL or device float32 [n_seqs][n_q_heads], as for
 *                  attn_prefill_kv
 *   cu_seqlens_k   host int32[n_seqs + 1], cu_seqlens_k[0] = 0, strictly
 *                  increasing (every sequence holds at least one key)
 *   workspace      device scratch of workspace_bytes >= the size
 *                  attn_decode_workspace_size reports for the same shape,
 *                  16-byte aligned, overlapping no other buffer; may be NULL
 *                  when that size is 0.  The caller owns it; calls that share
 *                  one workspace must be ordered (same stream).
 *   other arguments as for attn_prefill.
 *
 * Returns the codes of attn_prefill_kv, plus ATTN_EINVAL for an empty
 * sequence or a missing, small, misaligned or overlapping workspace.
 * n_seqs = 0 succeeds without device work.
 */
int attn_decode(const void *q, const void *k, const void *v, void *out, float *lse,
                const int32_t *cu_seqlens_k, int32_t n_seqs, int32_t n_q_heads,
                int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                int32_t mask_kind, int32_t window, float scale, void *workspace,
                uint64_t workspace_bytes, void *stream);

/* Bytes of workspace attn_decode needs for this shape (0 when it splits no
 * sequence's keys, or for dtypes and head dims it computes without
 * splitting); host-only.  Returns the argument codes of attn_decode. */
int attn_decode_workspace_size(const int32_t *cu_seqlens_k, int32_t n_seqs,
                               int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t head_dim, int32_t dtype,
                               int32_t mask_kind, int32_t window,
                               uint64_t *bytes);

/*
 * attn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and arguments as attn_decode, with the
 * workspace taken from a static device array of the library
 * (ATTN_DECODE_SCRATCH_BYTES, 16 MiB, one per GPU, held until the process
 * ends) instead of a caller buffer.  The array of the device the stream
 * belongs to (the current device for a NULL stream) is looked up on the first
 * call on that device; the call allocates nothing.  Every call on one GPU
 * shares that GPU's array, which keeps the last call's contents: calls that
 * overlap on one GPU (different streams or threads without ordering) race,
 * so callers order them.
 *
 * Returns the codes of attn_decode, plus ATTN_EUNSUPPORTED when the shape
 * needs more workspace than the array holds (attn_decode_workspace_size
 * reports that need) and ATTN_ELAUNCH when the array cannot be located.
 */
#define ATTN_DECODE_SCRATCH_BYTES 16777216 /* 16 MiB */
int attn_decode_noalloc(const void *q, const void *k, const void *v, void *out, float *lse,
                        const int32_t *cu_seqlens_k, int32_t n_seqs, int32_t n_q_heads,
                        int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                        int32_t mask_kind, int32_t window, float scale, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *attn_strerror(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PREFILL_H */
