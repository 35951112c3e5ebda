/*
 * fa.h -- C ABI of the MI355X (gfx950) attention forward library, libfa.so.
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T) V,   softmax over each row of the scores,
 * with causal and sliding-window masks, and also returns the per-row
 * log-sum-exp lse_i = ln sum_{allowed j} exp(scale * q_i . k_j).
 * The definition is the SDPA equation of "FlashAttention" (aiwiki.page),
 * section "Attention and the memory bottleneck"; the row statistics that make
 * the tiled evaluation exact are the update equations of its section "Tiling
 * and online normalisation"; lse is the compact normalisation information of
 * its section "Training and computational complexity".  The interfaces
 * offered (multi-head, causal and sliding-window masks, variable-length
 * sequences, inference against cached keys/values) are the ones listed in its
 * section "Software integration and limitations".
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers; the caller allocates and owns
 *    every buffer (including the decode workspace).  The library allocates
 *    nothing and keeps no global state; calls are thread-safe.
 *  - Tensors are contiguous, row-major, in the layouts stated per call.
 *    q, k, v, o and the workspace must be 16-byte aligned; lse 4-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Each call only
 *    enqueues kernels on it and returns; it never synchronises.
 *  - Errors are returned as fa_status codes, never by abort.  Arguments are
 *    checked on the host before anything is launched.  Lengths held in device
 *    arrays (cu_seqlens_*, seqlens_k) cannot be checked without a sync: their
 *    validity is a precondition (stated per call); the kernels clamp every
 *    read to the buffer sizes implied by the other arguments.
 *  - There is no fallback path: an unsupported combination returns
 *    FA_ERR_UNSUPPORTED instead of running something slower.
 *  - Masks (all positions 0-based within one sequence, delta = n_k - n_q):
 *      causal:        key j allowed for query i iff j <= i + delta
 *                     (bottom-right aligned);
 *      window_left W: key j allowed iff j >= i + delta - W  (W < 0: none);
 *    with both, a row sees at most W + 1 keys.  A row with no allowed key
 *    gets O = 0 and lse = -inf.  W >= seqlen_k admits every key and is
 *    treated as no window.
 *  - Head dim d must be 64 or 128 (FA_ERR_INVALID_ARG otherwise).
 *  - Arithmetic: bf16 inputs are multiplied on matrix cores with fp32
 *    accumulation; the softmax runs in fp32 in base 2 with log2(e) folded into
 *    the scale; the probabilities are rounded to bf16 (RNE) before the P V
 *    product; O is rounded to the output type once, at the end.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, negative size, head dim d other than
                              64 or 128, bad flag, scale not finite > 0 */
  FA_ERR_UNSUPPORTED = -2, /* well-formed but not built: decode chunk size, varlen+fp32,
                              fp8 at d = 64, a grid over 2^31 workgroups, a key row (heads*d)
                              over 64 MiB */
  FA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  FA_ERR_LAUNCH = -4       /* the HIP runtime rejected a kernel launch */
} fa_status;

/*
 * fa_fwd -- attention forward (prefill), bf16 in, bf16 out.
 *
 * Dense (cu_seqlens_q == cu_seqlens_k == NULL):
 *   q, o: [batch, seqlen_q, heads, d] bf16;  k, v: [batch, seqlen_k, heads, d] bf16;
 *   lse:  [batch, heads, seqlen_q] fp32, or NULL if not wanted.
 * Varlen (both cu_seqlens non-NULL): `batch` sequences packed along the rows;
 *   q, o: [total_q, heads, d];  k, v: [total_k, heads, d];
 *   lse:  [heads, total_q] fp32 or NULL;
 *   cu_seqlens_q/k: device int32 [batch + 1], cu[0] = 0, non-decreasing;
 *   sequence s owns rows cu[s] .. cu[s+1]-1; total_q = cu_seqlens_q[batch].
 *   seqlen_q / seqlen_k are then the maximum per-sequence lengths (they size
 *   the launch grid; every per-sequence length must be <= them).
 * d: head dim, 64 or 128.  scale: finite and > 0 (usually 1/sqrt(d)).
 * causal: 0 or 1.  window_left: < 0 for no window.
 * batch, heads or seqlen_q == 0 is a valid no-op; seqlen_k == 0 gives
 * O = 0, lse = -inf for every row.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int batch, int heads, int seqlen_q, int seqlen_k, int d,
           float scale, int causal, int window_left,
           const int* cu_seqlens_q, const int* cu_seqlens_k, void* stream);

/*
 * fa_fwd_fp32 -- the same operation and argument list with fp32 q, k, v, o
 * (products and accumulation in fp32 on matrix cores, softmax in fp32).
 * Dense only: varlen returns FA_ERR_UNSUPPORTED.  d: 64 or 128.
 */
int fa_fwd_fp32(const void* q, const void* k, const void* v, void* o, float* lse,
                int batch, int heads, int seqlen_q, int seqlen_k, int d,
                float scale, int causal, int window_left,
                const int* cu_seqlens_q, const int* cu_seqlens_k, void* stream);

/*
 * fa_fwd_kvcache -- several new query tokens per sequence (chunked prefill,
 * multi-token decode) against a KV cache that already holds them, bf16.
 * The pages list inference against cached keys/values among the interfaces
 * ("FlashAttention" (aiwiki.page), section "Software integration and
 * limitations"); the queries are the last seqlen_q positions of each
 * sequence, so causal masking is bottom-right aligned (delta = L_b - seqlen_q).
 *   q, o:             [batch, seqlen_q, heads, d] bf16;
 *   k_cache, v_cache: [batch, max_len, heads, d] bf16;
 *   seqlens_k:        device int32 [batch], L_b = keys of sequence b (rows
 *                     0 .. L_b-1 of its cache block, the new tokens last);
 *                     precondition 0 <= L_b <= max_len (reads are clamped to
 *                     the block).  Rows L_b .. max_len-1 are never read.
 *   lse:              [batch, heads, seqlen_q] fp32 or NULL.
 * d: 64 or 128.  causal, window_left: as for fa_fwd, relative to the
 * bottom-right diagonal; a query with no allowed key gets O = 0, lse = -inf.
 * The same kernels as dense fa_fwd serve it (query tiles of 256 rows at
 * d = 128, 128 at d = 64), so small seqlen_q leaves most of a tile idle;
 * seqlen_q == 1 is better served by fa_decode.
 */
int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                   const int* seqlens_k, void* o, float* lse, int batch, int heads,
                   int seqlen_q, int max_len, int d, float scale, int causal,
                   int window_left, void* stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs: two fp32
 * values per (batch, head, query row).  Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_size(int batch, int heads, int seqlen_q);

/*
 * fa_bwd -- attention backward (dense), bf16: the gradients dQ, dK, dV of
 * O = softmax(scale Q K^T) V for an output gradient dO, with the masks of
 * fa_fwd.  The probabilities are recomputed from the row log-sum-exp lse that
 * fa_fwd emitted (the use the pages give for keeping it: "FlashAttention"
 * (aiwiki.page), section "Training and computational complexity").
 *   q, o, dout, dq: [batch, seqlen_q, heads, d] bf16 (o and lse from fa_fwd
 *                   on the same q, k, v, scale and masks);
 *   k, v, dk, dv:   [batch, seqlen_k, heads, d] bf16;
 *   lse:            [batch, heads, seqlen_q] fp32 (natural log; -inf for rows
 *                   with no allowed key, whose dq is 0).
 * d: 64 or 128.  Keys that no query sees get dk = dv = 0.  workspace_bytes
 * must be at least fa_bwd_workspace_size(batch, heads, seqlen_q).  Every
 * output element is written once (no atomics), so results are deterministic.
 * FA_ERR_UNSUPPORTED when 128 rows of one tensor span 2 GiB or more.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int batch, int heads, int seqlen_q,
           int seqlen_k, int d, float scale, int causal, int window_left, void* workspace,
           size_t workspace_bytes, void* stream);

/*
 * fa_decode_workspace_size -- bytes of device workspace fa_decode needs:
 * per (batch, head, chunk) an fp32 partial output of d values and one fp32
 * partial log-sum-exp, chunks = ceil(max_len / chunk).  Returns 0 for
 * invalid sizes.
 */
size_t fa_decode_workspace_size(int batch, int heads, int max_len, int d, int chunk);

/*
 * fa_decode -- one new query token per sequence against a KV cache
 * (inference with cached keys and values; the cache already holds the
 * current token, so every one of the sequence's cached keys is allowed).
 *   q, o:             [batch, 1, heads, d] bf16;
 *   k_cache, v_cache: [batch, max_len, heads, d] bf16;
 *   seqlens_k:        device int32 [batch]; precondition 0 <= L_b <= max_len.
 *                     Rows L_b .. max_len-1 of the cache are never read.
 *   lse:              [batch, heads] fp32 or NULL.
 * The keys of each sequence are split into chunks of `chunk` keys (64, 128,
 * 256 or 512); a first kernel computes each chunk's normalised partial
 * output and log-sum-exp into `workspace`, a second merges the chunks with
 * log-sum-exp weights (the rescale of the online-softmax update applied to
 * whole chunk states).  d: 64 or 128.  workspace_bytes must be at least
 * fa_decode_workspace_size(batch, heads, max_len, d, chunk).
 * L_b == 0 gives O = 0 and lse = -inf for that sequence.
 * FA_ERR_UNSUPPORTED also when one chunk of cache rows spans 2 GiB or more
 * (chunk * heads * d * 2 bytes) or batch * heads * chunks exceeds 2^31 - 1.
 */
int fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* seqlens_k,
              void* o, float* lse, int batch, int heads, int max_len, int d, float scale,
              int chunk, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of the per-GPU device array that fa_decode_noalloc keeps its chunk
 * states in (80 MiB).
 */
#define FA_DECODE_SCRATCH_BYTES ((size_t)80 << 20)

/*
 * fa_decode_noalloc -- fa_decode with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments (minus workspace),
 * layouts, kernels and results as fa_decode (bit-identical outputs).
 *   The chunk states live in a static device array of FA_DECODE_SCRATCH_BYTES
 * per GPU, created when the library's code is loaded on that GPU and held
 * until the process ends; the call allocates nothing and frees nothing.
 * Its device address is looked up once per GPU, on the first call whose
 * stream belongs to that GPU.
 *   Limit: fa_decode_workspace_size(batch, heads, max_len, d, chunk) must be
 * at most FA_DECODE_SCRATCH_BYTES, else FA_ERR_WORKSPACE (checked on the host
 * before any HIP call).  At d = 128 that is about 162k (sequence, head,
 * chunk) states, e.g. 64 sequences x 32 heads x max_len 32768 with 512-key
 * chunks (67.6 MB); the same batch in 256-key chunks (135 MB) is rejected.
 *   Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents: calls that overlap in time on one GPU (other streams,
 * other threads) race and can return wrong results, so serialise them (one
 * stream).  Each value a call reads from the array it first writes itself,
 * so nothing needs clearing between calls.
 * FA_ERR_LAUNCH also when the array's address cannot be obtained.
 */
int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                      const int* seqlens_k, void* o, float* lse, int batch, int heads,
                      int max_len, int d, float scale, int chunk, void* stream);

/*
 * fa_fwd_fp8 -- attention forward (dense) on 8-bit floating-point inputs, the
 * low-precision variant named in "FlashAttention" (aiwiki.page), section
 * "Versions".  q, k, v hold OCP e4m3 codes (1 byte each, the float8_e4m3fn
 * format: sign, 4 exponent bits with bias 7, 3 mantissa bits, 0x7F/0xFF NaN,
 * no infinities) in the layouts of fa_fwd's dense mode; each (batch, head)
 * block of a tensor carries one dequantisation factor:
 *     Q = descale_q[b * heads + h] * decode(q), likewise K and V.
 * descale_*: device fp32 [batch * heads], 4-byte aligned.  The call computes
 * the attention of fa_fwd (same scale, causal and window_left semantics) on
 * the dequantised tensors and writes o as bf16 [batch, seqlen_q, heads, d]
 * and lse as fp32 [batch, heads, seqlen_q] (lse may be NULL).
 * Arithmetic: Q K^T and P V on the fp8 matrix instructions with fp32
 * accumulation, the softmax in fp32, the probabilities rounded to e4m3 before
 * the P V product, O divided by the sum of exactly those rounded
 * probabilities (so each output row is a convex combination of V rows),
 * lse from the unrounded sum.
 * No workspace.  FA_ERR_UNSUPPORTED for d = 64 (valid, not built here) or
 * when 64 rows of heads * d bytes reach 4 GiB.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               const float* descale_q, const float* descale_k, const float* descale_v, int batch,
               int heads, int seqlen_q, int seqlen_k, int d, float scale, int causal,
               int window_left, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
