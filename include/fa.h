/*
 * fa.h -- C ABI of libfa, the MI355X (gfx950) exact attention forward pass
 * and its backward pass.
 *
 *   O   = softmax(scale * Q K^T [+ causal mask]) V
 *   LSE = log-sum-exp of each row of the scaled, masked logits (natural log)
 *
 * The operation is the one defined on the page "解析 FlashAttention（2）：
 * FlashAttention-v1 前向传播" (section 1.1 for S = QK^T, P = softmax(S),
 * O = PV; section 2.1, eq. (2)-(5) for the safe softmax; section 3.2 for the
 * per-row output with its maximum m_i and sum l_i) and computed tile by tile
 * with online softmax (same page, sections 2.5-3.12 and its Algorithm 1;
 * loop order: query tiles outside, key/value tiles inside, as in the
 * FlashAttention-2 loop of "在线 Softmax 与 FlashAttention", loop-order
 * lesson).  The causal mask is the top-left one of that lesson's causal part:
 * query i sees keys j <= i; tiles wholly in the future are skipped.
 * The N x N score and probability matrices never reach device memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout:    q, k, v, o are dense, contiguous [B, H, N, d] row-major tensors
 *            (d fastest).  lse is a dense fp32 [B, H, N] tensor.  The query
 *            and key sequences have the same length N.
 * Memory:    every pointer is a device address the caller allocated (e.g. a
 *            torch tensor on the current device) and keeps ownership of.  The
 *            library allocates nothing and keeps no state between calls; it
 *            is re-entrant and may be called concurrently on different
 *            streams.  o and lse must not overlap q, k, v or each other.
 *            Every pointer must be 16-byte aligned.
 * Stream:    the work is enqueued on `stream` (NULL = the null stream) and
 *            the call returns without waiting for it.
 * LSE:       lse[b,h,i] = ln( sum_{j visible to i} exp(scale * q_i . k_j) ),
 *            in fp32.  (The pages keep the row maximum m and sum l, first
 *            page, section 4, last steps of Algorithm 1; this library returns
 *            the single number m*scale + ln(l) instead.)
 * Shapes:    B, H, N >= 1; N <= 2^30; B*H*N*d < 2^40; B*H*ceil(N/128)
 *            <= 2^22 (a launch-size limit: no kernel then launches 2^31 or
 *            more work-items; decode also needs B*H*Nq <= 2^22); the head dim
 *            d is a multiple of 16 from 16 to 128 for every entry point.
 * scale:     finite and > 0 (usually 1/sqrt(d)).
 * causal:    0 = no mask, any other value = top-left causal mask.
 * Errors:    all argument checks run before anything is enqueued; a failed
 *            check returns its code and touches no memory.  After a launch,
 *            a HIP launch error is reported as FA_ERR_HIP.  Errors that
 *            happen later on the device surface at the caller's next
 *            synchronisation, as for any asynchronous HIP work.  No C++
 *            exception crosses this interface.
 */
#ifndef FA_H_
#define FA_H_

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = 1,     /* a required pointer is NULL                       */
    FA_ERR_SHAPE = 2,    /* B, H or N < 1, N > 2^30, B*H*N*d >= 2^40, or     */
                         /* B*H*ceil(N/128) > 2^22 (launch-size limit)       */
    FA_ERR_HEADDIM = 3,  /* d not supported by the entry point (see Shapes)  */
    FA_ERR_SCALE = 4,    /* scale is not finite, or not > 0                  */
    FA_ERR_ALIGN = 5,    /* a pointer is not 16-byte aligned                 */
    FA_ERR_HIP = 6,      /* the kernel launch failed (hipGetLastError)       */
    FA_ERR_ALIAS = 7,    /* an output overlaps an input or another output    */
    FA_ERR_WORKSPACE = 8,/* workspace NULL or smaller than required          */
    FA_ERR_DTYPE = 9,    /* unknown element type                             */
    FA_ERR_STRIDE = 10,  /* strides invalid (row stride < d or > 2^24,       */
                         /* negative, or an output whose rows overlap)       */
    FA_ERR_SCRATCH = 11  /* fa_decode_noalloc: partials exceed its scratch   */
};

/* Bytes of the fixed device scratch of fa_decode_noalloc. */
#define FA_DECODE_SCRATCH_BYTES (17ul << 20)

/* Element types of fa_fwd_ex. */
enum fa_dtype { FA_DTYPE_BF16 = 0, FA_DTYPE_FP16 = 1 };

/*
 * fa_fwd -- bf16 inputs and output, fp32 accumulation.
 *   q, k, v : const bf16 [B, H, N, d]   (bf16 = IEEE binary32 upper half)
 *   o       : bf16 [B, H, N, d], written; each element rounded to nearest
 *             even from the fp32 result
 *   lse     : fp32 [B, H, N], written
 * Scores, softmax statistics and the output accumulator are fp32; the
 * probabilities are rounded to bf16 before they multiply V (the row sums use
 * the unrounded fp32 values).  Returns an fa_status code.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N, int d, float scale, int causal,
           hipStream_t stream);

/*
 * fa_fwd_f32 -- the same operation with fp32 inputs and output and fp32
 * arithmetic throughout (no rounding to a narrower type anywhere).
 * Same parameter list and conventions as fa_fwd.
 */
int fa_fwd_f32(const float *q, const float *k, const float *v, float *o,
               float *lse, int B, int H, int N, int d, float scale, int causal,
               hipStream_t stream);

/*
 * fa_bwd -- gradients of fa_fwd for an output gradient dout: dq = dL/dQ,
 * dk = dL/dK, dv = dL/dV when dout = dL/dO.
 *
 * The pages describe the backward pass as recomputation: the scores and
 * probabilities are rebuilt tile by tile from Q, K and the row statistics the
 * forward pass kept, never stored as N x N matrices ("解析 FlashAttention（2）",
 * section 1.2 (3) and the remark after Algorithm 1 that m and l are kept for
 * the backward pass; Triton page, section 5.1).  The gradients themselves are
 * the chain rule through the forward definition:
 *   P = exp(scale * Q K^T [masked] - LSE),  dV = P^T dout,  dP = dout V^T,
 *   dS = P o (dP - delta),  delta_i = dout_i . o_i,
 *   dQ = scale * dS K,  dK = scale * dS^T Q.
 *
 *   q, k, v : const bf16 [B, H, N, d], the forward pass's inputs
 *   o       : const bf16 [B, H, N, d], fa_fwd's output for them
 *   dout    : const bf16 [B, H, N, d]
 *   lse     : const fp32 [B, H, N], fa_fwd's LSE for the same q, k, v,
 *             scale and causal
 *   dq, dk, dv : bf16 [B, H, N, d], written (rounded to nearest even from
 *             the fp32 accumulators)
 *   delta   : fp32 [B, H, N], caller-provided workspace; on completion it
 *             holds delta_i = dout_i . o_i (fp32 sum of bf16 products)
 * Arithmetic: products on bf16 inputs with fp32 accumulation; P and dS are
 * rounded to bf16 before they enter the products that need them.
 * Two kernels are enqueued on `stream` (dq and delta first, then dk and dv).
 * Shapes, scale, causal, alignment and errors as for fa_fwd; none of dq, dk,
 * dv, delta may overlap an input or another output (FA_ERR_ALIAS).
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, void *dq, void *dk, void *dv, float *delta,
           int B, int H, int N, int d, float scale, int causal,
           hipStream_t stream);

/*
 * fa_decode -- attention of a few queries over many keys (a decode step):
 * O = softmax(scale * Q K^T [+ mask]) V with its LSE, for Nq <= 16 queries
 * per (batch, head) over Nk >= Nq keys.
 *
 * The queries are the LAST Nq positions of the sequence.  With causal != 0,
 * query i (0-based) sits at position Nk - Nq + i and sees keys
 * j <= Nk - Nq + i (for Nq = Nk this is fa_fwd's mask; a single query sees
 * every key, as the unit-12 causal lesson of "在线 Softmax 与 FlashAttention"
 * says of a single-token decode step).  The key axis is split into chunks
 * processed in parallel (split-K, named in that course's loop-order lesson);
 * each chunk's partial output and LSE are merged with the two-block rule of
 * "解析 FlashAttention（2）", eq. (17)/(20) and (37):
 *   LSE = ln sum_s e^(LSE_s),   O = sum_s e^(LSE_s - LSE) O_s.
 *
 *   q         : const bf16 [B, H, Nq, d]
 *   k, v      : const bf16 [B, H, Nk, d]
 *   o         : bf16 [B, H, Nq, d], written (rounded to nearest even)
 *   lse       : fp32 [B, H, Nq], written (natural log, as fa_fwd)
 *   num_splits: chunks of the key axis; <= 0 chooses automatically (about
 *               2048 chunks over all heads for one or two queries, 768 for
 *               more, at least 64 keys each); a larger request is cut to
 *               ceil(Nk / 64).  Chunks are whole multiples of 64 keys (96
 *               for three or more queries), so fewer chunks than asked for
 *               may run.
 *   workspace : device memory of at least fa_decode_workspace_size(...)
 *               bytes for the fp32 partials; its contents on return are
 *               unspecified; it must not overlap any other argument
 * Scores, statistics and sums are fp32.  Shapes: B, H >= 1, 1 <= Nq <= 16,
 * Nq <= Nk <= 2^30, d a multiple of 16 up to 128, B*H*Nk*d < 2^40,
 * B*H*ceil(Nk/128) <= 2^22 and B*H*Nq <= 2^22 (launch-size limits).  Two
 * kernels (chunks, then merge) are enqueued on `stream`; one query over at
 * most 16 chunks, or two over at most 8, run chunks and merge in a single
 * kernel (one workgroup per head, merging in LDS) and leave the workspace
 * untouched.  Errors as for fa_fwd, plus FA_ERR_WORKSPACE.
 */
int fa_decode(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int Nq, int Nk, int d, float scale, int causal,
              int num_splits, void *workspace, size_t workspace_bytes,
              hipStream_t stream);

/* Bytes of workspace fa_decode needs for these arguments (0 if they are
 * invalid shapes). */
size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d, int num_splits);

/*
 * fa_decode_noalloc -- fa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): no workspace argument; the fp32 partials go to a fixed
 * scratch array that the library holds in device memory, one per GPU, of
 * FA_DECODE_SCRATCH_BYTES (17 MiB) for the life of the process.  The call
 * allocates nothing and makes no allocating runtime call.
 *
 * Arguments, layout and results as for fa_decode (same kernels, same
 * num_splits rule); a call whose partials, fa_decode_workspace_size(B, H,
 * Nq, Nk, d, num_splits) bytes, exceed FA_DECODE_SCRATCH_BYTES returns
 * FA_ERR_SCRATCH before anything is enqueued (pass a smaller num_splits).
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (on different streams, or from different threads without
 * ordering) race on it and must not be issued; calls ordered on one stream
 * are safe.  The scratch needs no clearing (the split kernel writes every
 * partial it reads back).  Errors as for fa_decode with FA_ERR_SCRATCH in
 * place of FA_ERR_WORKSPACE; FA_ERR_HIP also if the scratch's device address
 * cannot be obtained.
 */
int fa_decode_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal,
                      int num_splits, hipStream_t stream);

/*
 * fa_decode_ex -- fa_decode generalised the way fa_fwd_ex generalises
 * fa_fwd: fp16 as well as bf16 tensors, and strided views (the Triton page's
 * kernel interface, "手写 FlashAttention", section 3.4), e.g. a key/value
 * cache kept as [B, Nk, H, d].
 *
 *   dtype   : FA_DTYPE_BF16 or FA_DTYPE_FP16 -- the type of q, k, v and o
 *             (scores, statistics and sums fp32; with three or more queries
 *             the products run on that type's MFMA and the probabilities
 *             are rounded to it; o rounded to nearest even)
 *   strides : host array of 12 element strides, for q, k, v, o in turn:
 *             batch, head, row (q and o have Nq rows, k and v Nk), with the
 *             rules of fa_fwd_ex; lse stays a dense fp32 [B, H, Nq] and the
 *             workspace is fa_decode_workspace_size(...) bytes as for
 *             fa_decode.
 * Other arguments, ownership and errors as for fa_decode, plus FA_ERR_DTYPE
 * and FA_ERR_STRIDE.  With the dense strides and dtype bf16 this runs
 * exactly fa_decode's kernels.
 */
int fa_decode_ex(int dtype, const void *q, const void *k, const void *v, void *o, float *lse,
                 int B, int H, int Nq, int Nk, int d, float scale, int causal, int num_splits,
                 void *workspace, size_t workspace_bytes, const int64_t *strides,
                 hipStream_t stream);

/*
 * fa_fwd_ex -- fa_fwd generalised to fp16 as well as bf16 tensors, and to
 * strided views, as the Triton page's kernel takes per-tensor strides
 * ("手写 FlashAttention", section 3.4, its kernel's parameter list).
 *
 *   dtype   : FA_DTYPE_BF16 or FA_DTYPE_FP16 -- the type of q, k, v and o
 *             (the MFMA products use that type's gfx950 instruction;
 *             probabilities are rounded to it before P.V; accumulation,
 *             scores and statistics are fp32; o is rounded to nearest even)
 *   strides : host array of 12 element strides, for q, k, v, o in turn:
 *             batch, head, row.  The d elements of a row are contiguous.
 *             Element (b, h, n, t) of q is q[b*s0 + h*s1 + n*s2 + t].
 *             Row strides must lie in [d, 2^24], every stride must be >= 0
 *             and a multiple of 8 (16-byte rows); input strides may be 0
 *             (e.g. k, v shared by all heads); o's rows must not overlap
 *             each other.  lse stays a dense fp32 [B, H, N].
 * Other arguments and errors as for fa_fwd, plus FA_ERR_DTYPE and
 * FA_ERR_STRIDE.  No part of o may overlap q, k, v or lse.  With the dense
 * strides of [B, H, N, d] and dtype bf16 this runs exactly fa_fwd's kernel.
 */
int fa_fwd_ex(int dtype, const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int N, int d, float scale, int causal,
              const int64_t *strides, hipStream_t stream);

/*
 * fa_bwd_ex -- fa_bwd generalised the way fa_fwd_ex generalises fa_fwd:
 * fp16 as well as bf16 tensors, and strided views (the Triton page's kernel
 * interface, "手写 FlashAttention", section 3.4; its section 5.1 on the
 * backward pass).
 *
 *   dtype   : FA_DTYPE_BF16 or FA_DTYPE_FP16 -- the type of q, k, v, o,
 *             dout, dq, dk and dv (products on that type's MFMA, P and dS
 *             rounded to it before the products that take them; scores,
 *             statistics and accumulation fp32; gradients rounded to
 *             nearest even)
 *   strides : host array of 24 element strides, for q, k, v, o, dout, dq,
 *             dk, dv in turn: batch, head, row (the d elements of a row
 *             contiguous), with the rules of fa_fwd_ex; the rows of dq, dk
 *             and dv must not overlap each other.  lse and delta stay dense
 *             fp32 [B, H, N].
 * Other arguments, ownership and errors as for fa_bwd, plus FA_ERR_DTYPE and
 * FA_ERR_STRIDE; no part of dq, dk, dv or delta may overlap an input or
 * another output.  fp16 holds dS = P (dP - delta) and the gradients, so
 * |dO| |V| and the gradients must stay within fp16's range.  With the dense
 * strides and dtype bf16 this runs exactly fa_bwd's kernels.
 */
int fa_bwd_ex(int dtype, const void *q, const void *k, const void *v, const void *o,
              const void *dout, const float *lse, void *dq, void *dk, void *dv, float *delta,
              int B, int H, int N, int d, float scale, int causal, const int64_t *strides,
              hipStream_t stream);

/*
 * fa_fwd_kv_outer -- the same result as fa_fwd (O and LSE, bf16 in/out) in
 * the loop order of Algorithm 1 of "解析 FlashAttention（2）：FlashAttention-v1
 * 前向传播" (section 4): key/value blocks outside, query blocks inside, the
 * output O and the statistics l, m written back to device memory after every
 * step and read again at the next one.  It exists to
 * measure that order against fa_fwd's (query blocks outside, which the
 * unit-12 loop-order lesson of "在线 Softmax 与 FlashAttention" shows gives
 * the same O without those round trips).
 *
 * One kernel launch per 64-key block j is enqueued on `stream`; each covers
 * the 128-row query blocks that can see block j.  Per (i, j) it computes the
 * block statistics with the block's own maximum, merges them with the
 * stored ones and rescales the stored, normalised O_i, as the algorithm's
 * inner step does.  The state O, l, m is fp32 in the caller's workspace (at least
 * fa_fwd_kv_outer_workspace_size bytes; contents on return unspecified; no
 * overlap with any other argument).  Arguments, shapes and errors otherwise
 * as for fa_fwd, plus FA_ERR_WORKSPACE.
 */
int fa_fwd_kv_outer(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int N, int d, float scale, int causal,
                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace fa_fwd_kv_outer needs (0 for invalid shapes). */
size_t fa_fwd_kv_outer_workspace_size(int B, int H, int N, int d);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
