/*
 * fa.h - C ABI of the exact, IO-aware attention library for MI355X (gfx950).
 *
 * The library computes exact scaled dot-product attention tile by tile with
 * the online-softmax recurrence, so the N x N score and probability matrices
 * never reach device memory, and its backward pass rebuilds those tiles on
 * chip from Q, K, V, the saved output and one statistic per row.
 *
 * Sources (the web pages the method is taken from):
 *   "What is FlashAttention?" (interview.clozo.ai): Step 2 (online softmax),
 *     Step 3 (tiling; the query-outer loop that keeps O and the statistics on
 *     chip until one final write), Step 4 (the backward recomputes instead of
 *     storing).
 *   "FlashAttention" (deepconcepts.dev): "Why it is allowed to be exact"
 *     (max, sum, rescale by exp(m_old - m_new), divide by l at the end),
 *     "What it does not do" (the backward rebuilds S and P), "Checking it on
 *     a real system" (a backend that cannot serve a shape must refuse it
 *     rather than fall back silently).
 *   "Explain FlashAttention and why it is IO-aware" (aiinfrainterviews.com):
 *     "Keep only the state needed for the final weighted average" (scaled
 *     scores plus mask; state m, l, o), "Executable recurrence, with an
 *     empty-state policy" (fully masked rows return zeros; causal masks use
 *     absolute positions).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, contiguous, row-major [B][H][N][d] (batch, head,
 *    position, feature); K and V may have another row count Nk than Q
 *    (fa_forward), and the *_varlen calls take packed, head-major
 *    [H][total][d] batches instead.
 *  - lse is fp32 [B][H][N]: the natural-log log-sum-exp of the visible scaled
 *    scores of each query row, LSE_i = m_i + ln(l_i).
 *  - Scores are s_ij = scale * q_i . k_j.  A pair (i, j) of sequence b is
 *    visible iff j < L_b and (causal == 0 or j <= i + Nk - Nq), with absolute
 *    positions i in [0, Nq) and j in [0, Nk): the pages state the causal mask
 *    j <= i for Nq = Nk, and with Nq != Nk the queries are the last Nq
 *    positions of the sequence.  L_b = seqlens_k[b] clamped to [0, Nk], or
 *    Nk when seqlens_k is NULL.  Query rows are never masked: row i still
 *    attends to the keys below L_b that the causal mask allows.
 *  - A row with no visible key gets O = 0 and LSE = -inf (explicit empty-row
 *    policy); its gradients are 0.
 *  - Every pointer is a device pointer owned by the caller.  The library
 *    allocates and frees nothing, keeps no state between calls, and only
 *    enqueues work on `stream` (calls return without synchronising).  Calls
 *    are re-entrant.  Outputs must not alias inputs.  The one exception is
 *    fa_backward_noalloc, whose workspace is a static device array of the
 *    library shared by every call on a GPU (see there).
 *  - Data pointers must be 16-byte aligned.
 *  - Inputs must be finite; NaN or infinite inputs propagate unchecked.  Key
 *    and value rows at or past a sequence's key length are never read, so
 *    they may hold anything.
 *  - B, H or N equal to 0 is an empty problem: FA_SUCCESS, nothing is
 *    launched and pointers are not inspected.
 *
 * Errors are returned as fa_status codes, never thrown.  Argument checks
 * run before any HIP call, so an invalid call launches nothing.
 *  FA_ERROR_INVALID_VALUE  NULL data pointer, negative size, misaligned
 *                          pointer, scale not finite or not > 0, causal not
 *                          0/1, workspace missing or too small, or a problem
 *                          too large for the launch grid.
 *  FA_ERROR_UNSUPPORTED    (dtype, d) pair outside the compiled set (see
 *                          below), or one head of one sequence (N rows of d
 *                          elements) of 2^31 bytes or more; there is no
 *                          fallback path.
 *  FA_ERROR_LAUNCH         the HIP runtime reported an error when the kernel
 *                          was enqueued (hipGetLastError).  Faults inside a
 *                          kernel surface at the caller's next synchronise.
 *  FA_ERROR_SCRATCH_LIMIT  fa_backward_noalloc only: the problem needs more
 *                          workspace than the library's static array holds.
 *
 * Compiled (dtype, d) set:
 *  forward : FA_DTYPE_F32, FA_DTYPE_BF16 or FA_DTYPE_F16 with d in
 *            {64, 96, 128, 192, 256}
 *  backward: FA_DTYPE_F32, FA_DTYPE_BF16 or FA_DTYPE_F16 with d in
 *            {64, 96, 128, 192, 256}
 *            (fp32 on the fp32 MFMA: fp32 inputs, arithmetic and outputs)
 *  decode and merge: FA_DTYPE_F32, FA_DTYPE_BF16 or FA_DTYPE_F16 with d in
 *  {64, 96, 128, 192, 256}
 *  fa_forward_fp8: E4M3 inputs, bf16 output, d = 128
 * The 16-bit formats and head dimensions up to 256 are those the pages list
 * for fused kernels ("What is FlashAttention?", "Trade-offs and edge cases");
 * both 16-bit formats run the same kernels, on the MFMA of their format, with
 * fp32 accumulation and statistics.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_SUCCESS = 0,
  FA_ERROR_INVALID_VALUE = 1,
  FA_ERROR_UNSUPPORTED = 2,
  FA_ERROR_LAUNCH = 3,
  FA_ERROR_SCRATCH_LIMIT = 4 /* fa_backward_noalloc: the problem needs more
                                than FA_NOALLOC_SCRATCH_BYTES of scratch  */
} fa_status;

typedef enum {
  FA_DTYPE_F32 = 0,  /* IEEE binary32 inputs and outputs                 */
  FA_DTYPE_BF16 = 1, /* bfloat16 inputs and outputs, fp32 accumulation   */
  FA_DTYPE_F16 = 2   /* IEEE binary16 inputs and outputs, fp32 accumulation */
} fa_dtype;

/* Version of this ABI; bumped on any incompatible change. */
int fa_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_string(fa_status s);

/*
 * Forward pass: O = softmax(scale * Q K^T restricted to visible pairs) V and
 * LSE, computed tile by tile with the running maximum m, running sum l and an
 * output accumulator rescaled by exp(m_old - m_new) and divided by l after
 * the last tile ("FlashAttention", "Why it is allowed to be exact";
 * "Explain FlashAttention and why it is IO-aware", "Keep only the state
 * needed for the final weighted average").  Key tiles that are entirely
 * masked for a query tile are skipped, never loaded.
 *
 *   dtype      element type of q, k, v and o
 *   B, H       batch, heads
 *   Nq, Nk     query rows and key/value rows per head (usually equal)
 *   d          head dimension (in the compiled set)
 *   q          [B][H][Nq][d] queries; k, v [B][H][Nk][d] (read only)
 *   seqlens_k  [B] int32 key lengths on the device, or NULL for all Nk;
 *              each value is clamped to [0, Nk] inside the kernel
 *   scale      multiplier of q . k; finite and > 0 (1/sqrt(d) is usual)
 *   causal     0 or 1; 1 masks keys j > i + Nk - Nq (absolute positions;
 *              the pages state the mask for Nq = Nk, j > i, and the queries
 *              are read as the last Nq positions of the sequence, so with
 *              Nq = 1 the query sees every key, and with Nq > Nk the first
 *              Nq - Nk rows see none)
 *   o          [B][H][Nq][d] output, same dtype as q, rounded to nearest even
 *   lse        [B][H][Nq] fp32 output (natural log); the backward needs it
 *   stream     HIP stream the work is enqueued on (0 = default stream)
 * Rows that see no key get o = 0 and lse = -inf.  Nq = 0 writes nothing;
 * Nk = 0 writes those empty rows.
 * Launch: bf16 and f16 problems without key lengths and with more query
 * tiles than the device holds work-groups at once run a persistent grid (as
 * many work-groups as fit, each working through a fixed list of query
 * tiles); the result is bit for bit that of one work-group per tile.  Other
 * work running on the device at the same time only delays it.
 */
fa_status fa_forward(fa_dtype dtype, int B, int H, int Nq, int Nk, int d,
                     const void* q, const void* k, const void* v,
                     const int32_t* seqlens_k, float scale, int causal,
                     void* o, float* lse, hipStream_t stream);

/*
 * Forward pass on FP8 inputs: q, k and v hold OCP FP8 E4M3 codes (one byte
 * per element: sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
 * finite value 448) and each tensor has one fp32 descale factor, so the real
 * inputs are code * descale.  The pages name an FP8 forward among the newest
 * kernels ("What is FlashAttention?", sections "Trade-offs and edge cases"
 * and "What is FlashAttention 3?") without its scaling rules; this call computes the attention of the real inputs, exactly as
 * fa_forward defines it, with the products on the FP8 MFMA:
 *   s_ij = scale * q_descale * k_descale * (q_i . k_j over the codes),
 *   O = v_descale * softmax(s) V_codes, LSE as for fa_forward.
 * The probabilities of each key tile are rounded to E4M3 (after scaling by
 * 2^8 into its normal range) for the second product; the row sums use them
 * before rounding.
 *
 *   B, H, Nq, Nk, seqlens_k, scale, causal   as for fa_forward
 *   d                  128
 *   q                  [B][H][Nq][d] E4M3 codes; k, v [B][H][Nk][d]
 *   q_descale, k_descale, v_descale   finite and > 0
 *   o                  [B][H][Nq][d] bf16 output (round to nearest even)
 *   lse                [B][H][Nq] fp32 output (natural log)
 */
fa_status fa_forward_fp8(int B, int H, int Nq, int Nk, int d,
                         const void* q, const void* k, const void* v,
                         const int32_t* seqlens_k, float scale,
                         float q_descale, float k_descale, float v_descale,
                         int causal, void* o, float* lse, hipStream_t stream);

/*
 * Bytes of device workspace fa_backward needs for this problem (0 for an
 * empty problem); N is the number of query rows.  The workspace holds the
 * fp32 row dot products D_i = sum_t dO_it O_it, one per query row.
 */
size_t fa_backward_workspace_size(fa_dtype dtype, int B, int H, int N, int d);

/*
 * Backward pass: gradients of the scalar <dO, O> with respect to Q, K and V.
 * S and P are recomputed tile by tile from Q, K, V and the saved per-row
 * LSE instead of being stored ("What is FlashAttention?", Step 4; "FlashAttention",
 * "What it does not do"):  P_ij = exp(s_ij - LSE_i) on visible pairs,
 * dV = P^T dO, dP = dO V^T, D_i = sum_t dO_it O_it, dS = P * (dP - D),
 * dQ = scale dS K, dK = scale dS^T Q, all accumulated in fp32.
 *
 *   q, o, dout         [B][H][Nq][d]; k, v [B][H][Nk][d] (o and lse as
 *                      written by fa_forward)
 *   lse                [B][H][Nq] fp32
 *   Nq, Nk, seqlens_k, scale, causal  exactly as passed to fa_forward
 *   dq                 [B][H][Nq][d] output; dk, dv [B][H][Nk][d] outputs;
 *                      same dtype as q (keys no query sees get zeros)
 *   workspace          device buffer of at least
 *                      fa_backward_workspace_size(...) bytes, 16-byte
 *                      aligned; its contents on entry do not matter
 *   workspace_bytes    size of that buffer
 * The result is deterministic: it does not depend on scheduling order.
 */
fa_status fa_backward(fa_dtype dtype, int B, int H, int Nq, int Nk, int d,
                      const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse,
                      const int32_t* seqlens_k, float scale, int causal,
                      void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * The three launches fa_backward makes, callable one by one (same arguments,
 * same validation, same results).  Issued in this order on one stream they
 * are exactly fa_backward; dkdv and dq only read `delta` and may run
 * concurrently on two streams once preprocess has finished.
 *
 * fa_backward_preprocess: delta[b][h][i] = sum_t dout_it o_it in fp32 (the
 *   row term D of dS = P * (dP - D)); N is Nq; delta is [B][H][Nq] fp32,
 *   16-byte aligned.
 * fa_backward_dkdv: dk and dv.  Each work-group keeps a block of keys and
 *   their gradient accumulators on chip and streams query tiles past them,
 *   recomputing S and P per tile.
 * fa_backward_dq: dq.  Each work-group keeps a block of query rows on chip
 *   and streams key tiles past them, recomputing S and P per tile.
 */
fa_status fa_backward_preprocess(fa_dtype dtype, int B, int H, int N, int d,
                                 const void* o, const void* dout, float* delta,
                                 hipStream_t stream);
fa_status fa_backward_dkdv(fa_dtype dtype, int B, int H, int Nq, int Nk, int d,
                           const void* q, const void* k, const void* v,
                           const void* dout, const float* lse, const float* delta,
                           const int32_t* seqlens_k, float scale, int causal,
                           void* dk, void* dv, hipStream_t stream);
fa_status fa_backward_dq(fa_dtype dtype, int B, int H, int Nq, int Nk, int d,
                         const void* q, const void* k, const void* v,
                         const void* dout, const float* lse, const float* delta,
                         const int32_t* seqlens_k, float scale, int causal,
                         void* dq, hipStream_t stream);

/*
 * fa_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not call hipMalloc, harnesses that forbid allocation).  The workspace
 * fa_backward takes (one fp32 per query row, fa_backward_workspace_size
 * bytes) lives instead in a static device array of the library,
 * FA_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held from the library's first
 * use of that GPU until the process ends.  This call allocates nothing and
 * calls no allocating routine; it uses the copy of the array on the calling
 * thread's current device, so `stream` must belong to that device.
 *
 * Arguments, layouts, results and the other errors are those of fa_backward
 * (same kernels, bit-identical outputs).  Limit: B * H * Nq <= 8,388,608
 * query rows; a larger problem returns FA_ERROR_SCRATCH_LIMIT before any HIP
 * call.  Every call on one GPU shares that GPU's array and it keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap
 * on one GPU, on different streams or host threads, race on it and must be
 * serialised by the caller.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
fa_status fa_backward_noalloc(fa_dtype dtype, int B, int H, int Nq, int Nk, int d,
                              const void* q, const void* k, const void* v,
                              const void* o, const void* dout, const float* lse,
                              const int32_t* seqlens_k, float scale, int causal,
                              void* dq, void* dk, void* dv, hipStream_t stream);

/*
 * Packed batches: B sequences of different lengths stored back to back
 * without padding.  The tensors are head-major, and sequence b owns query
 * rows cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 and key rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1 of every head.  The pages define
 * attention for one sequence; each packed sequence is computed as its own
 * problem of that definition, exactly as fa_forward / fa_backward compute
 * one (batch, head): the causal mask uses the sequence's own lengths
 * (a query sees keys j <= i + nk_b - nq_b, positions counted from the
 * sequence's first row), and nothing crosses from one sequence to another.
 *
 *   B                  number of sequences
 *   total_q, total_k   query / key rows per head of the packed tensors
 *   max_seqlen_q, max_seqlen_k
 *                      the longest sequence's query / key rows: the launch
 *                      covers that many rows per sequence, and a longer
 *                      sequence is cut to it
 *   q, o               [H][total_q][d]; k, v [H][total_k][d]
 *   lse                [H][total_q] fp32
 *   cu_seqlens_q, cu_seqlens_k
 *                      [B + 1] int32 offsets on the device, non-decreasing,
 *                      from >= 0 to <= total_q (total_k), 4-byte aligned.
 *                      The kernels clamp every offset and length to the
 *                      buffers, so a malformed array gives meaningless
 *                      values but never an access outside q, k, v, o or lse
 *                      (overlapping sequences write the same rows in an
 *                      unspecified order).
 *   dtype, d, scale, causal, stream   as for fa_forward
 * Rows that belong to no sequence are neither read nor written.  A sequence
 * without keys gets o = 0 and lse = -inf on its rows.
 */
fa_status fa_forward_varlen(fa_dtype dtype, int B, int H, int total_q, int total_k,
                            int max_seqlen_q, int max_seqlen_k, int d,
                            const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            float scale, int causal, void* o, float* lse,
                            hipStream_t stream);

/*
 * Backward of fa_forward_varlen; the arguments are those of fa_forward_varlen
 * and of fa_backward: dq, o, dout [H][total_q][d], dk, dv [H][total_k][d].
 * The workspace needs fa_backward_workspace_size(dtype, 1, H, total_q, d)
 * bytes.  Key rows of a sequence that no query sees get zero gradients; rows
 * that belong to no sequence are not written.
 */
fa_status fa_backward_varlen(fa_dtype dtype, int B, int H, int total_q, int total_k,
                             int max_seqlen_q, int max_seqlen_k, int d,
                             const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             float scale, int causal, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * Decoding: one new query row per (batch, head) against a key/value cache,
 * split over the key dimension ("FlashAttention" (deepconcepts.dev), "What
 * it does not do": a decode step has a single query row and reads the whole
 * cache; the parallelism that helps is across the sequence dimension when the
 * batch is too small to fill the GPU, flash-decoding).  The query attends to
 * every cached key j < L_b (no causal flag: it is the newest position).  The
 * keys of each (batch, head) are cut into parts whose length the library
 * chooses (a multiple of 64, at most 4096); one work-group per part writes
 * the part's normalised output and LSE to the workspace, then
 * fa_merge_states combines the parts.
 *
 *   q          [B][H][d] query rows (read only)
 *   k, v       [B][H][N][d] cache of capacity N (read only); N <= 2^24
 *   seqlens_k  [B] int32 cached lengths on the device, clamped to [0, N],
 *              or NULL for N
 *   scale      multiplier of q . k; finite and > 0
 *   o          [B][H][d] output, same dtype as q (zeros for an empty cache)
 *   lse        [B][H] fp32 output, natural log (-inf for an empty cache)
 *   workspace  device buffer of at least fa_decode_workspace_size(...)
 *              bytes, 16-byte aligned; contents on entry do not matter
 * The result is deterministic.
 */
size_t fa_decode_workspace_size(fa_dtype dtype, int B, int H, int N, int d);
fa_status fa_decode(fa_dtype dtype, int B, int H, int N, int d,
                    const void* q, const void* k, const void* v,
                    const int32_t* seqlens_k, float scale,
                    void* o, float* lse,
                    void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * Merge of partial results of the same softmax rows over disjoint key sets:
 * the rescale-and-add step of the online recurrence applied to whole parts
 * ("FlashAttention", "Why it is allowed to be exact"; "Explain
 * FlashAttention and why it is IO-aware", "Keep only the state needed for
 * the final weighted average").  For each row,
 *   LSE = ln sum_s exp(lse_s),  O = sum_s exp(lse_s - LSE) o_s;
 * parts with lse_s = -inf contribute nothing, and a row whose parts are all
 * -inf gets O = 0 and LSE = -inf.
 *
 *   rows       number of rows (0 is an empty call)
 *   n_parts    parts per row, 1 <= n_parts <= 4096
 *   o_parts    [rows][n_parts][d] fp32 normalised partial outputs
 *   lse_parts  [rows][n_parts] fp32 partial LSEs (natural log)
 *   o          [rows][d] output in dtype
 *   lse        [rows] fp32 output, or NULL
 */
fa_status fa_merge_states(fa_dtype dtype, int rows, int n_parts, int d,
                          const float* o_parts, const float* lse_parts,
                          void* o, float* lse, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
