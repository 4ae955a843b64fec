/*
 * osm.h -- exact softmax attention via the online-softmax recurrence,
 * for AMD Instinct MI355X (gfx950).  C ABI of libosm.so.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "Online softmax: how FlashAttention skips the N x N matrix" (dev.to)
 *   [P2] "Online softmax" (guide.dupenodi.dev)
 *   [P3] "Online softmax" (zerotofrontier.app, efficient-attention chapter)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is DEVICE memory owned by the caller (for example a
 *   PyTorch tensor's data_ptr()).  The library never allocates, frees or
 *   retains memory and is safe to call from several host threads.  Its only
 *   global state is the per-GPU scratch array of
 *   osm_attn_decode_splitkv_noalloc (reserved with the library's code, see
 *   there) and the table of its addresses.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   runs asynchronously.  Outputs are valid after the stream is synchronized.
 *   Faults inside a kernel surface at the caller's next synchronization.
 * - Tensors are contiguous, row-major.  Attention tensors are
 *   [batch][heads][positions][head_dim]; per-query LSE is [batch][heads][positions].
 * - Every argument check happens on the host BEFORE any HIP call: on any
 *   error code other than OSM_ERR_HIP nothing was launched and no output was
 *   touched.  OSM_ERR_HIP means a HIP runtime call (device query or launch)
 *   failed; some kernels of the call may already have been enqueued.
 * - No C++ exception crosses this interface.  Sizes and offsets are 64-bit
 *   where a tensor can exceed 2^31 elements.
 * - Device-side length arrays are clamped to [0, extent] by the kernels.
 * - Natural logarithms throughout the interface (m, LSE).  Kernels work in
 *   base 2 internally ([P3] "Precision, and what can still go wrong": fold
 *   log2(e) into the score scale, convert the stored log-sum-exp back).
 * - A query row with no visible key (fully masked, padded, or zero keys)
 *   produces O = +0 and LSE = -inf ([P3] same section: a row masked
 *   everywhere ends with l = 0 and is handled explicitly; [P3] "Merging
 *   partial results": the empty set's summary is (-inf, 0, 0)).
 */
#ifndef OSM_H
#define OSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    OSM_OK = 0,
    OSM_ERR_NULL = 1,        /* a required pointer is NULL */
    OSM_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or inconsistent */
    OSM_ERR_UNSUPPORTED = 3, /* valid request this library does not implement (dtype, head_dim, alignment) */
    OSM_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than osm_decode_workspace_bytes() */
    OSM_ERR_HIP = 5          /* a HIP runtime call failed (no device, launch failure) */
} osm_status;

typedef enum {
    OSM_F32 = 0,             /* IEEE fp32 */
    OSM_BF16 = 1             /* bfloat16 (8-bit exponent, 7-bit mantissa), round-to-nearest-even on output */
} osm_dtype;

typedef void *osm_stream;    /* hipStream_t */

/* Human-readable name of a status code (static string, never NULL). */
const char *osm_status_str(osm_status status);

/*
 * osm_softmax_rows -- softmax of each row of an fp32 matrix with the
 * two-pass online normalizer.
 *
 * [P3] "Two numbers that can be updated" and "The recurrence, and a proof
 * that it is right": pass 1 keeps a running maximum m and a running sum l of
 * exp(x - m), rescaling l by exp(m_old - m_new) whenever the maximum grows;
 * partial (m, l) pairs of pieces of a row are combined with the merge of
 * [P3] "Merging partial results".  Pass 2 writes y_i = exp(x_i - m) / l.
 * [P2] "Walking through it" gives the same per-tile procedure.
 *
 *   x        fp32, row r at x + r*ld_x, `cols` valid entries (read only)
 *   y        fp32, row r at y + r*ld_y (written, `cols` entries per row)
 *   rows, cols  rows >= 0, cols >= 0 (rows == 0: nothing is launched)
 *   ld_x, ld_y  row strides in elements, >= cols
 *   row_max  optional fp32 [rows]: m = max_i x_i (natural units)
 *   row_sum  optional fp32 [rows]: l = sum_i exp(x_i - m)
 * A row of all -inf (or cols == 0) gives y = 0, m = -inf, l = 0.
 * +inf or NaN inside a row is not special-cased (NaN results).
 * x and y may not overlap unless they are the same buffer with ld_x == ld_y.
 * Errors: OSM_ERR_NULL (x or y NULL with rows*cols > 0), OSM_ERR_SHAPE
 * (negative sizes, ld < cols), OSM_ERR_HIP.
 */
osm_status osm_softmax_rows(const float *x, float *y, int64_t rows, int64_t cols,
                            int64_t ld_x, int64_t ld_y, float *row_max, float *row_sum,
                            osm_stream stream);

/*
 * osm_softmax_rows_twopass -- osm_softmax_rows computed exactly as the
 * pages count it: two passes over the row in memory.
 *
 * [P3] "Three passes, and why that is a problem" and "The recurrence, and a
 * proof that it is right": pass 1 reads the row once and keeps the running
 * (m, l), pass 2 reads it again and writes y, three memory accesses per
 * element (against four for the three-pass safe softmax).  osm_softmax_rows
 * holds rows of up to 65536 columns on chip and reads them once; this entry
 * point always re-reads, for any width.  Within a row each lane runs the
 * recurrence over its share of the elements and the lanes' (m, l) are
 * merged ([P3] "Merging partial results").
 * Arguments, results, special cases and errors: as osm_softmax_rows.
 */
osm_status osm_softmax_rows_twopass(const float *x, float *y, int64_t rows, int64_t cols,
                                    int64_t ld_x, int64_t ld_y, float *row_max, float *row_sum,
                                    osm_stream stream);

/*
 * osm_attn_fwd -- fused exact attention forward, O = softmax(scale * Q K^T) V,
 * plus the per-query log-sum-exp.
 *
 * [P3] "Blocks, the bridge to FlashAttention" (the block step with matrices
 * m, l, O~: S_j = Q K_j^T scaled, m_new = max(m, rowmax S_j),
 * P~ = exp(S_j - m_new), l = exp(m - m_new) l + rowsum P~,
 * O~ = diag(exp(m - m_new)) O~ + P~ V_j), one division at the end
 * ([P3] "From weights to outputs"), LSE = m + log l ([P3] same section);
 * masks applied inside the tile loop ([P2] "Walking through it", the mask
 * paragraph).  The N x N score matrix is never written to memory ([P1] "Why
 * does removing the N x N matrix matter if the FLOPs are the same?").
 *
 *   q     [batch][heads_q][seqlen_q][head_dim]  (dtype)
 *   k, v  [batch][heads_kv][seqlen_k][head_dim] (dtype)
 *   o     [batch][heads_q][seqlen_q][head_dim]  (dtype, written)
 *   lse   fp32 [batch][heads_q][seqlen_q] (written; may be NULL)
 *   heads_q % heads_kv == 0; query head h reads key/value head
 *         h / (heads_q / heads_kv).
 *   seqlens_q, seqlens_k  optional DEVICE int32 [batch]: valid prefix
 *         lengths (right padding).  NULL = full length.  Key j is visible to
 *         query i iff i < Lq_b and j < Lk_b and (causal == 0 or j <= i).
 *         Positions past the valid length are never read into a sum; they
 *         may hold any bits (NaN included).  Query rows i >= Lq_b are
 *         written as O = 0, LSE = -inf.
 *   scale multiplies Q K^T (for example 1/sqrt(head_dim)); must be finite and > 0.
 *   causal 0 or 1 (top-left aligned: j <= i).
 * Supported: dtype OSM_BF16, head_dim 128 or 64, batch * heads_q < 2^31;
 * q, k, v and o 16-byte aligned; fp32 accumulation of both products, fp32
 * running state, O rounded to bf16 once at the end.
 * Errors: OSM_ERR_NULL, OSM_ERR_SHAPE (non-positive batch/heads/head_dim,
 * negative seqlens, heads_q % heads_kv != 0, scale not finite or <= 0),
 * OSM_ERR_UNSUPPORTED (other dtype or head_dim, a misaligned pointer,
 * batch * heads_q >= 2^31, or one head's K, Q or O rows spanning 2 GiB or
 * more: seqlen_k or seqlen_q >= 2^23 at head_dim 128, 2^24 at 64),
 * OSM_ERR_HIP.
 */
osm_status osm_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                        osm_dtype dtype, int32_t batch, int32_t heads_q, int32_t heads_kv,
                        int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                        const int32_t *seqlens_q, const int32_t *seqlens_k, float scale,
                        int32_t causal, osm_stream stream);

/*
 * osm_attn_fwd_fp8 -- the fused attention forward of osm_attn_fwd with Q, K
 * and V in FP8 (OCP E4M3 codes, one byte per element): O = v_scale *
 * softmax(scale * Q K^T) V, plus the per-query log-sum-exp.
 *
 * [P3] "Precision, and what can still go wrong": the running m, l and O~
 * stay in float32 when the inputs are FP8.  The block step is that of
 * osm_attn_fwd ([P3] "Blocks, the bridge to FlashAttention"); both matrix
 * products run on the FP8 matrix instruction: Q K^T of E4M3 codes with fp32
 * accumulation, and P~ V with the weights P~ (at most 2^8 each, relative to
 * the running reference) rounded to E4M3.
 *
 *   q     [batch][heads_q][seqlen_q][head_dim]  (E4M3 codes)
 *   k, v  [batch][heads_kv][seqlen_k][head_dim] (E4M3 codes)
 *   o     [batch][heads_q][seqlen_q][head_dim]  (bf16, written)
 *   lse   fp32 [batch][heads_q][seqlen_q] (written; may be NULL); natural log
 *         of sum_j exp(scale q.k_j)
 *   scale multiplies Q K^T (fold the dequantization factors of Q and K in
 *         here); finite and > 0.  v_scale multiplies O (the dequantization
 *         factor of V); finite.
 *   heads, seqlens_q, seqlens_k, causal: as osm_attn_fwd.  Codes past the
 *         valid lengths may hold anything (NaN codes included).
 * Supported: head_dim 128, batch * heads_q < 2^31; every pointer 16-byte
 * aligned.
 * Errors: OSM_ERR_NULL, OSM_ERR_SHAPE (as osm_attn_fwd, or v_scale not
 * finite), OSM_ERR_UNSUPPORTED (other head_dim, a misaligned pointer,
 * batch * heads_q >= 2^31, seqlen_k >= 2^24, seqlen_q >= 2^23: one head's
 * bf16 O rows spanning 2 GiB), OSM_ERR_HIP.
 */
osm_status osm_attn_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                            int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t seqlen_q,
                            int32_t seqlen_k, int32_t head_dim, const int32_t *seqlens_q,
                            const int32_t *seqlens_k, float scale, float v_scale, int32_t causal,
                            osm_stream stream);

/*
 * osm_attn_bwd_workspace_bytes -- bytes of device workspace that
 * osm_attn_bwd needs: 8 bytes per query row (batch * heads_q * seqlen_q).
 * Returns 0 for invalid sizes.
 */
size_t osm_attn_bwd_workspace_bytes(int32_t batch, int32_t heads_q, int32_t seqlen_q);

/*
 * osm_attn_bwd -- gradients of osm_attn_fwd's output with respect to Q, K
 * and V, given the gradient dO of the output and the forward's O and LSE.
 *
 * [P3] "From weights to outputs", the log-sum-exp paragraph: the stored lse
 * is all a backward pass needs to rebuild the weights, P_ij =
 * exp(s_ij - lse_i).  The pages do not write the backward out; it is the
 * derivative of the forward definition (chain rule through O = P V and the
 * softmax): dV = P^T dO, dP = dO V^T, dS = P * (dP - D) with
 * D_i = dO_i . O_i, dQ = scale dS K, dK = scale dS^T Q.  dK and dV of a
 * key/value head sum over the query heads that read it.
 *
 *   q, o, dout  [batch][heads_q][seqlen_q][head_dim] (dtype); o as written
 *         by osm_attn_fwd for the same q, k, v and arguments
 *   k, v  [batch][heads_kv][seqlen_k][head_dim] (dtype)
 *   lse   fp32 [batch][heads_q][seqlen_q], as written by osm_attn_fwd
 *   dq    shaped like q; dk, dv shaped like k (dtype, written)
 *   seqlens_q, seqlens_k, scale, causal, heads: as osm_attn_fwd.  Rows past
 *         the valid lengths are never read into a sum (q, k, v, o and dout
 *         there may hold any bits) and their gradients are written as 0;
 *         a query row that sees no key contributes nothing.
 *   workspace  DEVICE memory of at least osm_attn_bwd_workspace_bytes()
 *         bytes (caller-owned, 256-byte aligned, contents on entry ignored).
 * Two kernels are enqueued on `stream`: dQ (query-major), which also stores
 * each row's (lse, dO . O) in the workspace, then dK/dV (key-major).  No
 * atomics: the result is deterministic.
 * Supported: dtype OSM_BF16, head_dim 128 or 64, batch * heads_q < 2^31;
 * fp32 accumulation, P and dS rounded to bf16 as matrix-product operands,
 * gradients rounded to bf16 once at the end; every pointer 16-byte aligned.
 * Errors: OSM_ERR_NULL, OSM_ERR_SHAPE (as osm_attn_fwd),
 * OSM_ERR_UNSUPPORTED (other dtype or head_dim, a pointer not 16-byte
 * aligned, batch * heads_q >= 2^31, seqlen_q or seqlen_k >= 2^23 at
 * head_dim 128, 2^24 at 64),
 * OSM_ERR_WORKSPACE, OSM_ERR_HIP.
 */
osm_status osm_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                        const void *dout, const float *lse, void *dq, void *dk, void *dv,
                        osm_dtype dtype, int32_t batch, int32_t heads_q, int32_t heads_kv,
                        int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                        const int32_t *seqlens_q, const int32_t *seqlens_k, float scale,
                        int32_t causal, void *workspace, size_t workspace_bytes,
                        osm_stream stream);

/*
 * osm_decode_workspace_bytes -- bytes of device workspace that
 * osm_attn_decode_splitkv needs for these sizes: fp32 partial triples
 * m [batch][heads_q][C], l [batch][heads_q][C], O~ [batch][heads_q][C][head_dim]
 * with C = ceil(max_seqlen_k / split_size), each array 256-byte aligned.
 * Returns 0 for invalid sizes.
 */
size_t osm_decode_workspace_bytes(int32_t batch, int32_t heads_q, int32_t max_seqlen_k,
                                  int32_t head_dim, int32_t split_size);

/*
 * osm_attn_decode_splitkv -- attention of one new query token per
 * (batch, query head) against a KV cache, with the keys split into pieces
 * of `split_size` that are summarized independently and then merged.
 *
 * [P1] "How does this connect to KV-cache decoding?": the cache holds raw
 * K and V.  [P3] "Merging partial results": each piece c of a row's keys is
 * summarized by (m_c, l_c, O~_c) relative to its own maximum, and the
 * pieces are combined with the merge (associative and commutative, identity
 * (-inf, 0, 0)); [P3] "The same merge, in log-sum-exp form" names this split
 * of one query's keys across many thread blocks.
 *
 *   q        [batch][heads_q][head_dim]                 (dtype)
 *   k_cache, v_cache  [batch][heads_kv][max_seqlen_k][head_dim] (dtype)
 *   o        [batch][heads_q][head_dim]                 (dtype, written)
 *   lse      fp32 [batch][heads_q] (written; may be NULL)
 *   seqlens_k  DEVICE int32 [batch], required: keys j < L_b are visible;
 *            cache rows past L_b are never read into a sum (may hold NaN).
 *            L_b == 0 gives O = 0, LSE = -inf.
 *   scale    multiplies q . k; finite, > 0.
 *   split_size  keys per piece, a multiple of 64 in [64, 8192]; piece c
 *            covers keys [c*split, min((c+1)*split, L_b)).
 *   workspace  DEVICE memory of at least osm_decode_workspace_bytes() bytes
 *            (caller-owned, 256-byte aligned, contents on entry ignored).
 * Two kernels are enqueued on `stream`: the per-piece summaries, then the
 * merge (same as osm_merge_partials) reading the workspace.
 * Supported: dtype OSM_F32 or OSM_BF16; head_dim 64 or 128;
 * heads_q / heads_kv in {1, 2, 4, 8} with (heads_q / heads_kv) * split_size
 * <= 16384; batch * heads_q < 2^31; q, k_cache and v_cache 16-byte aligned.
 * Errors: OSM_ERR_NULL, OSM_ERR_SHAPE, OSM_ERR_UNSUPPORTED (anything outside
 * the supported set), OSM_ERR_WORKSPACE, OSM_ERR_HIP.
 */
osm_status osm_attn_decode_splitkv(const void *q, const void *k_cache, const void *v_cache,
                                   void *o, float *lse, osm_dtype dtype, int32_t batch,
                                   int32_t heads_q, int32_t heads_kv, int32_t max_seqlen_k,
                                   int32_t head_dim, const int32_t *seqlens_k, float scale,
                                   int32_t split_size, void *workspace, size_t workspace_bytes,
                                   osm_stream stream);

/*
 * osm_attn_decode_splitkv_noalloc -- osm_attn_decode_splitkv without a
 * caller-supplied workspace, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that
 * forbid allocation.  Neither this call nor anything it calls allocates or
 * frees memory.
 *
 * The piece summaries go to a scratch array the library holds on each GPU:
 * OSM_DECODE_SCRATCH_BYTES (64 MiB) of device memory, reserved when the
 * library's code is loaded on that GPU and kept until the process ends.  Its
 * address on the current device is looked up on the first call there.  Every
 * call on one GPU shares that array, so calls that overlap on one GPU (on
 * different streams, or from different host threads without ordering) race
 * and give wrong results: order them on one stream.  No part of the array
 * needs clearing between calls: every summary the merge reads is written by
 * the same call first (empty pieces' vectors included, which are weighted
 * out).
 *
 * Arguments, semantics, results and errors: as osm_attn_decode_splitkv,
 * except that there is no workspace, and OSM_ERR_WORKSPACE means that
 * osm_decode_workspace_bytes() for these sizes exceeds
 * OSM_DECODE_SCRATCH_BYTES (nothing is launched); OSM_ERR_HIP also covers a
 * failed lookup of the array's address.  The kernels are the same, so the
 * result is bit-identical to osm_attn_decode_splitkv's.
 */
#define OSM_DECODE_SCRATCH_BYTES ((size_t)64 << 20)
osm_status osm_attn_decode_splitkv_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                           void *o, float *lse, osm_dtype dtype, int32_t batch,
                                           int32_t heads_q, int32_t heads_kv, int32_t max_seqlen_k,
                                           int32_t head_dim, const int32_t *seqlens_k, float scale,
                                           int32_t split_size, osm_stream stream);

/*
 * osm_merge_partials -- merge per-piece summaries of each row into the
 * row's output and log-sum-exp.
 *
 * [P3] "Merging partial results": with m = max(m_A, m_B),
 * l = l_A exp(m_A - m) + l_B exp(m_B - m) and O~ likewise; the empty set
 * (-inf, 0, 0) is the identity and drops out: its l and O~ are loaded with
 * the other pieces but weighted out by a select, so they may hold any bits
 * (NaN included), though their memory must be valid.  Then o = O~ / l and
 * LSE = m + log l ([P3] "From weights to outputs").
 *
 *   part_m  fp32 [rows][num_splits]  piece maxima (natural-log units of the
 *           scaled scores); -inf marks an empty piece
 *   part_l  fp32 [rows][num_splits]  piece sums, relative to part_m
 *   part_o  fp32 [rows][num_splits][head_dim]  unnormalized piece outputs
 *   o       [rows][head_dim] (out_dtype, written)
 *   lse     fp32 [rows] (written; may be NULL)
 * A row whose pieces are all empty gives o = 0, LSE = -inf.
 * Supported: out_dtype OSM_F32 or OSM_BF16; head_dim 1..512;
 * num_splits >= 1.
 * Errors: OSM_ERR_NULL, OSM_ERR_SHAPE, OSM_ERR_UNSUPPORTED, OSM_ERR_HIP.
 */
osm_status osm_merge_partials(const float *part_m, const float *part_l, const float *part_o,
                              int64_t rows, int32_t num_splits, int32_t head_dim, void *o,
                              osm_dtype out_dtype, float *lse, osm_stream stream);

/*
 * osm_attn_extend -- streaming attention: fold a chunk of newly arrived keys
 * into a persisted per-row online-softmax summary.
 *
 * [P1] "How does this connect to KV-cache decoding?": as keys arrive, the
 * running state of one query is carried forward instead of recomputing over
 * the whole cache.  [P3] "Merging partial results": a row's summary
 * (m, l, O~) -- maximum of the scaled scores seen so far, sum of
 * e^(s - m), and sum of e^(s - m) v -- merges with the summary of the new
 * keys exactly (the recurrence over one more block is this merge); the
 * empty set (-inf, 0, 0) is the identity, so a fresh stream starts there.
 * The new keys are split into pieces of split_size, summarized as in
 * osm_attn_decode_splitkv, and merged with the state in place.  To read the
 * result, call osm_merge_partials(state_m, state_l, state_o, rows, 1, ...)
 * (o = O~ / l, LSE = m + log l), which leaves the state untouched.
 *
 *   q        [batch][heads_q][head_dim]            (dtype)
 *   k_new, v_new  [batch][heads_kv][n_new][head_dim] (dtype), all keys valid
 *   state_m  fp32 [batch * heads_q]  (read and written; natural-log units
 *            of the scaled scores; -inf for an empty stream)
 *   state_l  fp32 [batch * heads_q]  (read and written; 0 for an empty stream)
 *   state_o  fp32 [batch * heads_q][head_dim]  (read and written; unnormalized)
 *   scale    multiplies q . k; finite, > 0.
 *   split_size, workspace  as for osm_attn_decode_splitkv, with
 *            osm_decode_workspace_bytes(batch, heads_q, n_new, head_dim, split_size).
 * n_new == 0 leaves the state as it is (and q, k_new, v_new may be NULL).
 * Two kernels are enqueued on `stream`; calls that update the same state
 * must be ordered on one stream.
 * Supported: dtype OSM_F32 or OSM_BF16; head_dim 64 or 128;
 * heads_q / heads_kv in {1, 2, 4, 8} with (heads_q / heads_kv) * split_size
 * <= 16384; batch * heads_q < 2^31; q, k_new and v_new 16-byte aligned.
 * Errors: OSM_ERR_NULL, OSM_ERR_SHAPE, OSM_ERR_UNSUPPORTED (anything outside
 * the supported set), OSM_ERR_WORKSPACE, OSM_ERR_HIP.
 */
osm_status osm_attn_extend(const void *q, const void *k_new, const void *v_new, osm_dtype dtype,
                           int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t n_new,
                           int32_t head_dim, float scale, float *state_m, float *state_l,
                           float *state_o, int32_t split_size, void *workspace,
                           size_t workspace_bytes, osm_stream stream);

/*
 * osm_merge_lse -- combine normalized attention results of disjoint key
 * sets (for example separate osm_attn_fwd calls over chunks of the keys)
 * into the result over their union.
 *
 * [P3] "The same merge, in log-sum-exp form": each piece s carries its
 * normalized output o_s and its log-sum-exp lse_s; the union has
 * lse = log sum_s e^lse_s (computed as M + log sum_s e^(lse_s - M),
 * M = max_s lse_s) and o = sum_s e^(lse_s - lse) o_s.  A piece with
 * lse_s = -inf is the empty set: it drops out whatever its o_s holds (any
 * bits, NaN included; the memory must still be valid).
 *
 *   o_parts    [num_parts][rows][head_dim] (in_dtype)
 *   lse_parts  fp32 [num_parts][rows], natural log; each entry finite or -inf
 *   o          [rows][head_dim] (out_dtype, written)
 *   lse        fp32 [rows] (written; may be NULL)
 * A row whose pieces are all empty gives o = 0, LSE = -inf.
 * Supported: in_dtype and out_dtype OSM_F32 or OSM_BF16; head_dim 1..1024
 * (even) or 1..511 (odd); num_parts >= 1; o_parts and o 16-byte aligned
 * (they are read and written in vectors of up to 16 bytes).  fp32
 * accumulation.
 * Errors: OSM_ERR_NULL, OSM_ERR_SHAPE (rows < 0, num_parts < 1,
 * head_dim < 1), OSM_ERR_UNSUPPORTED (other dtype or head_dim, o_parts or o
 * not 16-byte aligned), OSM_ERR_HIP.
 */
osm_status osm_merge_lse(const void *o_parts, const float *lse_parts, int64_t rows,
                         int32_t num_parts, int32_t head_dim, osm_dtype in_dtype, void *o,
                         osm_dtype out_dtype, float *lse, osm_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* OSM_H */
