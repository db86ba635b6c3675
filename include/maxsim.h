/*
 * maxsim.h -- C ABI of the MI355X (gfx950) MaxSim scoring library.
 *
 * The operator is late-interaction MaxSim, "Flash-MaxSim" Eq. (1) and the
 * "Problem" passage of the late-interaction-kernels design notes:
 *
 *     score[i, j] = sum_s  max_t  <Q[i, s], D[j, t]>
 *
 * with optional 0/1 masks: a masked doc token is -inf before every max, a
 * masked query row adds 0 to the sum (but still gets its argmax).
 *
 * Conventions shared by every entry point
 *   - Array arguments are DEVICE pointers owned by the caller. The library
 *     allocates no device memory and keeps no per-call state.
 *   - Every tensor is C-contiguous, row-major, with the embedding dimension d
 *     innermost. Any width 1 <= d <= 1024 is accepted (TileMaxSim Sec. 3
 *     "dimension tiling" and Sec. 6 Table 9, widths 64 to 768); other values
 *     return MAXSIM_ERR_UNSUPPORTED. d = 128 runs the kernels tuned for it;
 *     every other width runs a kernel that walks rows in 256-byte chunks
 *     (rows whose byte length is not a multiple of 16 are read element by
 *     element, more slowly). Those other widths also need Nd*Ld < 2^31 for
 *     uniform docs (OVERFLOW otherwise).
 *   - Q, D, dQ and dD must be 16-byte aligned (any hipMalloc or torch
 *     allocation is); every other array needs the alignment of its element
 *     type. A misaligned pointer returns MAXSIM_ERR_UNSUPPORTED.
 *   - Calls are asynchronous on `stream` (NULL = the null stream). Outputs are
 *     valid after the stream is synchronised; inputs must stay unchanged until
 *     then. Outputs must not alias inputs or each other.
 *   - All checks that need no device data run on the host BEFORE anything is
 *     enqueued; on failure the call returns a non-zero status and enqueues
 *     nothing. Device-data contents (mask bytes in {0,1}, monotone offsets,
 *     argmax in [0, Ld), int8 values != -128, finite float inputs: no NaN or
 *     Inf in Q, D or grad_scores) are preconditions: breaking them gives
 *     unspecified values, never an out-of-bounds access, with one exception:
 *     the packed forwards (maxsim_fwd_varlen, maxsim_fwd_pairs_varlen) take
 *     no packed row counts, so they read the rows cu_q and cu_d name, and
 *     offsets past the packed tensors read out of bounds.
 *   - Sizes of 0 are valid. Nq == 0 or Nd == 0 enqueues nothing.
 *   - Reductions run in a fixed order and no result is written by an atomic
 *     (the CSR and top-k builders use integer atomics on LDS only, for
 *     counts and for the sets of lanes holding equal keys, whose outcome
 *     does not depend on their order): results are bitwise reproducible run
 *     to run.
 *   - Ties among equal maxima go to the lowest doc-token index.
 */
#ifndef MAXSIM_H
#define MAXSIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAXSIM_ABI_VERSION 1

typedef struct ihipStream_t* maxsim_stream_t; /* a hipStream_t */

typedef enum {
    MAXSIM_OK = 0,
    MAXSIM_ERR_NULL = 1,        /* a required pointer is NULL */
    MAXSIM_ERR_SHAPE = 2,       /* a negative size or inconsistent sizes */
    MAXSIM_ERR_UNSUPPORTED = 3, /* d outside 1..1024, an unknown dtype, a misaligned pointer */
    MAXSIM_ERR_OVERFLOW = 4,    /* an index or an int32 sum could overflow */
    MAXSIM_ERR_LAUNCH = 5       /* the HIP runtime refused a launch */
} maxsim_status_t;

typedef enum { MAXSIM_F16 = 0, MAXSIM_BF16 = 1 } maxsim_dtype_t;

/*
 * Cross-product forward ("Flash-MaxSim" Sec. 4.1; design notes "Forward",
 * "Mask handling", "Long-query chunking").
 *   Q        [Nq, Lq, d] of `dtype`             D [Nd, Ld, d] of `dtype`
 *   q_mask   [Nq, Lq] uint8 0/1 or NULL (all rows kept)
 *   d_mask   [Nd, Ld] uint8 0/1 or NULL (all tokens valid)
 *   scores   [Nq, Nd] float32, required, fully overwritten
 *   argmax   [Nq, Nd, Lq] int32 or NULL: index t in [0, Ld) of the max for
 *            every query row (masked rows included); 0 when the doc has no
 *            valid token.
 * Products are exact in fp32 and accumulated in fp32. Errors: NULL for a
 * missing Q, D or scores (when the output is non-empty); SHAPE for negative
 * sizes; UNSUPPORTED for d outside 1..1024 or a bad dtype; OVERFLOW when
 * argmax is requested and Nq*Nd*Lq >= 2^31.
 */
maxsim_status_t maxsim_fwd(maxsim_dtype_t dtype, const void* Q, const void* D, int64_t Nq,
                           int64_t Nd, int64_t Lq, int64_t Ld, int64_t d, const uint8_t* q_mask,
                           const uint8_t* d_mask, float* scores, int32_t* argmax,
                           maxsim_stream_t stream);

/*
 * Padding-free forward ("Flash-MaxSim" Sec. 4.3.2; design notes "Varlen /
 * packed path"): sequence b occupies rows [cu[b], cu[b+1]) of its packed
 * tensor (FlashAttention cu_seqlens convention).
 *   Q     [cu_q[Nq], d]   cu_q int32 [Nq+1], cu_q[0] = 0, non-decreasing
 *   D     [cu_d[Nd], d]   cu_d int32 [Nd+1], cu_d[0] = 0, non-decreasing
 *   max_lq  an upper bound on every query length (rows beyond it are ignored)
 *   scores  [Nq, Nd] float32, required
 *   argmax  [Nq, Nd, max_lq] int32 or NULL: doc-relative index; rows s at or
 *           past the query's length, and every row of an empty doc, are 0.
 * Empty sequences contribute 0. Token offsets are 64-bit inside the kernels.
 * Q (or D) may be NULL only when its packed tensor has no rows.
 * Errors: NULL (cu_q, cu_d or scores missing), SHAPE (negative sizes,
 * max_lq < 0), UNSUPPORTED (d, dtype),
 * OVERFLOW when argmax is requested and Nq*Nd*max_lq >= 2^31.
 */
maxsim_status_t maxsim_fwd_varlen(maxsim_dtype_t dtype, const void* Q, const int32_t* cu_q,
                                  int64_t Nq, int32_t max_lq, const void* D, const int32_t* cu_d,
                                  int64_t Nd, int64_t d, float* scores, int32_t* argmax,
                                  maxsim_stream_t stream);

/*
 * INT8 x INT8 forward with one symmetric scale per tensor ("Flash-MaxSim"
 * Sec. 4.3.1, quantisation fused into the kernel).
 *   Q int8 [Nq, Lq, d], D int8 [Nd, Ld, d], values in [-127, 127]
 *   scores_i32 [Nq, Nd] int32 or NULL: the exact integer max-sum
 *   scores     [Nq, Nd] float32 or NULL: (double)sum * q_scale * d_scale,
 *              rounded once to float
 *   (at least one of the two), argmax as in maxsim_fwd.
 * Errors as maxsim_fwd, plus NULL when both score outputs are NULL and
 * OVERFLOW when Lq*d*127^2 >= 2^31 (the int32 sum could overflow).
 */
maxsim_status_t maxsim_fwd_i8(const int8_t* Q, float q_scale, const int8_t* D, float d_scale,
                              int64_t Nq, int64_t Nd, int64_t Lq, int64_t Ld, int64_t d,
                              const uint8_t* q_mask, const uint8_t* d_mask, int32_t* scores_i32,
                              float* scores, int32_t* argmax, maxsim_stream_t stream);

/*
 * INT8 x INT8 forward with one symmetric scale per token ("Flash-MaxSim"
 * Sec. 4.3.1): the similarity of query row s and doc row t is
 *     q_scale[i,s] * d_scale[j,t] * <Q[i,s], D[j,t]>
 * (exact int32 dot product, then float), through the masked max and sum of
 * maxsim_fwd.
 *   Q int8 [Nq, Lq, d], q_scale [Nq, Lq] float32
 *   D int8 [Nd, Ld, d], d_scale [Nd, Ld] float32
 *   masks as in maxsim_fwd; scores [Nq, Nd] float32; argmax as in maxsim_fwd
 *   or NULL
 * Scales must be positive and finite (the query-token scale multiplies the
 * max over doc tokens); values in [-127, 127]. Errors as maxsim_fwd.
 */
maxsim_status_t maxsim_fwd_i8_tok(const int8_t* Q, const float* q_scale, const int8_t* D,
                                  const float* d_scale, int64_t Nq, int64_t Nd, int64_t Lq,
                                  int64_t Ld, int64_t d, const uint8_t* q_mask,
                                  const uint8_t* d_mask, float* scores, int32_t* argmax,
                                  maxsim_stream_t stream);

/*
 * Scores of listed (query, doc) pairs, for rescoring candidates (the second
 * stage of the INT8 -> FP16 top-K scan, "Flash-MaxSim" Sec. 4.1.4): pair p is
 * Eq. (1) for query pair_q[p] of Q [Nq, Lq, d] against doc pair_d[p] of
 * D [Nd, Ld, d], with the masks of maxsim_fwd.
 *   pair_q, pair_d [P] int32 in [0, Nq) and [0, Nd) (a precondition: entries
 *     outside are clamped, never read out of bounds); pairs may repeat
 *   scores [P] float32; argmax [P, Lq] int32 or NULL
 * Errors: SHAPE (negative sizes; P > 0 with Nq == 0 or Nd == 0), NULL,
 * UNSUPPORTED (d, dtype, alignment), OVERFLOW (P*Lq >= 2^31 with argmax).
 */
maxsim_status_t maxsim_fwd_pairs(maxsim_dtype_t dtype, const void* Q, const void* D, int64_t Nq,
                                 int64_t Nd, int64_t Lq, int64_t Ld, int64_t d,
                                 const uint8_t* q_mask, const uint8_t* d_mask,
                                 const int32_t* pair_q, const int32_t* pair_d, int64_t P,
                                 float* scores, int32_t* argmax, maxsim_stream_t stream);

/*
 * Top-k after scoring (TileMaxSim paper, Sec. 6.8 "End-to-End Retrieval
 * Latency"): for each row i of scores [Nq, Nd] float32 (no NaN), the K
 * largest values in decreasing order; equal values are taken in increasing
 * column order (-0 and +0 are equal).
 *   ids  [Nq, Nd] int32 or NULL: idx reports ids[i, column] instead of the
 *        column (e.g. the doc ids of a candidate list)
 *   idx  [Nq, K] int32, val [Nq, K] float32 (the input values, bit for bit)
 *   rows [Nq, K] int32 or NULL: the row index i of each entry (a pair list)
 * 0 <= K <= Nd and K <= 1024. K == 0 or Nq == 0 enqueues nothing.
 * Errors: SHAPE (negative sizes, K > Nd), UNSUPPORTED (K > 1024, alignment),
 * NULL, OVERFLOW (Nq or Nd >= 2^31).
 */
maxsim_status_t maxsim_topk(const float* scores, int64_t Nq, int64_t Nd, int64_t K,
                            const int32_t* ids, int32_t* idx, float* val, int32_t* rows,
                            maxsim_stream_t stream);

/*
 * Scores of listed (query, doc) pairs of packed batches (design notes
 * "Varlen / packed path", the pair-list scorer for sparse pair lists):
 * pair p is Eq. (1) for packed query pair_q[p] against packed doc pair_d[p],
 * with the layout of maxsim_fwd_varlen.
 *   pair_q, pair_d [P] int32 in [0, Nq) and [0, Nd) (a precondition: entries
 *     outside are clamped, never read out of bounds); pairs may repeat
 *   scores [P] float32; argmax [P, max_lq] int32 or NULL (doc-relative,
 *     rows at or past the query's length 0)
 * P == 0 enqueues nothing. Errors: SHAPE (negative sizes; P > 0 with Nq == 0
 * or Nd == 0), NULL, UNSUPPORTED (d, dtype, alignment), OVERFLOW
 * (P * max_lq >= 2^31 with argmax, or Nq, Nd, P >= 2^31 - 1).
 */
maxsim_status_t maxsim_fwd_pairs_varlen(maxsim_dtype_t dtype, const void* Q, const int32_t* cu_q,
                                        int64_t Nq, int32_t max_lq, const void* D,
                                        const int32_t* cu_d, int64_t Nd, int64_t d,
                                        const int32_t* pair_q, const int32_t* pair_d, int64_t P,
                                        float* scores, int32_t* argmax, maxsim_stream_t stream);

/*
 * Padding-free backward through the saved argmax of maxsim_fwd_varlen
 * ("Flash-MaxSim" Sec. 4.2.1 Eqs. (2)-(3), Sec. 4.2.2 inverse-grid CSR,
 * Sec. 4.2.3 destination-owned reduction, on the cu_seqlens layout of
 * Sec. 4.3.2):
 *   dQ[cu_q[i] + s] = sum_j live(j) g[i,j] D[cu_d[j] + argmax[i,j,s]]
 *   dD[cu_d[j] + t] = sum over (i,s) with argmax[i,j,s] = t of g[i,j] Q[cu_q[i] + s]
 * with live(j) = doc j has a token (an empty doc takes no gradient).
 *   Q [total_q, d], D [total_d, d] packed, cu_q [Nq+1], cu_d [Nd+1] int32 as
 *     in maxsim_fwd_varlen, with cu_q[Nq] == total_q, cu_d[Nd] == total_d and
 *     every query length <= max_lq (preconditions)
 *   argmax [Nq, Nd, max_lq] int32 doc-relative (in [0, L_j) for docs with a
 *     token); grad_scores [Nq, Nd] float32
 *   dQ [total_q, d], dD [total_d, d] float32, fully overwritten
 *   csr_row_ptr [total_d + 1], csr_col_idx [total_q * Nd] int32: outputs.
 *     Row r is packed doc token r; it lists the flat sources
 *     (i*Nd + j)*max_lq + s that picked it, ascending. The sources are the
 *     total_q query rows of every doc with a token, so the first
 *     total_q * (docs with a token) entries of csr_col_idx are written.
 *     dD's first element of each such doc holds scratch until dD is written.
 * Sums run in fp32 in a fixed order: dQ over j ascending, dD over the CSR row.
 * Errors: SHAPE (negative sizes; packed rows with Nq or Nd == 0; total_q > 0
 * with max_lq == 0), NULL, UNSUPPORTED (d, dtype, alignment), OVERFLOW when
 * Nq*Nd*max_lq or total_q*Nd >= 2^31 or total_d + 1 >= 2^31.
 */
maxsim_status_t maxsim_bwd_varlen(maxsim_dtype_t dtype, const void* Q, const int32_t* cu_q,
                                  int64_t Nq, int64_t total_q, int32_t max_lq, const void* D,
                                  const int32_t* cu_d, int64_t Nd, int64_t total_d, int64_t d,
                                  const int32_t* argmax, const float* grad_scores, float* dQ,
                                  float* dD, int32_t* csr_row_ptr, int32_t* csr_col_idx,
                                  maxsim_stream_t stream);

/*
 * Backward through a saved forward argmax ("Flash-MaxSim" Sec. 4.2.1
 * Eqs. (2)-(3), Sec. 4.2.2 inverse-grid CSR, Sec. 4.2.3 destination-owned
 * reduction; design notes "Backward"):
 *   dQ[i,s] = sum_j w(i,j,s) * D[j, argmax[i,j,s]]
 *   dD[j,t] = sum over sources (i,s) with argmax[i,j,s] = t of w(i,j,s) * Q[i,s]
 * with w(i,j,s) = grad_scores[i,j] * q_mask[i,s] * live(j), live(j) = doc j
 * has at least one valid token.
 *   Q, D, masks     as in maxsim_fwd; argmax [Nq, Nd, Lq] int32 in [0, Ld)
 *   grad_scores     [Nq, Nd] float32
 *   dQ [Nq, Lq, d], dD [Nd, Ld, d] float32, fully overwritten
 *   csr_row_ptr [Nd*Ld + 1] int32, csr_col_idx [Nq*Nd*Lq] int32: outputs,
 *     the inverse map (row r = j*Ld + t lists the flat sources
 *     (i*Nd + j)*Lq + s that picked it, ascending). The backward uses no
 *     other memory: per-doc flags are kept in dD until dD is written.
 * Sums run in fp32 in a fixed order: dQ over j ascending, dD over the CSR row.
 * Errors: NULL, SHAPE (negative sizes; Ld == 0 with Nq*Nd*Lq > 0),
 * UNSUPPORTED (also misaligned pointers), OVERFLOW when Nq*Nd*Lq >= 2^31 or
 * Nd*Ld + 1 >= 2^31.
 */
maxsim_status_t maxsim_bwd(maxsim_dtype_t dtype, const void* Q, const void* D, int64_t Nq,
                           int64_t Nd, int64_t Lq, int64_t Ld, int64_t d, const uint8_t* q_mask,
                           const uint8_t* d_mask, const int32_t* argmax, const float* grad_scores,
                           float* dQ, float* dD, int32_t* csr_row_ptr, int32_t* csr_col_idx,
                           maxsim_stream_t stream);

/*
 * Chamfer distance between batches of 3-D point sets ("Flash-MaxSim"
 * Sec. 4.2.4: the MaxSim pattern with a min of squared Euclidean distances in
 * place of the max of inner products):
 *   dist1[b,p] = min_q ||P[b,p] - Q[b,q]||^2, idx1[b,p] = the lowest q attaining it
 *   dist2[b,q] = min_p ||Q[b,q] - P[b,p]||^2, idx2[b,q] likewise
 *   loss[b]    = (1/N) sum_p dist1[b,p] + (1/M) sum_q dist2[b,q]
 *   P [B, N, 3], Q [B, M, 3] float32 (finite); dist1, idx1 [B, N] float32 /
 *   int32; dist2, idx2 [B, M]; loss [B] float32 or NULL.
 * Each distance is the fp32 direct form (dx*dx + dy*dy) + dz*dz of the
 * raw coordinates at the index written beside it, and that index is one an
 * fp32 direct-form evaluation could pick: its exact squared distance exceeds
 * the exact minimum by at most gamma_5 (u = 2^-23) times their sum, ties
 * going to the lowest index. (The search itself runs on the matrix cores in
 * the expanded form with bf16 hi/lo parts of the coordinates; every
 * candidate inside that form's rounding bound of the minimum is re-evaluated
 * in the direct form, and a source with too many such candidates is decided
 * by a direct-form scan of its whole target set.)
 * The loss sums each set's distances in a fixed order whose rounding depth
 * is at most ceil(n / 16384) + 25 additions. B == 0 enqueues nothing.
 * Errors: SHAPE (negative sizes; N == 0 or M == 0 with B > 0), NULL,
 * UNSUPPORTED (misaligned pointers), OVERFLOW (B*N or B*M >= 2^31).
 */
maxsim_status_t maxsim_chamfer_fwd(const float* P, const float* Q, int64_t B, int64_t N, int64_t M,
                                   float* dist1, int32_t* idx1, float* dist2, int32_t* idx2,
                                   float* loss, maxsim_stream_t stream);

/*
 * Chamfer backward through the saved nearest-neighbour indices ("Flash-MaxSim"
 * Sec. 4.2.4 with the inverse-grid CSR of Sec. 4.2.2): the gradients of
 * sum g1*dist1 + sum g2*dist2 at fixed idx1, idx2,
 *   dP[b,p] = 2 g1[b,p] (P[b,p] - Q[b,idx1[b,p]])
 *             + sum over q with idx2[b,q] = p of 2 g2[b,q] (P[b,p] - Q[b,q])
 *   dQ[b,q] = 2 g2[b,q] (Q[b,q] - P[b,idx2[b,q]])
 *             + sum over p with idx1[b,p] = q of 2 g1[b,p] (Q[b,q] - P[b,p])
 * (the loss gradient is g1 = dloss/N, g2 = dloss/M).
 *   idx1 [B,N] in [0,M), idx2 [B,M] in [0,N) int32 (a precondition: entries
 *   outside are clamped, never read out of bounds); grad_dist1 [B,N],
 *   grad_dist2 [B,M] float32; dP [B,N,3], dQ [B,M,3] float32, overwritten.
 *   csr_row_ptr1 [B*M+1], csr_col_idx1 [B*N]: outputs, the inverse of idx1
 *   (row b*M + q lists the flat indices b*N + p that chose it, ascending);
 *   csr_row_ptr2 [B*N+1], csr_col_idx2 [B*M]: the inverse of idx2.
 * Sums run in fp32 in a fixed order (the CSR row order); no atomics on
 * results (the CSR builds count in LDS as in maxsim_bwd). dP and
 * dQ hold intermediates of the CSR build until the gradients are written.
 * B == 0 enqueues nothing. Errors as maxsim_chamfer_fwd, OVERFLOW also when
 * B*N + 1 or B*M + 1 >= 2^31.
 */
maxsim_status_t maxsim_chamfer_bwd(const float* P, const float* Q, int64_t B, int64_t N, int64_t M,
                                   const int32_t* idx1, const int32_t* idx2, const float* grad_dist1,
                                   const float* grad_dist2, float* dP, float* dQ,
                                   int32_t* csr_row_ptr1, int32_t* csr_col_idx1,
                                   int32_t* csr_row_ptr2, int32_t* csr_col_idx2,
                                   maxsim_stream_t stream);

/* A static, human-readable name of a status. Never NULL. */
const char* maxsim_status_string(maxsim_status_t s);

/* MAXSIM_ABI_VERSION of the built library. */
int maxsim_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAXSIM_H */
