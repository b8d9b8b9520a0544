/*
 * dflash2.h - C ABI of the DFlash2 draft-block head on AMD Instinct MI355X (gfx950).
 *
 * Three operations of the DFlash2 drafter:
 *   1. the block-local grouped dynamic causal convolution that wraps every
 *      draft sublayer (dflash2_conv_prepare / dflash2_conv_finish);
 *   2. full-vocabulary unary LM-head logits with a per-position top-K
 *      (dflash2_unary_topk);
 *   3. the candidate selector S_t(a,b) = U_t(b) + <A(a) * H(h_t), B(b)>,
 *      walked greedily from the anchor (dflash2_selector_walk), sampled from
 *      the same scores (dflash2_selector_sample), or scored in one
 *      shot with teacher-forced predecessors (dflash2_selector_score_tf).
 *
 * Sources, cited by page title and section:
 *   [Speculators] "DFlash2" page of the vLLM Speculators user guide.
 *   [SpecForge]   "DFlash2" concept page of the SpecForge docs.
 *   [verl PR]     "feat: add DFlash2 drafter training backend" (verl-SpeCo #62).
 *   [Explainer]   "DFlash 2 Explanation".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer is a DEVICE pointer owned by the caller, except where noted.
 *   The library never allocates, never frees and keeps no state between calls
 *   (dflash2_selector_walk_noalloc alone works in a library-owned device
 *   array, see there).  Calls are re-entrant; concurrent calls must use
 *   distinct workspaces.
 * - All work is enqueued on `stream` (a hipStream_t; NULL is the default
 *   stream).  No entry point synchronises, except dflash2_read_device_status.
 * - Matrices are row-major.  Weights follow the [out, in] layout of a linear
 *   layer: w_lm [V, H], w_proj [2*T*G, H], w_h [r, H]; the selector codebooks
 *   are materialised tables cb_pred = A [V, r] and cb_succ = B [V, r].
 * - `dtype` (dflash2_dtype) is the storage type of every activation and weight
 *   argument marked "dtype" below: IEEE float32, or bf16 (the high 16 bits of
 *   a float32).  All arithmetic accumulates in float32.
 * - Errors the host can see are returned BEFORE anything is enqueued:
 *   DFLASH2_ERR_NULL for a missing required pointer, DFLASH2_ERR_SHAPE for a
 *   size that breaks a rule of the method, DFLASH2_ERR_UNSUPPORTED for a size
 *   the kernels do not handle, DFLASH2_ERR_DTYPE for an unknown dtype,
 *   DFLASH2_ERR_ALIAS for an output that overlaps an input it must not,
 *   DFLASH2_ERR_WORKSPACE for a workspace smaller than
 *   dflash2_workspace_bytes().  A failed launch returns DFLASH2_ERR_LAUNCH.
 * - Token ids found out of range [0, V) on the device (anchors, predecessors,
 *   gold ids, candidate ids) are never dereferenced: the affected outputs get
 *   a sentinel (id -1, NaN score, valid 0) and a status word in the workspace
 *   is set; dflash2_read_device_status() reports it as
 *   DFLASH2_ERR_DEVICE_ID_RANGE.  The word is cleared at the start of every
 *   call that takes a workspace.
 * - Workspaces: caller-owned device memory of at least
 *   dflash2_workspace_bytes() bytes, any contents.  Calls that share a
 *   workspace must not run concurrently.
 * - Alignment: every floating-point array (dtype, float32) and the
 *   workspace start on a multiple of 16 bytes, every int32 array on a
 *   multiple of 4 (uint8 arrays: any address); the kernels read and write
 *   them 16 bytes at a time.  A pointer that is not returns
 *   DFLASH2_ERR_UNSUPPORTED.  (Allocations are; a view stays aligned when its
 *   offset is a multiple of 8 bf16 or 4 float32 elements.)
 */
#ifndef DFLASH2_H_
#define DFLASH2_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DFLASH2_OK = 0,
    DFLASH2_ERR_NULL = 1,
    DFLASH2_ERR_SHAPE = 2,
    DFLASH2_ERR_DTYPE = 3,
    DFLASH2_ERR_UNSUPPORTED = 4,
    DFLASH2_ERR_ALIAS = 5,
    DFLASH2_ERR_WORKSPACE = 6,
    DFLASH2_ERR_LAUNCH = 7,
    DFLASH2_ERR_DEVICE_ID_RANGE = 8
} dflash2_status;

typedef enum { DFLASH2_F32 = 0, DFLASH2_BF16 = 1 } dflash2_dtype;

typedef enum {
    DFLASH2_OP_UNARY_TOPK = 0,
    DFLASH2_OP_SELECTOR_WALK = 1,
    DFLASH2_OP_SELECTOR_TF = 2,
    DFLASH2_OP_SELECTOR_CE_BACKWARD = 3,
    DFLASH2_OP_DECODE_HEAD = 4
} dflash2_op;

/* Kernel limits (sizes beyond them return DFLASH2_ERR_UNSUPPORTED). */
#define DFLASH2_MAX_TOP_K 64
#define DFLASH2_MAX_TAPS 16
#define DFLASH2_MAX_BLOCK_SIZE 64
#define DFLASH2_MAX_RANK 4096     /* selector rank */

/*
 * Pre-sublayer half of the conv wrapper ([verl PR] "What DFlash2 adds";
 * [Speculators] "Local Convolution"; [Explainer] "Problem 2").
 *
 * One bias-free projection of the current hidden state gives the dynamic
 * corrections of both the input and the output kernel:
 *   c[n, s, j, g] = sum_h w_proj[(s*T + j)*G + g, h] * x[n, h],
 * s = 0 input kernel, s = 1 output kernel, j < T tap, g < G = H / group_size.
 * The input is convolved at once, block-locally:
 *   x_out[n, h] = sum_{j <= min(T-1, n mod bs)} (base[0, j, h] + c[n, 0, j, h / gs]) * x[n - j, h]
 * (a tap that would reach before the start of its anchor block reads zero;
 * [verl PR] "Two deltas", item 1), and the output kernel's dynamic part is
 * handed to dflash2_conv_finish:  k_post[n, j, g] = c[n, 1, j, g].
 *
 *   dtype       storage type of x, w_proj, base, x_out
 *   n_tokens    N, flattened draft length; must be a multiple of block_size
 *   block_size  bs, anchor-block length
 *   hidden      H;  taps T in [1, min(block_size, 16)];  group_size divides H
 *   x           [N, H]       sublayer input
 *   w_proj      [2*T*G, H]   kernel projection
 *   base        [2, T, H]    static per-channel kernels (input, output)
 *   x_out       [N, H]       convolved input (one rounding to dtype); must not overlap x
 *   k_post      [N, T, G]    float32, dynamic part of the output kernel
 * Rules (DFLASH2_ERR_SHAPE): N % bs != 0, T < 1 or T > bs, H % gs != 0, sizes < 1.
 */
dflash2_status dflash2_conv_prepare(int dtype, int64_t n_tokens, int32_t block_size,
                                    int32_t hidden, int32_t taps, int32_t group_size,
                                    const void *x, const void *w_proj, const void *base,
                                    void *x_out, float *k_post, void *stream);

/*
 * Post-sublayer half of the conv wrapper ([verl PR] "What DFlash2 adds"):
 *   y_out[n, h] = sum_{j <= min(T-1, n mod bs)} (base[1, j, h] + k_post[n, j, h / gs]) * y[n - j, h]
 * y [N, H] is the sublayer's output, k_post comes from dflash2_conv_prepare,
 * y_out [N, H] must not overlap y.  Same rules as dflash2_conv_prepare.
 */
dflash2_status dflash2_conv_finish(int dtype, int64_t n_tokens, int32_t block_size,
                                   int32_t hidden, int32_t taps, int32_t group_size,
                                   const void *y, const float *k_post, const void *base,
                                   void *y_out, void *stream);

/*
 * Unary LM-head logits over the full vocabulary and the per-row top-K
 * candidate lattice ([Speculators] "Candidate Selector" and its full-vocabulary
 * requirement; [Explainer] "Component Breakdown", shared lm_head and top-16
 * per position).
 *   U[n, v] = sum_h h[n, h] * w_lm[v, h]   (float32 accumulation; never written out)
 *   out_ids[n, :]  the top_k ids of row n by U, value descending, lower id
 *                  first on an exact tie;   out_vals[n, :] their U values.
 *   If gold_ids is given: out_gold_logit[n] = U[n, gold_ids[n]] (required then).
 *
 *   n_rows N >= 1, hidden H, vocab V, top_k K in [1, min(V, 64)]
 *   h [N, H] dtype; w_lm [V, H] dtype; gold_ids [N] int32 or NULL
 *   out_ids [N, K] int32; out_vals [N, K] float32; out_gold_logit [N] float32
 *   workspace: device bytes, at least dflash2_workspace_bytes(DFLASH2_OP_UNARY_TOPK, ...)
 */
dflash2_status dflash2_unary_topk(int dtype, int64_t n_rows, int32_t hidden, int32_t vocab,
                                  int32_t top_k, const void *h, const void *w_lm,
                                  const int32_t *gold_ids, int32_t *out_ids, float *out_vals,
                                  float *out_gold_logit, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * dflash2_unary_topk with the unary-logit transforms of the draft config and
 * the candidate metrics of the same pass ([SpecForge] "Export and serve":
 * output_multiplier and final_logit_softcapping act on the unary logits;
 * [Explainer] "Problem 1", recall@K; [SpecForge] "Selector objective and
 * schedule", selector coverage; [verl PR] "What DFlash2 adds", unary
 * candidate recall and target mass).
 *   U'[n, v] = softcap(output_multiplier * U[n, v]),
 *   softcap(x) = c * tanh(x / c) with c = final_logit_softcapping (0: off).
 *   out_ids / out_vals: the top_k of U' (ids as dflash2_unary_topk: the
 *   transform is increasing), values U'; out_gold_logit[n] = U'[n, gold[n]].
 *   out_lse[n] = log sum_v exp(U'[n, v]) over the full vocabulary, or NULL.
 *   out_gold_prob[n] = exp(U'[n, gold[n]] - lse[n]), the gold's softmax
 *   probability (target mass), or NULL; needs gold_ids.
 *   out_gold_hit[n] = 1 if gold[n] is among out_ids[n, :] (recall@K and
 *   coverage indicator), else 0; uint8 or NULL; needs gold_ids.
 *   output_multiplier > 0 and finite, final_logit_softcapping >= 0 and finite
 *   (DFLASH2_ERR_SHAPE otherwise).  Asking for out_lse or out_gold_prob
 *   adds a sum of exponentials to every logit tile (about a fifth more time
 *   on many bf16 rows, a few percent at decode sizes); without them the
 *   kernels are those of dflash2_unary_topk.
 *   w_h [rank, H] dtype and out_g [N, rank] float32, both or neither: the
 *   selector's context projection g = h w_hᵀ of the same rows ([verl PR]
 *   "What DFlash2 adds", H(h)), for dflash2_selector_walk, _sample and
 *   _score_tf to take as their g.  On the many-row bf16 path its weight rows
 *   stream through the LM-head kernel after the vocabulary's, as extra
 *   tiles, so the selector adds no pass over h of its own; elsewhere it is
 *   one more launch (the sums may round in another order than the selector
 *   calls' own projection: float32 over H products either way).
 *   rank >= 1 (DFLASH2_ERR_SHAPE), a multiple of 8 and at
 *   most DFLASH2_MAX_RANK (DFLASH2_ERR_UNSUPPORTED) when out_g is given.
 *   Outputs must not overlap each other, the workspace or any input.
 *   Workspace: that of DFLASH2_OP_UNARY_TOPK.  Other rules as
 *   dflash2_unary_topk.
 */
dflash2_status dflash2_unary_topk_ex(int dtype, int64_t n_rows, int32_t hidden, int32_t vocab, int32_t top_k,
                                     const void *h, const void *w_lm, const int32_t *gold_ids,
                                     float output_multiplier, float final_logit_softcapping, const void *w_h,
                                     int32_t rank, int32_t *out_ids, float *out_vals, float *out_gold_logit,
                                     float *out_lse, float *out_gold_prob, uint8_t *out_gold_hit, float *out_g,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Greedy selector walk per anchor block ([verl PR] "What DFlash2 adds",
 * selector equation; [Speculators] "Candidate Selector"; [Explainer]
 * "Problem 1" and the "One Cycle, Step by Step" diagram: candidate lists plus
 * the last verified token in, one path out).
 *   g[n] = w_h h[n]  (the context projection H(h_n), float32)
 *   S_t(a, b) = cand_vals[n, slot(b)] + sum_r cb_pred[a, r] * g[n, r] * cb_succ[b, r]
 * with n = blk*bs + t.  path[blk, 0] = anchor_ids[blk]; for t = 1..bs-1 the
 * candidate of row n with the highest S_t(path[blk, t-1], .) is taken (lowest
 * slot on an exact tie).  With float32 codebooks or fewer than 128 blocks,
 * every adjacent pair is scored at once, each predecessor keeps its best
 * successor, and one wave follows those links from the anchor; with bf16
 * codebooks and 128 blocks or more the walk follows
 * the path, scoring each position against the previous pick only (about half
 * the gathered bytes).  The scores, and so the path, are the same either way.
 *
 *   n_blocks, block_size (<= 64), hidden H, vocab V, rank r (multiple of 8, <= 4096),
 *   top_k K (<= 64)
 *   h [N, H] dtype (N = n_blocks*bs); w_h [r, H] dtype
 *   g [N, r] float32 or NULL: the context rows formed beforehand (the out_g of
 *   dflash2_unary_topk_ex); then h and w_h are not read and may be NULL, and
 *   no projection runs (hidden is still checked; the workspace is the same).
 *   Without g, h and w_h are required (DFLASH2_ERR_NULL).
 *   cb_pred, cb_succ [V, r] dtype; cand_ids [N, K] int32; cand_vals [N, K] float32
 *   anchor_ids [n_blocks] int32
 *   out_path [n_blocks, bs] int32; out_path_score [n_blocks, bs] float32 or NULL
 *   (0 at position 0, S_t of the chosen step elsewhere).
 */
dflash2_status dflash2_selector_walk(int dtype, int32_t n_blocks, int32_t block_size,
                                     int32_t hidden, int32_t vocab, int32_t rank, int32_t top_k,
                                     const void *h, const void *w_h, const float *g, const void *cb_pred,
                                     const void *cb_succ, const int32_t *cand_ids,
                                     const float *cand_vals, const int32_t *anchor_ids,
                                     int32_t *out_path, float *out_path_score, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * dflash2_selector_walk for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that forbid allocation): the same
 * inputs, outputs and kernels, without a workspace argument.  The status word
 * and the context rows live in a library-owned device array of
 * DFLASH2_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends; its
 * address on a device is looked up on the first call there.  Nothing is
 * allocated.  Sizes whose walk workspace (dflash2_workspace_bytes with
 * DFLASH2_OP_SELECTOR_WALK) exceeds that array return DFLASH2_ERR_UNSUPPORTED.
 * Every call on one GPU shares the array and overwrites what the last call
 * left there: calls that overlap on one GPU (other streams, other threads)
 * race and must not be issued.  The status word cannot be read back;
 * out-of-range ids show in the outputs (path -1, score NaN).
 */
#define DFLASH2_NOALLOC_SCRATCH_BYTES (8u * 1024u * 1024u + 256u)
dflash2_status dflash2_selector_walk_noalloc(int dtype, int32_t n_blocks, int32_t block_size,
                                             int32_t hidden, int32_t vocab, int32_t rank, int32_t top_k,
                                             const void *h, const void *w_h, const float *g,
                                             const void *cb_pred,
                                             const void *cb_succ, const int32_t *cand_ids,
                                             const float *cand_vals, const int32_t *anchor_ids,
                                             int32_t *out_path, float *out_path_score, void *stream);

/*
 * Sampled selector walk per anchor block ([Explainer] "Problem 1", the
 * paragraph after the selector equation: the walk may sample from the same
 * scores instead of following the best successor; "Draft-Verify Cycle"
 * flowchart, the walk node).  Same inputs, scores and outputs as
 * dflash2_selector_walk, except that the pick at t is the first argmax over
 * the slots j of
 *   S_t(path[blk, t-1], c_{t,j}) / temperature + G[blk, t, j],
 * G[blk, t, j] = -log(-log(u)), u = ((x >> 8) + 1/2) / 2^24 with x the first
 * word of Philox4x32-10 at counter (j, t, blk, 0) under the key (seed & 0xffffffff,
 * seed >> 32): a draw from softmax(S_t / temperature) over the candidates
 * (Gumbel-max), reproducible from (seed, blk, t).  out_path_score holds the
 * picked candidate's S_t, without the noise.
 *   temperature > 0 and finite (DFLASH2_ERR_SHAPE otherwise); the workspace
 *   is that of DFLASH2_OP_SELECTOR_WALK.
 */
dflash2_status dflash2_selector_sample(int dtype, int32_t n_blocks, int32_t block_size,
                                       int32_t hidden, int32_t vocab, int32_t rank, int32_t top_k,
                                       const void *h, const void *w_h, const float *g, const void *cb_pred,
                                       const void *cb_succ, const int32_t *cand_ids,
                                       const float *cand_vals, const int32_t *anchor_ids,
                                       float temperature, uint64_t seed, int32_t *out_path,
                                       float *out_path_score, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * Decode step of the draft head in two launches: the unary top-K lattice of
 * dflash2_unary_topk and the greedy walk of dflash2_selector_walk, for at most
 * 8 rows ([Explainer] "One Cycle, Step by Step": the lattice from the draft's
 * hidden states, then one path per block from the last verified token;
 * [Speculators] "Candidate Selector").  The context projection's weight rows
 * w_h stream through the LM-head kernel after the vocabulary's, so the
 * selector adds no pass over h of its own; one workgroup then merges the
 * candidate lists and walks every block.
 *   out_ids / out_vals: as dflash2_unary_topk (no gold ids);
 *   out_path / out_path_score: as dflash2_selector_walk on that lattice.
 * With w_h NULL (and cb_pred, cb_succ, anchor_ids, out_path, out_path_score
 * NULL) only the lattice is formed; giving some of the selector's arguments
 * but not all of w_h, cb_pred, cb_succ, anchor_ids and out_path returns
 * DFLASH2_ERR_NULL.
 *   dtype must be DFLASH2_BF16; N = n_blocks * block_size <= 8; hidden a
 *   multiple of 512 (DFLASH2_ERR_UNSUPPORTED otherwise); rank as
 *   dflash2_selector_walk (pass 0 without the selector); top_k in
 *   [1, min(V, 64)].
 *   h [N, H], w_lm [V, H], w_h [r, H], cb_pred / cb_succ [V, r]: bf16;
 *   anchor_ids [n_blocks] int32; out_ids [N, K] int32; out_vals [N, K] float32;
 *   out_path [n_blocks, bs] int32; out_path_score [n_blocks, bs] float32 or NULL.
 *   workspace: at least dflash2_workspace_bytes(DFLASH2_OP_DECODE_HEAD, N,
 *   hidden, vocab, rank (0 without the selector), top_k) bytes, any contents.
 */
dflash2_status dflash2_decode_head(int dtype, int32_t n_blocks, int32_t block_size, int32_t hidden,
                                   int32_t vocab, int32_t rank, int32_t top_k, const void *h,
                                   const void *w_lm, const void *w_h, const void *cb_pred,
                                   const void *cb_succ, const int32_t *anchor_ids, int32_t *out_ids,
                                   float *out_vals, int32_t *out_path, float *out_path_score,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Teacher-forced selector scoring of every row at once ([verl PR] "Selector
 * training objective"; [Speculators] "Training Objective"; [SpecForge]
 * "Selector objective and schedule").
 *   out_scores[n, k] = S(pred_ids[n], cand_ids[n, k]) over the strict set;
 *   out_best_ids[n]  = the candidate with the highest score (lowest slot on ties).
 * With gold_ids: the forced set C' replaces slot K-1 by (gold, gold_logit[n])
 * when force[n] != 0 and the gold id is not among the candidates; a row is
 * valid when its gold id is in C'; out_ce[n] = logsumexp_k S'[n, k] -
 * S'[n, gold] for valid rows, 0 otherwise; out_valid[n] in {0, 1}.
 *
 *   h [N, H], w_h [r, H], cb_pred/cb_succ [V, r]: dtype
 *   g [N, r] float32 or NULL: precomputed context rows, as in
 *   dflash2_selector_walk (then h and w_h may be NULL)
 *   cand_ids [N, K] int32, cand_vals [N, K] float32, pred_ids [N] int32
 *   gold_ids [N] int32 or NULL; force [N] uint8 or NULL (needs gold_ids);
 *   gold_logit [N] float32, required when force is given
 *   out_scores [N, K] float32; out_best_ids [N] int32;
 *   out_ce [N] float32 and out_valid [N] uint8: required when gold_ids is given
 */
dflash2_status dflash2_selector_score_tf(int dtype, int64_t n_rows, int32_t hidden,
                                         int32_t vocab, int32_t rank, int32_t top_k,
                                         const void *h, const void *w_h, const float *g,
                                         const void *cb_pred,
                                         const void *cb_succ, const int32_t *cand_ids,
                                         const float *cand_vals, const int32_t *pred_ids,
                                         const int32_t *gold_ids, const uint8_t *force,
                                         const float *gold_logit, float *out_scores,
                                         int32_t *out_best_ids, float *out_ce,
                                         uint8_t *out_valid, void *workspace,
                                         size_t workspace_bytes, void *stream);

/*
 * Backward of the teacher-forced selector CE ([verl PR] "Selector training
 * objective": the selector's inputs are detached, so the CE trains only the
 * selector's own parameters; [SpecForge] "Selector objective and schedule",
 * the stop-gradient switch; [Speculators] "Training Objective", the forced
 * set).  With the forced set C', valid rows and CE exactly as in
 * dflash2_selector_score_tf (gold_ids required), and L = sum over valid rows
 * of grad_ce[n] * CE[n], ADDS dL/dA into grad_pred, dL/dB into grad_succ and
 * dL/dW_H into grad_wh.  h and the unary logits (cand_vals, gold_logit) are
 * constants: no gradient flows into them.
 *   h [N, H], w_h [r, H], cb_pred/cb_succ [V, r]: dtype
 *   cand_ids [N, K] int32, cand_vals [N, K] float32, pred_ids [N] int32,
 *   gold_ids [N] int32; force [N] uint8 or NULL; gold_logit [N] float32,
 *   required when force is given; grad_ce [N] float32 (dL/dCE per row, e.g.
 *   the loss weight over the number of valid rows)
 *   grad_pred [V, r], grad_succ [V, r], grad_wh [r, H]: float32, accumulated
 *   into (zero them for a fresh gradient); distinct, and overlapping no input
 *   and not the workspace; ordinary device memory (not host-mapped).
 *   The (row, slot) contributions are counting-sorted by target codebook row
 *   and each row's contributions are summed in chunks of 64 and added with
 *   one read-modify-write per chunk (a row with more than 64 contributions
 *   adds its chunks with float atomics).  The placement inside a row's
 *   segment follows atomic counters, so the summation order of grad_pred and
 *   grad_succ, and with it their last bits, may differ from call to call;
 *   grad_wh is summed in a fixed order.
 *   out_ce [N] float32, out_valid [N] uint8: optional (NULL to skip), as in
 *   dflash2_selector_score_tf
 *   workspace: at least dflash2_workspace_bytes(DFLASH2_OP_SELECTOR_CE_BACKWARD, ...)
 * Rows whose ids fall outside [0, V) are excluded (no gradient, valid 0) and
 * set the device status word.
 */
dflash2_status dflash2_selector_ce_backward(int dtype, int64_t n_rows, int32_t hidden, int32_t vocab,
                                            int32_t rank, int32_t top_k, const void *h, const void *w_h,
                                            const void *cb_pred, const void *cb_succ,
                                            const int32_t *cand_ids, const float *cand_vals,
                                            const int32_t *pred_ids, const int32_t *gold_ids,
                                            const uint8_t *force, const float *gold_logit,
                                            const float *grad_ce, float *grad_pred, float *grad_succ,
                                            float *grad_wh, float *out_ce, uint8_t *out_valid,
                                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace bytes an operation needs (host only, no device call).  `op` is a
 * dflash2_op; n_rows is N (for the walk: n_blocks * block_size).  Arguments an
 * op does not use are ignored.  Returns 0 for an unknown op or invalid sizes.
 */
size_t dflash2_workspace_bytes(int op, int64_t n_rows, int32_t hidden, int32_t vocab,
                               int32_t rank, int32_t top_k);

/* Human-readable name of a status code (static string, host only). */
const char *dflash2_status_str(int status);

/*
 * Synchronises `stream`, then reads the status word of the last call that
 * used `workspace`: DFLASH2_OK or DFLASH2_ERR_DEVICE_ID_RANGE
 * (DFLASH2_ERR_LAUNCH if the read itself fails).
 */
dflash2_status dflash2_read_device_status(const void *workspace, void *stream);

/*
 * Debug knob for determinism tests (host only, process-wide).  Fixes how many
 * vocabulary slabs (partial top-K lists per row) the LM-head kernels of
 * dflash2_unary_topk(_ex) and dflash2_decode_head split the vocabulary into,
 * clamped to each kernel's own limit; 0 restores the automatic choice.  Every
 * logit is formed the same way whatever the split and keys merge in one total
 * order, so the ids and values returned must not change with it (the
 * log-sum-exp outputs may differ in the last bits).  It changes
 * dflash2_workspace_bytes for those operations: size workspaces after setting
 * it.  Not synchronised with calls running on other host threads.
 * n_slabs in [0, 4096] (DFLASH2_ERR_SHAPE otherwise).
 */
dflash2_status dflash2_debug_force_slabs(int32_t n_slabs);

/* Library version, e.g. "dflash2-gfx950 0.1.0" (static string). */
const char *dflash2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH2_H_ */
