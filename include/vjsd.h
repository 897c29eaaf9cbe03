/*
 * vjsd.h -- C ABI of libvjsd: per-token softmax statistics, generalized
 * Jensen-Shannon divergence, KL, entropy and log-probabilities over a vocabulary
 * split into logical shards, for AMD Instinct MI355X (gfx950).
 *
 * Page keys used in the citations:
 *   [JSD-PR] DeepSpeed PR #8958, "[VocabTP] Add vocabulary-parallel generalized JSD
 *            with Triton kernels".
 *   [OPS-PR] DeepSpeed PR #8791, "Add vocabulary-parallel logprobs, entropy and KL
 *            ops", and its review thread.
 *
 * ---------------------------------------------------------------------------------
 * Conventions shared by every entry point
 *
 * Rows.  N tokens ("rows") are processed; each row holds V vocabulary logits split
 * into S >= 1 consecutive shards.  Shard k covers the global vocabulary ids
 * [vocab_start_k, vocab_start_k + width_k); shards are ordered and contiguous
 * (vocab_start_{k+1} = vocab_start_k + width_k) and a width may be 0 (an empty
 * shard joins the merge as (max, sum-exp) = (-inf, 0), [OPS-PR, review: empty
 * shards]).  One GPU stands in for the tensor-parallel ranks of the pages: a
 * shard's statistics are reduced locally and merged on the device where the pages
 * all-reduce them [OPS-PR, How].
 *
 * Views.  A shard's student / teacher logits (and its gradients) are views with
 * unit column stride.  Row r of a view is at element
 *     rows_per_batch == 0:  r * row_stride
 *     rows_per_batch  > 0:  (r / rows_per_batch) * batch_stride
 *                           + (r % rows_per_batch) * row_stride
 * relative to p, so the causal-shift slices [B, T-1, V] of a [B, T, V] tensor are
 * taken without a copy [JSD-PR, Changes].  Strides count elements.  Student,
 * teacher and both gradients share the same dtype and shard layout [JSD-PR, Scope
 * and limitations].  Pointers are device pointers and must be aligned to their
 * element size; 16-byte alignment of every row (same offset in all views of a
 * shard) selects the vector path, any other alignment runs a slower scalar path.
 *
 * Dtypes.  Inputs are fp32, fp16 or bf16 (vjsd_dtype) and are widened to fp32 in
 * registers; all arithmetic is fp32 with fp64 per-row bookkeeping.  Per-token
 * outputs are fp32 [JSD-PR, Changes]; gradients are written in the input dtype,
 * rounded to nearest even.
 *
 * Statistics.  `stats` is double[N][4] = (m_s, lnZ_s, m_t, lnZ_t): the row max of
 * the student / teacher logits and ln sum_j exp(x_j - m), kept apart so that a large
 * common offset costs no precision [OPS-PR, How].  One-input ops use (m_s, lnZ_s)
 * and leave the teacher half unspecified.  An undefined row (all -inf) has
 * m = -inf, lnZ = -inf.
 *
 * Workspace.  `part` is caller-owned device memory of vjsd_workspace_bytes(N, S)
 * bytes (16-byte aligned) holding per-row constants and per-shard partial results
 * between the launches of one call, and between vjsd_stats and vjsd_merge.  Its
 * contents are otherwise unspecified; calls that share one workspace must not
 * overlap in time.
 *
 * Ownership and streams.  The caller owns every buffer.  The library allocates no
 * memory, keeps no state between calls (vjsd_bwd_noalloc's device array aside) and is
 * reentrant; every call only enqueues
 * kernels on `stream` (a hipStream_t; NULL is the null stream) and returns without
 * synchronising.  Buffers must stay valid until the enqueued work completes.
 * Outputs must not alias inputs.
 *
 * Errors.  Arguments are validated on the host before anything is enqueued; an
 * invalid call returns a negative VJSD_ERR_* code and enqueues nothing.  N == 0 is
 * valid and enqueues nothing [JSD-PR, Validation: empty token batches].  A launch
 * failure returns VJSD_ERR_HIP.  A row that is -inf everywhere is not an error: its
 * per-token value is NaN and every gradient in it is exactly 0, whatever the
 * upstream gradient [OPS-PR, review: NaN gradients of fully masked rows].
 * ---------------------------------------------------------------------------------
 */
#ifndef VJSD_H
#define VJSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Entry points are the library's only exported symbols. */
#if defined(__GNUC__) || defined(__clang__)
#define VJSD_API __attribute__((visibility("default")))
#else
#define VJSD_API
#endif

typedef enum { VJSD_F32 = 0, VJSD_F16 = 1, VJSD_BF16 = 2 } vjsd_dtype;

enum {
    VJSD_OK = 0,
    VJSD_ERR_ARG = -1,         /* null pointer, negative size, bad stride, misaligned pointer */
    VJSD_ERR_DTYPE = -2,       /* dtype not one of vjsd_dtype */
    VJSD_ERR_BETA = -3,        /* beta NaN or outside [0, 1] */
    VJSD_ERR_LAYOUT = -4,      /* shards not ordered/contiguous, or vocabulary size mismatch */
    VJSD_ERR_EMPTY_SHARD = -5, /* a shard of width 0 given to the log-probability op */
    VJSD_ERR_HIP = -6,         /* the HIP runtime refused a launch */
    VJSD_ERR_SCRATCH = -7      /* more rows than the no-allocation scratch holds */
};

/* Read-only view of one shard of one input (see "Views"). */
typedef struct {
    const void *p;
    int64_t row_stride;
    int64_t rows_per_batch;
    int64_t batch_stride;
} vjsd_view;

/* Writable view; p == NULL means "this output is not wanted". */
typedef struct {
    void *p;
    int64_t row_stride;
    int64_t rows_per_batch;
    int64_t batch_stride;
} vjsd_mview;

/* One logical vocabulary shard. */
typedef struct {
    int64_t vocab_start; /* first global vocabulary id of the shard */
    int64_t width;       /* number of vocabulary columns, >= 0 */
    vjsd_view s;         /* student logits; the one input of entropy / logprobs */
    vjsd_view t;         /* teacher logits; ignored by one-input ops */
    vjsd_mview gs;       /* gradient w.r.t. s, written by the backward entry points */
    vjsd_mview gt;       /* gradient w.r.t. t, written by the backward entry points */
} vjsd_shard;

/* Human-readable text of a VJSD_* code (static storage). */
VJSD_API const char *vjsd_strerror(int code);

/* Bytes of the `part` workspace for N rows and S shards. */
VJSD_API size_t vjsd_workspace_bytes(int64_t N, int S);

/*
 * Per-shard paired softmax statistics [JSD-PR, Changes: fused paired softmax
 * statistics; OPS-PR, How].  For every shard k and row r, and for the inputs
 * selected by `which` (1 = student, 2 = teacher, 3 = both), computes the shard's
 * max and sum of exponentials into `part`.  This is the first input pass.
 */
VJSD_API int vjsd_stats(const vjsd_shard *shards, int S, int64_t N, int dtype, int which,
               float *part, void *stream);

/*
 * Cross-shard merge [OPS-PR, How: MAX then SUM of the [N] statistics]: the global
 * max is the max of the shard maxima and each shard's sum-exp is rescaled to it;
 * shards with max -inf add nothing [OPS-PR, review: empty shards].  Reads `part` as
 * left by vjsd_stats with the same S, N, which; writes stats[N][4] (only the halves
 * selected by `which`).
 */
VJSD_API int vjsd_merge(const float *part, int S, int64_t N, int which, double *stats, void *stream);

/*
 * Generalized JSD forward [JSD-PR, Motivation and Changes]: with
 * M = beta p_t + (1 - beta) p_s, writes per token
 *     kl[r]   = (KL(p_t || M), KL(p_s || M))   (float[N][2], saved for backward)
 *     loss[r] = beta KL(p_t || M) + (1 - beta) KL(p_s || M)   for 0 < beta < 1,
 *               KL(p_t || p_s)  (forward KL) for beta == 0,
 *               KL(p_s || p_t)  (reverse KL) for beta == 1,
 * the endpoints being exact branches, not limits [JSD-PR, Changes].  At beta == 0
 * kl[r][1] is 0 and at beta == 1 kl[r][0] is 0.  KL is +inf when the target puts
 * mass on a token the other side masked, decided on the logits [OPS-PR, Tests].
 * `stats` must hold both halves (vjsd_stats/vjsd_merge with which = 3).  This is the
 * second input pass; shard partials go through `part` and are summed in shard order.
 */
VJSD_API int vjsd_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, const double *stats,
             double beta, float *part, float *kl, float *loss, void *stream);

/*
 * The whole JSD forward in one call: vjsd_stats (both inputs), vjsd_merge and
 * vjsd_fwd, with the same outputs (stats, kl, loss), the same semantics and the
 * same workspace `part` [JSD-PR, Changes].  How it runs:
 *   beta = 0 or 1   the forward / reverse KL, in one input pass (as vkl_fwd)
 *   one shard       one launch, a workgroup per row: statistics, then divergence.
 *                   Rows 16-byte aligned, a multiple of 16 bytes and at most
 *                   80 KiB wide (40960 bf16 / fp16 or 20480 fp32 columns) are held
 *                   in registers and read from HBM once; wider rows are swept twice
 *   2 to 8 shards   one launch, a workgroup per row: each shard's slice is swept for
 *                   its (max, sum-exp) pairs, the pairs are merged in shard order as
 *                   vjsd_merge merges them, then the slices are swept for the
 *                   divergence; `part` is not written
 *   more shards     the three separate launches
 * Results agree with the separate calls within rounding (the reduction order
 * differs) and are deterministic for a given layout and device.  Errors as vjsd_fwd.
 */
VJSD_API int vjsd_forward(const vjsd_shard *shards, int S, int64_t N, int dtype, double beta,
                          float *part, double *stats, float *kl, float *loss, void *stream);

/*
 * The distillation loss around the per-token JSD: what the pages' callers do before
 * and after the per-token op, fused into its passes.  [JSD-PR, Changes] leaves
 * temperature, optional T^2 scaling, masking and normalisation to the caller;
 * DeepSpeedExamples PR #1019 ("vocab-parallel KL route for OPSD") divides both
 * logits by a temperature other than 1 in fp32 first (a full-size fp32 copy of each
 * input), then keeps the T^2 scaling and a token mean over the response tokens.
 *
 *   temperature  T > 0, finite.  Both inputs are divided by T in registers: the
 *                kernels' exponent scale log2(e) becomes fl32(log2(e) / T), so
 *                nothing is copied.  T = 1 reproduces vjsd_forward / vjsd_bwd.
 *   scale_t2     nonzero: per-token losses (and their gradients) carry T^2.
 *   mask         NULL, or a device uint8_t[N]; a zero entry drops the token: its
 *                logits are never read, its per-token loss is 0, it is left out of
 *                the reduction and its gradients are exactly 0.
 *   reduction    VJSD_REDUCE_NONE: per-token losses only; VJSD_REDUCE_SUM: out[0] =
 *                their sum over kept tokens; VJSD_REDUCE_MEAN: that sum divided by
 *                the number of kept tokens, 0 when no token is kept (the count is
 *                clamped at 1).  The sum runs in fp64 in a fixed order; an undefined
 *                kept token (NaN) makes the result NaN.
 * A NULL opts pointer means T = 1, no T^2, no mask, no reduction.
 */
enum { VJSD_REDUCE_NONE = 0, VJSD_REDUCE_SUM = 1, VJSD_REDUCE_MEAN = 2 };
typedef struct {
    double temperature;
    int scale_t2;
    const uint8_t *mask;
    int reduction;
} vjsd_loss_opts;

/*
 * Forward of the distillation loss (routed like vjsd_forward).  Writes stats[N][4]
 * (raw row maxima, lnZ of the tempered logits), kl[N][2] (the KL pair of the
 * tempered distributions, not scaled by T^2), rows[N] (per-token losses, times T^2
 * when scale_t2, 0 for dropped tokens) and, for a reduction, out[0] (out may be NULL
 * for VJSD_REDUCE_NONE).  With N == 0 only out[0] = 0 is written.  Errors as
 * vjsd_fwd, plus VJSD_ERR_ARG for a bad temperature or reduction, or a NULL out
 * with a reduction.
 */
VJSD_API int vjsd_loss_forward(const vjsd_shard *shards, int S, int64_t N, int dtype, double beta,
                               const vjsd_loss_opts *opts, float *part, double *stats, float *kl,
                               float *rows, float *out, void *stream);

/*
 * Backward of the distillation loss: gradients w.r.t. the raw logits, into each
 * shard's gs / gt views (NULL gs.p / gt.p skip one, as in vjsd_bwd).  grad is the
 * upstream gradient: float[N] per token for VJSD_REDUCE_NONE, float[1] for a
 * reduction.  Row r's upstream scale is g_r * (T^2 if scale_t2) / T (the chain rule
 * through x / T), g_r / max(kept, 1) for a mean, and 0 for a dropped row.  Takes
 * the forward's stats and kl and the same opts, beta and mask.  Errors as vjsd_bwd.
 */
VJSD_API int vjsd_loss_backward(const vjsd_shard *shards, int S, int64_t N, int dtype, double beta,
                                const vjsd_loss_opts *opts, const double *stats, const float *kl,
                                const float *grad, float *part, void *stream);

/*
 * Generalized JSD backward, closed form and local [JSD-PR, Changes: recompute
 * probabilities in registers; OPS-PR, How: no communication].  With g = grad_loss[r]:
 *   interior: d/ds = g (1-beta) p_s (lp_s - lM - KS),  d/dt = g beta p_t (lp_t - lM - KT)
 *   beta = 0: d/ds = g (p_s - p_t),                   d/dt = g p_t (lp_t - lp_s - KT)
 *   beta = 1: d/ds = g p_s (lp_s - lp_t - KS),         d/dt = g (p_t - p_s)
 * written into each shard's gs / gt views; a NULL gs.p (gt.p) skips that gradient
 * (teacher or student detached) [JSD-PR, Changes].  A -inf logit's own term is 0.
 * In a row whose KL is +inf the target-side gradient is not finite.  Reads the
 * inputs, stats and kl of the forward; `part` (workspace) receives per-row constants.
 * This is the third input pass.
 */
VJSD_API int vjsd_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, const double *stats,
             const float *kl, double beta, const float *grad_loss, float *part, void *stream);

/*
 * vjsd_bwd without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The per-row constants that vjsd_bwd writes into `part` go instead to an
 * array the library owns in device memory, VJSD_NOALLOC_MAX_ROWS rows of 64 bytes
 * (4 MiB), which each device the library runs on holds until the process ends.  Its
 * address on a device is looked up once, on the first call there.  The call itself
 * allocates nothing; every other argument, the results and the errors are those of
 * vjsd_bwd, which shares its kernels.  Every call on one device uses that device's one
 * array, and a call fully rewrites the rows it reads before reading them: calls that
 * overlap on one device (concurrent streams, or threads) race on the array, so the
 * caller must serialise them.  `stream` must belong to the current device (NULL: the
 * current device's null stream).  Extra errors: VJSD_ERR_SCRATCH when N exceeds
 * VJSD_NOALLOC_MAX_ROWS; VJSD_ERR_ARG when the stream belongs to another device;
 * VJSD_ERR_HIP when the array's address cannot be obtained.
 */
#define VJSD_NOALLOC_MAX_ROWS 65536
VJSD_API int vjsd_bwd_noalloc(const vjsd_shard *shards, int S, int64_t N, int dtype,
                              const double *stats, const float *kl, double beta,
                              const float *grad_loss, void *stream);

/*
 * Forward and backward of the distillation loss in one call, for callers that know
 * the upstream gradient before the forward (a per-token weight, or the reduction's
 * scale of a loss that is itself the objective): the outputs of vjsd_loss_forward
 * (stats, kl, rows, out) and the gradients of vjsd_loss_backward for `grad`, into
 * each shard's gs / gt views, bit for bit [JSD-PR, Changes: the backward reuses the
 * forward's global statistics and recomputes probabilities from the logits].  Same
 * arguments as those two calls, same meaning and ownership; `part` as there.  How it
 * runs:
 *   one shard, 0 < beta < 1, no mask   one launch, a workgroup per row: the forward of
 *                   vjsd_forward's single-shard route, then that row's gradients in
 *                   the same workgroup.  A row held in registers is read from HBM
 *                   once for both passes (its gradient views must start on 16-byte
 *                   boundaries like the inputs', else the two calls run); a wider row
 *                   reuses the sweep steps it holds on chip and reads the rest a
 *                   third time.
 *   otherwise       vjsd_loss_forward, then vjsd_loss_backward (with a mask too: when
 *                   few tokens are kept, the kept rows' whole work in one workgroup
 *                   each would end the launch on a tail).
 * Errors as vjsd_loss_forward and vjsd_loss_backward; on an error nothing is
 * launched, except a VJSD_ERR_HIP from a launch.
 */
VJSD_API int vjsd_loss_forward_backward(const vjsd_shard *shards, int S, int64_t N, int dtype,
                                        double beta, const vjsd_loss_opts *opts,
                                        const float *grad, float *part, double *stats,
                                        float *kl, float *rows, float *out, void *stream);

/*
 * vjsd_forward, then vjsd_bwd with the upstream gradient grad_loss[N], in one call:
 * vjsd_loss_forward_backward with NULL opts (T = 1, no mask, per-token losses into
 * `loss`).  Outputs equal those of the two calls bit for bit [JSD-PR, Changes].
 */
VJSD_API int vjsd_forward_backward(const vjsd_shard *shards, int S, int64_t N, int dtype,
                                   double beta, const float *grad_loss, float *part,
                                   double *stats, float *kl, float *loss, void *stream);

/*
 * KL divergence [OPS-PR, What]: KL(p_t || p_s), or KL(p_s || p_t) when reverse != 0,
 * with the forward computed in a single input pass by online accumulation (as the
 * single-pass KL forward of [JSD-PR, Scope and limitations]).  Writes stats[N][4]
 * (both halves), kl[N][2] in the layout of vjsd_fwd at beta = 0 (reverse = 0) or
 * beta = 1 (reverse != 0), and loss[N].
 */
VJSD_API int vkl_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int reverse, float *part,
            double *stats, float *kl, float *loss, void *stream);

/*
 * KL backward: vjsd_bwd at beta = 0 (reverse = 0) or beta = 1 (reverse != 0); closed
 * form from the saved [N] statistics and the inputs, probabilities recomputed, and a
 * row with no distribution gets exactly zero gradients [OPS-PR, How].
 */
VJSD_API int vkl_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int reverse,
            const double *stats, const float *kl, const float *grad_loss, float *part,
            void *stream);

/*
 * Entropy [OPS-PR, What]: ent[r] = -sum_j p_j lp_j over the student view, single
 * input pass.  Writes stats (student half) and ent[N].
 */
VJSD_API int ventropy_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, float *part,
                 double *stats, float *ent, void *stream);

/*
 * Entropy backward: d/dx_j = -g p_j (lp_j + H), into each shard's gs view; closed form
 * from the saved statistics and ent, a -inf token and an undefined row get exactly
 * zero [OPS-PR, How].
 */
VJSD_API int ventropy_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, const double *stats,
                 const float *ent, const float *grad, float *part, void *stream);

/*
 * Log-probabilities of K ids per row [OPS-PR, What]: out[r][k] = lp(ids[r][k]),
 * ids being global vocabulary ids in [0, vocab_global); out is exactly 0 where
 * ids[r][k] == ignore_index.  The shards must cover [0, vocab_global) and none may
 * be empty (VJSD_ERR_EMPTY_SHARD) [OPS-PR, review: empty shards].  An id outside the
 * range that is not ignore_index cannot be seen on the host: the kernels set
 * *dev_err (device int32, caller-zeroed) to 1, and the caller must check it after
 * synchronising and treat the call as failed [OPS-PR, review: the index range check
 * runs every call].  Writes stats (student half) and out[N][K].
 */
VJSD_API int vlogprobs_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                  const int64_t *ids, int K, int64_t ignore_index, float *part, double *stats,
                  float *out, int32_t *dev_err, void *stream);

/*
 * Log-probabilities backward [OPS-PR, How: closed form, local, from the saved
 * statistics]: d/dx_j = sum_{k valid} g_k [j == ids_k] - (sum_{k valid} g_k) p_j, with
 * g = grad[N][K]; repeated ids accumulate.  Writes each shard's gs view.  Out-of-range
 * ids are skipped (the forward reported them).
 */
VJSD_API int vlogprobs_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                  const double *stats, const int64_t *ids, int K, int64_t ignore_index,
                  const float *grad, float *part, void *stream);

/*
 * Cross-entropy of integer labels over the sharded vocabulary, the loss a
 * vocabulary-parallel causal-LM head installs (DeepSpeed PR #8309, "[AutoTP]
 * vocab-parallel LM head": vocab_parallel_cross_entropy):
 *     rows[r] = -lp_s(r, labels[r]),  exactly 0 where labels[r] == ignore_index
 * with lp_s the log-softmax of the shards' `s` views (labels: device int64[N],
 * global ids).  A row whose label is ignore_index is never read.  reduction as in
 * vjsd_loss_opts: out[0] = sum over labelled rows, or their mean (0 when none).
 * An undefined labelled row is NaN; a label outside [0, vocab_global) that is not
 * ignore_index sets *dev_err = 1 and makes its row NaN.  Writes stats (s half) and
 * rows[N].  Shard rules and errors as vlogprobs_fwd, plus VJSD_ERR_ARG for a bad
 * reduction or a NULL out with a reduction.  With N == 0 only out[0] = 0 is written.
 */
VJSD_API int vce_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                     const int64_t *labels, int64_t ignore_index, int reduction, float *part,
                     double *stats, float *rows, float *out, int32_t *dev_err, void *stream);

/*
 * Its backward into each shard's gs view: d/dx_j = g_r (p_j - [j == label_r]) for
 * labelled rows (g_r = grad[r] for VJSD_REDUCE_NONE, grad[0] for a sum, grad[0] /
 * max(labelled, 1) for a mean), exactly 0 for ignored and undefined rows, which are
 * not read.  Errors as vlogprobs_bwd.
 */
VJSD_API int vce_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                     const double *stats, const int64_t *labels, int64_t ignore_index, int reduction,
                     const float *grad, float *part, void *stream);

/*
 * Teacher top-k forward KL per token [OPS-PR, What: the teacher top-k forward KL
 * pattern built on the log-probabilities of the teacher's top-k ids]:
 *     kl[r] = sum_k exp(tlogp[r][k]) * (tlogp[r][k] - lp_s(r, ids[r][k]))
 * with lp_s the student's log-softmax over the whole (sharded) vocabulary.  ids
 * (device int64[N][K], global vocabulary ids) and tlogp (device float[N][K], the
 * teacher's log-probabilities at those ids) are data.  A slot whose id equals
 * ignore_index, or whose tlogp is -inf, is padding and adds nothing.  A valid slot
 * on a student logit of -inf makes kl +inf (decided on the logits); an undefined
 * student row gives NaN.  An id outside [0, vocab_global) that is not ignore_index
 * sets *dev_err = 1 and makes its row NaN (the flag is never cleared by the library).
 * The sum runs in fp64 per row (shards in groups of 16; more groups add in fp32).
 * Writes stats (student half), kl[N].  Shard rules and errors as vlogprobs_fwd.
 */
VJSD_API int vtopk_kl_fwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                          const int64_t *ids, const float *tlogp, int K, int64_t ignore_index,
                          float *part, double *stats, float *kl, int32_t *dev_err, void *stream);

/*
 * Its backward, to the student logits only: d kl[r] / d lp_s(id_k) = -exp(tlogp[r][k])
 * on valid slots, through the log-probability backward, so
 *     d/dx_j = sum_k w_k [j == id_k] - (sum_k w_k) p_j,   w_k = -grad[r] exp(tlogp[r][k]).
 * grad is float[N]; undefined rows get exactly 0.  Errors as vlogprobs_bwd.
 */
VJSD_API int vtopk_kl_bwd(const vjsd_shard *shards, int S, int64_t N, int dtype, int64_t vocab_global,
                          const double *stats, const int64_t *ids, const float *tlogp, int K,
                          int64_t ignore_index, const float *grad, float *part, void *stream);

/*
 * Memory-bandwidth probe: the streaming ceiling the passes above are judged against
 * (their inputs and gradients move through HBM once per pass with 16-byte
 * streaming accesses, so a plain streaming read or copy of the same size bounds
 * them).  op 0 reads `bytes` from src; op 1 copies `bytes` from src to dst; both use
 * 16-byte nontemporal loads (and stores), consecutive lanes on consecutive 16-byte
 * words.  bytes must be a positive multiple of 16 and src / dst 16-byte aligned.
 * op 0 writes at most 16 bytes at dst (only if the data hashes to a fixed value; the
 * write keeps the reads live); op 1 writes `bytes` at dst, which must not overlap
 * src.  VJSD_ERR_ARG for a bad op, size or pointer; VJSD_ERR_HIP for a failed
 * launch.
 */
VJSD_API int vjsd_membw_probe(const void *src, void *dst, size_t bytes, int op, void *stream);

/* ---- fused linear + JSD ------------------------------------------------------------- */

/*
 * Matrix operand of vlin_gemm: element (row, k) at p[row*ld + k] when kmajor, else at
 * p[k*ld + row].  dtype VJSD_BF16, or VJSD_F32 for the first operand only (each
 * value rounded to bf16, nearest even, before its product).  p must be 16-byte
 * aligned and ld a multiple of 8 elements (4 for VJSD_F32), at least the extent of
 * the contiguous index, and the operand readable over whole rows of ld elements
 * (edge tiles read full 16-byte chunks up to a row's ld and discard what lies past
 * the contiguous index).
 */
typedef struct {
    const void *p;
    int64_t ld;
    int dtype;
    int kmajor;
} vlin_operand;

enum { VLIN_OUT_F32 = 0, VLIN_OUT_F32_ACC = 1, VLIN_OUT_BF16 = 2 };

/*
 * The matrix-core product the fused-linear loss is built from ([JSD-PR, Motivation]:
 * the divergence evaluated from tiled LM-head projections; [JSD-PR, Scope and
 * limitations] / [OPS-PR, Limitations]: a fused-linear variant is future work):
 *     C[i][j] = sum_k A(i, k) * B(j, k),   i < M, j < N, k < K
 * bf16 products accumulated in fp32 (v_mfma_f32_32x32x16_bf16).  out selects fp32
 * C (VLIN_OUT_F32), fp32 C += product (VLIN_OUT_F32_ACC) or bf16 C rounded to
 * nearest even (VLIN_OUT_BF16); C row-major with row stride ldc >= N, element
 * aligned, not overlapping A or B.  K == 0 gives C = 0 (or leaves C unchanged when
 * accumulating).  VJSD_ERR_ARG for negative sizes, a NULL, misaligned or too-short
 * operand, or a bad out; VJSD_ERR_DTYPE for another operand dtype.
 */
VJSD_API int vlin_gemm(int64_t M, int64_t N, int64_t K, vlin_operand a, vlin_operand b, void *c,
                       int64_t ldc, int out, void *stream);

/*
 * One side of the fused-linear loss: hidden states h [N][dim] (row stride ldh) and
 * LM-head weight w [V][dim] (row stride ldw), both bf16, 16-byte aligned, strides
 * multiples of 8 elements.  The side's logits are h w^T [N][V].
 */
typedef struct {
    const void *h;
    int64_t ldh;
    const void *w;
    int64_t ldw;
    int64_t dim;
} vlin_head;

/*
 * Fused-linear distillation loss: the loss of vjsd_loss_forward on the logits
 * h_s w_s^T (student) and h_t w_t^T (teacher), computed `chunk` tokens at a time, so
 * that only chunk-row blocks of logits ever exist (in the workspace, fp32); with more
 * than one chunk, chunk is rounded down to a multiple of 8 (at least 8).  opts as
 * vjsd_loss_opts (temperature, T^2, token mask, reduction).  out is float[N] for
 * VJSD_REDUCE_NONE, else out[0] is the sum or the mean over the kept tokens.
 * grad_h (bf16 [N][dim_s], row stride ldgh) and grad_w (bf16 [V][dim_s], row stride
 * ldgw), each optional (NULL), receive d out[0] / d h_s and d out[0] / d w_s; they
 * need a reduction (VJSD_ERR_ARG otherwise).  The teacher is a constant.  The logit
 * gradient is rounded to bf16 (the operand precision of the products); each chunk's
 * goes into its grad_h rows at once, and, transposed, it is kept for `group` tokens
 * at a time (rounded up to whole chunks; 0: as many as fit 4 GiB) for the head
 * gradient's product; with more than one group the head gradient is summed across
 * groups in fp32.  Masked tokens get exactly zero rows of grad_h.  workspace: device
 * memory of vljsd_workspace_bytes(N, V, dim_s, chunk, group) bytes, 256-byte aligned
 * (for a fixed group it does not grow with N).  VJSD_ERR_ARG for a bad size, chunk,
 * group, pointer, alignment or stride; VJSD_ERR_BETA as vjsd_fwd.
 */
VJSD_API size_t vljsd_workspace_bytes(int64_t N, int64_t V, int64_t dim_s, int64_t chunk,
                                      int64_t group);
VJSD_API int vljsd(const vlin_head *student, const vlin_head *teacher, int64_t N, int64_t V,
                   double beta, const vjsd_loss_opts *opts, int64_t chunk, int64_t group,
                   void *workspace, float *out, void *grad_h, int64_t ldgh, void *grad_w,
                   int64_t ldgw, void *stream);

/*
 * Scales n values in place by a device scalar: p[i] *= g[0] (the upstream gradient
 * of a reduced loss applied to gradients computed for a unit upstream gradient: the
 * fused-linear loss, or vjsd_loss_forward_backward with a unit grad).  dtype VJSD_F32,
 * VJSD_F16 or VJSD_BF16 (nearest even); p 16-byte aligned.  When g[0] is exactly 1
 * the launched kernel returns at once and p is neither read nor written (x * 1 == x
 * in every format), so applying a unit upstream gradient costs one short launch.
 */
VJSD_API int vlin_scale(void *p, int64_t n, int dtype, const float *g, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VJSD_H */
