/*
 * packed_ctc.h — CTC loss and gradient over sequence-packed log probabilities on MI355X (gfx950).
 *
 * The operation is the one defined on the NVIDIA-NeMo/Speech pull request page "feat(asr): native
 * CTC loss kernel over sequence-packed log probabilities" ([PR] below): the public function
 * `packed_ctc_loss` of its Triton file, its two kernels `_alpha_kernel` / `_beta_grad_kernel`, its
 * autograd backward, and the reductions of `forward_packed` in its `ctc.py` diff.
 *
 * Layout (the token-flat packing of [PR], module description and `packed_ctc_loss` arguments):
 *   log_probs  (T_total, D) row-major, float32 / bfloat16 / float16, the blank among the D classes.
 *              Utterance b owns rows [cu_seqlens[b], cu_seqlens[b] + lengths[b]).  Rows owned by no
 *              utterance (gaps, trailing rows) get a zero gradient.
 *   cu_seqlens (B + 1,) int32 or int64 first row of each utterance (entry B is not read).
 *   lengths    (B,)     int32 or int64 frames per utterance.
 *   targets    (B, target_width) int32 or int64 row-major, label ids in [0, D); only the first
 *              target_lengths[b] entries of row b are read (the rest may hold anything).
 *              A target equal to the blank id is an ordinary label ([PR] `_alpha_kernel`).
 *   target_lengths (B,) int32 or int64.
 *
 * All pointers except the stream are DEVICE pointers owned by the caller.  Calls are asynchronous
 * on `stream` (a hipStream_t passed as void*; NULL = the default stream) and allocate nothing: all
 * scratch lives in the caller's `workspace`.  No call keeps a pointer after it returns.
 * Every function returns PCTC_OK (0) or one of the error codes below; on error nothing has been
 * launched and packed_ctc_last_error() holds a message (thread-local).
 */
#ifndef PACKED_CTC_H
#define PACKED_CTC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* log_probs / grad dtypes ([PR] `PACKED_CTC_LOSS_DTYPES`: float32, bfloat16, float16, computed in
 * float32; the page sends float64 to the padded path, which keeps float64 precision).  F64 is this
 * library's own addition: float64 log probs are computed in float64 throughout (recursions,
 * posteriors, gradient), on the packed layout; it is the precision path, not a fast one. */
#define PCTC_DTYPE_F32 0
#define PCTC_DTYPE_BF16 1
#define PCTC_DTYPE_F16 2
#define PCTC_DTYPE_F64 3

/* index_flags: a set bit makes that array int64, a clear bit int32 */
#define PCTC_I64_CU_SEQLENS 1
#define PCTC_I64_LENGTHS 2
#define PCTC_I64_TARGETS 4
#define PCTC_I64_TARGET_LENGTHS 8

/* reductions of [PR] `forward_packed`: none, sum, and the mean of each loss over its clamped
 * target length max(U_b, 1), then the batch mean */
#define PCTC_REDUCTION_NONE 0
#define PCTC_REDUCTION_SUM 1
#define PCTC_REDUCTION_MEAN 2

/* error codes, one per failure class of [PR] `packed_ctc_loss` argument checks */
#define PCTC_OK 0
#define PCTC_ERR_SHAPE 1              /* a size is negative or inconsistent (the page's ValueError on shapes) */
#define PCTC_ERR_DTYPE 2              /* log_probs dtype not F32/BF16/F16/F64 (the page's TypeError) */
#define PCTC_ERR_BLANK 3              /* blank outside [0, D) */
#define PCTC_ERR_NEG_TARGET_LENGTH 4  /* a negative target length (checked on the host read) */
#define PCTC_ERR_TARGET_LENGTH_WIDTH 5/* a target length beyond target_width (checked on the host read) */
#define PCTC_ERR_WORKSPACE 6          /* workspace missing or smaller than packed_ctc_workspace_size() */
#define PCTC_ERR_HIP 7                /* a HIP runtime or launch error */
#define PCTC_ERR_ARG 8                /* a required pointer is NULL, or an unknown flag / reduction */
#define PCTC_ERR_LIMIT 9              /* beyond what the library supports (see packed_ctc_limits) */

/* Pipelines of a packed_ctc_loss call that forms the gradient (packed_ctc_set_pipeline). */
#define PCTC_PIPELINE_GROUPED 0   /* length-sorted groups on concurrent streams, rows after each group's recursions */
#define PCTC_PIPELINE_STREAMED 1  /* one persistent launch: rows formed as the recursions pass them (default) */

/*
 * Bytes of device workspace a call needs for T_total frames, D classes, B utterances, target lengths
 * up to max_target_length and alpha checkpoint interval checkpoint_interval (see packed_ctc_loss;
 * 1 keeps every alpha row).  Returns 0 for negative sizes or an interval that is not a power of two
 * in [1, 32].
 */
size_t packed_ctc_workspace_size(int64_t T_total, int64_t D, int64_t B, int64_t max_target_length,
                                 int checkpoint_interval);

/*
 * Supported maxima of the library: the longest target (labels) and the class count D.
 * Either pointer may be NULL.
 */
void packed_ctc_limits(int64_t* max_target_length, int64_t* max_classes);

/*
 * Host-synchronous read of target_lengths ([PR] `packed_ctc_loss`: the host check of the padded
 * kernel, no negative length and none beyond the targets width, and the longest target sizes the
 * states).  Copies the B lengths to the host on `stream`, waits, and stores their maximum (0 when
 * B = 0) in *max_out.  Errors: PCTC_ERR_NEG_TARGET_LENGTH, PCTC_ERR_TARGET_LENGTH_WIDTH.
 * Must not be called while `stream` is being captured into a graph.
 */
int packed_ctc_max_target_length(const void* target_lengths, int index_flags, int64_t B, int64_t target_width,
                                 void* stream, int64_t* max_out);

/*
 * CTC loss per utterance and its gradient ([PR] `packed_ctc_loss`, `_PackedCTCLoss`, the kernels).
 *
 * Computes, per utterance b with T = lengths[b] frames and U = target_lengths[b] labels over the
 * extended label sequence blank, l1, blank, ..., lU, blank (S = 2U + 1 states):
 *   nll_b = -log(sum over alignments) by the log-space alpha recursion; T = 0 gives 0 when U = 0
 *           and +inf otherwise; no alignment gives +inf;
 *   losses_out[b] = nll_b, or 0 when zero_infinity and nll_b = +inf   (B values of the loss type:
 *                   float32 for F32 / BF16 / F16 inputs, float64 for F64 inputs);
 *   reduced_out   = sum_b losses_out[b] (SUM) or mean_b losses_out[b] / max(U_b, 1) (MEAN), one
 *                   value of the loss type; not written for NONE; may be NULL;
 *   grad_out      = (T_total, D) in the dtype of log_probs, round-to-nearest-even:
 *                   w_b * (exp(log_probs) - posterior summed per class) on the rows of utterance b,
 *                   0 on rows owned by no utterance.  This is the gradient with respect to the
 *                   logits of a log_softmax ([PR] module description).  w_b is
 *                   (grad_scale ? grad_scale[b] : 1; B values of the loss type, like
 *                   losses_out) times 1/(B * max(U_b, 1)) for MEAN, and 0
 *                   when zero_infinity and nll_b = +inf.  An infeasible utterance with w_b != 0
 *                   gets NaN in every column of its rows; w_b = 0 gives zero rows whatever the
 *                   log probs hold.  May be NULL (loss only).
 *   NaN inputs (the page does not treat them): a NaN at the blank's or one of utterance b's label
 *   columns in any of its rows makes nll_b NaN (zero_infinity leaves a NaN loss alone) and, with
 *   w_b != 0, every column of its rows NaN; a NaN at any other column shows only in that entry of
 *   the gradient row.
 *   An utterance with fewer frames than its labels need (T < U + the number of equal neighbouring
 *   labels) has no alignment whatever the log probs hold; its recursions are not run.
 *
 * max_target_length >= 0: a caller-promised bound on every target length (no host read; the call
 *   is then graph-capturable).  Lengths beyond it, negative lengths, label ids outside [0, D), or
 *   utterance rows outside [0, T_total) are precondition violations: the kernels clamp them so
 *   that every memory access stays in bounds, and the results for that utterance are unspecified.
 * max_target_length < 0: the library reads target_lengths on the host exactly as
 *   packed_ctc_max_target_length does, except while `stream` is being captured, where
 *   target_width stands in ([PR] `packed_ctc_loss`: no host read under graph capture).
 * Streams: large batches run in up to three length-sorted groups, two of them on streams of the
 *   library's own (created on the first such call on a device, forked from and joined back into
 *   `stream` with events, so the call stays ordered on `stream` and is graph-capturable).  A call
 *   captured before that device's streams exist runs as one group on `stream`.
 * checkpoint_interval K (a power of two in [1, 32]; [PR] `_alpha_kernel` keeps every alpha row):
 *   alpha is kept for the steps 0, K, 2K, ... of each utterance only, and the rows of each K-step
 *   interval recompute it from the kept step, so the alpha part of the workspace shrinks about
 *   K-fold (beta is kept for every step).  K = 1 keeps every row.  K > 1 runs the grouped pipeline
 *   (see packed_ctc_set_pipeline), takes float32 / bfloat16 / float16 inputs (PCTC_ERR_ARG for
 *   float64) and target lengths up to 1023 (PCTC_ERR_LIMIT beyond).  Results agree with K = 1 to
 *   float32 rounding.
 * The workspace must be at least packed_ctc_workspace_size(T_total, D, B, bound, K) bytes, bound =
 *   max_target_length if >= 0 else target_width, and 256-byte aligned.
 * log_probs and grad_out must be 16-byte aligned (PCTC_ERR_ARG otherwise).
 * Rows of different utterances must not overlap.  Inputs are read only; outputs are fully written.
 */
int packed_ctc_loss(const void* log_probs, int dtype, int64_t T_total, int64_t D, const void* cu_seqlens,
                    const void* lengths, int64_t B, const void* targets, int64_t target_width,
                    const void* target_lengths, int index_flags, int64_t max_target_length, int blank,
                    int zero_infinity, int reduction, const void* grad_scale, void* losses_out, void* reduced_out,
                    void* grad_out, int checkpoint_interval, void* workspace, size_t workspace_bytes, void* stream);

/*
 * packed_ctc_loss without a workspace argument, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid hipMalloc).  Arguments and
 * results as for packed_ctc_loss, with these differences:
 *   - the workspace is a 128 MiB device array of the library's own, one per device, held from the
 *     library's first use on that device until the process ends; a call whose workspace
 *     (packed_ctc_workspace_size) exceeds 128 MiB fails with PCTC_ERR_WORKSPACE and launches nothing;
 *   - max_target_length must be >= 0 (no host read; PCTC_ERR_ARG otherwise);
 *   - the call runs on `stream` alone (one utterance group, no streams or events of the library).
 * The call allocates nothing: no hipMalloc, hipFree or allocating library routine.  Every region of
 * the array that a call's kernels read is written earlier in the same call, so nothing carries over
 * from the previous call; calls that overlap on one device (other streams, other host threads)
 * share the array and race: callers serialise them.
 */
int packed_ctc_loss_noalloc(const void* log_probs, int dtype, int64_t T_total, int64_t D, const void* cu_seqlens,
                            const void* lengths, int64_t B, const void* targets, int64_t target_width,
                            const void* target_lengths, int index_flags, int64_t max_target_length, int blank,
                            int zero_infinity, int reduction, const void* grad_scale, void* losses_out,
                            void* reduced_out, void* grad_out, int checkpoint_interval, void* stream);

/*
 * The same computation split at the autograd boundary ([PR] `_PackedCTCLoss.forward` stores alpha
 * and the inputs; `_PackedCTCLoss.backward` runs beta and the gradient with the upstream
 * `grad_output`).
 *
 * packed_ctc_forward: losses_out and reduced_out exactly as packed_ctc_loss with grad_out = NULL,
 *   and the workspace left holding what packed_ctc_backward reads: with the streamed pipeline
 *   (float32 / 16-bit inputs, checkpoint_interval 1, up to 2048 utterances) every row's posterior
 *   sums per class, formed while the recursions run, so the backward only writes the gradient
 *   rows; otherwise the recursions' state (alpha at every step or every checkpoint_interval-th,
 *   beta, offsets, schedule).  Arguments as for packed_ctc_loss.
 * packed_ctc_backward: grad_out (T_total, D) exactly as packed_ctc_loss would write it with the
 *   given grad_scale and reduction (w_b = grad_scale[b] or 1, times 1/(B * max(U_b, 1)) for MEAN,
 *   0 under zero_infinity for an infinite loss).  For autograd, grad_scale[b] is the upstream
 *   gradient of loss b (NONE), or the upstream scalar for every b (SUM, MEAN).
 *   Precondition: `workspace` holds the state of a packed_ctc_forward call on the same stream with
 *   the same log_probs, sizes, index arrays, blank, checkpoint_interval and max_target_length (>= 0
 *   here: it must be the bound the forward used; PCTC_ERR_ARG if negative), not reused by another
 *   call since.  The
 *   workspace is read, and only its weight, class-map and row-sum regions are rewritten, so the
 *   backward may be repeated with other grad_scale values.  zero_infinity and reduction may differ
 *   from the forward's; they only set the weights.
 * Error codes and alignment rules as for packed_ctc_loss.  Both calls are asynchronous on `stream`
 *   and allocate nothing.
 */
int packed_ctc_forward(const void* log_probs, int dtype, int64_t T_total, int64_t D, const void* cu_seqlens,
                       const void* lengths, int64_t B, const void* targets, int64_t target_width,
                       const void* target_lengths, int index_flags, int64_t max_target_length, int blank,
                       int zero_infinity, int reduction, void* losses_out, void* reduced_out,
                       int checkpoint_interval, void* workspace, size_t workspace_bytes, void* stream);

int packed_ctc_backward(const void* log_probs, int dtype, int64_t T_total, int64_t D, const void* cu_seqlens,
                        const void* lengths, int64_t B, const void* targets, int64_t target_width,
                        const void* target_lengths, int index_flags, int64_t max_target_length, int blank,
                        int zero_infinity, int reduction, const void* grad_scale, void* grad_out,
                        int checkpoint_interval, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The split for autograd when the upstream gradient is usually one (a reduced loss that is
 * backpropagated as it is): the forward writes the gradient too, and the backward leaves it alone
 * when the upstream weights are all one, deciding on the device (no host read, graph-capturable).
 * [PR] `_PackedCTCLoss.backward` forms the rows with `grad_output` as each utterance's weight; these
 * calls give the same rows.
 *
 * packed_ctc_forward_grad: losses_out, reduced_out and grad_out exactly as packed_ctc_loss with
 *   grad_scale = NULL (w_b from the reduction and zero_infinity alone), and the workspace left
 *   holding what packed_ctc_backward reads (with the streamed pipeline: every row's class sums, as
 *   packed_ctc_forward leaves them), with a record that grad_out holds the rows for unit upstream
 *   weights under this zero_infinity and reduction.  max_target_length must be >= 0
 *   (PCTC_ERR_ARG otherwise).  Other arguments as for packed_ctc_loss.
 * packed_ctc_backward_update: grad_out as packed_ctc_backward writes it, with one difference: when
 *   every grad_scale[b] is exactly 1 (or grad_scale is NULL) and zero_infinity and reduction are
 *   the forward's, the rows are left as they are and no row is read or written (a few microseconds).
 *   Precondition, beside packed_ctc_backward's: grad_out is the buffer packed_ctc_forward_grad
 *   wrote, changed since only by packed_ctc_backward_update calls on the same workspace (an update
 *   with other weights rewrites the rows and clears the record, so a later update with unit
 *   weights rewrites them again).  Arguments, error codes and alignment as for packed_ctc_backward.
 * Both calls are asynchronous on `stream` and allocate nothing.
 */
int packed_ctc_forward_grad(const void* log_probs, int dtype, int64_t T_total, int64_t D, const void* cu_seqlens,
                            const void* lengths, int64_t B, const void* targets, int64_t target_width,
                            const void* target_lengths, int index_flags, int64_t max_target_length, int blank,
                            int zero_infinity, int reduction, void* losses_out, void* reduced_out, void* grad_out,
                            int checkpoint_interval, void* workspace, size_t workspace_bytes, void* stream);

int packed_ctc_backward_update(const void* log_probs, int dtype, int64_t T_total, int64_t D, const void* cu_seqlens,
                               const void* lengths, int64_t B, const void* targets, int64_t target_width,
                               const void* target_lengths, int index_flags, int64_t max_target_length, int blank,
                               int zero_infinity, int reduction, const void* grad_scale, void* grad_out,
                               int checkpoint_interval, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Reduction of per-utterance losses ([PR] `ctc.py` `forward_packed`): SUM = sum of losses[b];
 * MEAN = mean over b of losses[b] / max(target_lengths[b], 1); B = 0 gives 0 (SUM) or NaN (MEAN).
 * Writes one float to *out (device).  NONE is PCTC_ERR_ARG.  Only the target-length bit of
 * index_flags is read.
 */
int packed_ctc_reduce(const float* losses, const void* target_lengths, int index_flags, int64_t B, int reduction,
                      float* out, void* stream);

/*
 * Health word of the last call that used this workspace.  The recursions of one utterance run as a
 * pipeline of state blocks that wait on each other, and the rows of the streamed pipeline wait on
 * the recursions; every such wait is bounded in wall-clock time (packed_ctc_set_wait_limit).  A wave
 * that runs out of time sets the health word and carries on, so every kernel still ends; the call
 * then writes NaN into every entry of losses_out and into reduced_out, and its gradient is
 * unspecified (the rows formed after the give-up are NaN).  Waits for `stream`, then stores 0
 * (healthy) or non-zero in *status_out.
 */
int packed_ctc_workspace_status(const void* workspace, void* stream, int* status_out);

/*
 * Wall-clock bound, in microseconds, of each wait of one wave on another inside the kernels
 * (default 2 s, far beyond any wait of a healthy call; 0 makes every wait that is not met at once
 * give up, which tests use to check the failure path).  Process-wide; read when a call is enqueued.
 * Returns PCTC_OK, or PCTC_ERR_ARG outside [0, 3600 s].  packed_ctc_wait_limit returns the bound.
 */
int packed_ctc_set_wait_limit(int64_t microseconds);
int64_t packed_ctc_wait_limit(void);

/* Message of the last failing call on this thread ("" if none). */
const char* packed_ctc_last_error(void);

/* Library version string. */
const char* packed_ctc_version(void);

/*
 * Process-wide choice of pipeline for packed_ctc_loss calls with a gradient; both compute the same
 * losses and gradient rows (the page's `_alpha_kernel` / `_beta_grad_kernel` split, NVIDIA-NeMo/Speech
 * pull request "feat(asr): native CTC loss kernel over sequence-packed log probabilities", leaves the
 * order of the work open).
 *   PCTC_PIPELINE_STREAMED (default): after the label gather, one persistent launch runs the alpha
 *     and beta recursions and hands out each utterance's rows in bands as soon as both recursions
 *     have passed them (middle frames first), so posteriors and gradient rows stream beside the
 *     recursions.  Used for float32, bfloat16 and float16 inputs of up to 2048 utterances whose
 *     per-wave LDS (class sums, class bitmap) fits; other calls take the grouped pipeline.
 *   PCTC_PIPELINE_GROUPED: utterances sorted by frame count and cut into up to three groups on
 *     concurrent streams; each group forms its rows after its recursions end.
 * Loss-only calls and the split forward / backward entry points do not depend on it.
 * packed_ctc_set_pipeline returns PCTC_OK or PCTC_ERR_ARG (unknown value); packed_ctc_pipeline returns
 * the current choice.  Calls already enqueued are not affected.
 */
int packed_ctc_set_pipeline(int pipeline);
int packed_ctc_pipeline(void);

/*
 * Measurement hook.  While enabled, packed_ctc_loss records a HIP event before and after each of
 * its kernels on the call's stream, for up to the last 128 calls.  Enabling (or disabling) resets
 * the record.  packed_ctc_phase_times waits for the last recorded call and writes up to n
 * (name, mean milliseconds over the recorded calls) pairs; it returns the number of phases, 0 if
 * none were recorded, or minus an error code.  Names are static strings.  Not thread-safe and not
 * for use under graph capture.
 */
int packed_ctc_set_phase_timing(int enable);
int packed_ctc_phase_times(const char** names, float* ms, int n);

#ifdef __cplusplus
}
#endif

#endif /* PACKED_CTC_H */
