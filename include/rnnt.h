/*
 * rnnt.h -- C ABI of librnnt, a fused RNN-T (transducer) loss, forward and
 * backward, for AMD Instinct MI355X (gfx950).
 *
 * The operation (rnnt-loss-ascend README: "Main features", the parameter
 * table, "Constraints" and "Architecture"):
 *
 *   Each sample i has T_i encoder frames and U_i target labels y_1..y_{U_i}.
 *   Its joiner logits cover the T_i x (U_i+1) lattice and are packed, without
 *   padding, as T_i*(U_i+1) consecutive rows of V classes; samples follow each
 *   other in batch order, so the whole input is a (N, V) row-major matrix with
 *   N = sum_i T_i*(U_i+1).  Inside a sample, rows are t-major: row
 *   t*(U_i+1) + u is lattice node (t,u).
 *
 *   With fused_log_softmax set, a log_softmax over V is applied at every node;
 *   otherwise the inputs are taken as log-probabilities as they are.  The
 *   loss of a sample is -log of the total probability of all alignments from
 *   node (0,0) that emit blank to advance t and emit y_{u+1} to advance u, and
 *   end by emitting blank at (T_i-1, U_i) (warp-transducer build post,
 *   section 1.1; README "Value" section 2 gives the gradient of it).  The
 *   forward (alpha) and backward (beta) recursions are both run and their
 *   two losses cross-checked (README "Value" section 3).  The README fixes
 *   the log domain for stability; here the recursions carry fp64
 *   probabilities rescaled by a power of two per block of anti-diagonals
 *   (exact up to fp64 rounding while the nodes that carry alignment mass
 *   stay in fp64's range, which a per-sample check verifies), and a sample
 *   that leaves that range is recomputed in the log domain (see the
 *   numerics note under rnnt_loss_fused).
 *
 *   The gradient is with respect to the packed input (logits, or the given
 *   log-probabilities when fused_log_softmax is 0).  With clamp > 0 every
 *   gradient element of a sample is clipped to [-clamp, clamp] before the
 *   reduction scale is applied (README "Operator features"); clamp <= 0
 *   disables clipping.  Reduction none / mean / sum follows the README usage
 *   example (mean is over the batch dimension).
 *
 * Conventions for every entry point:
 *   - "host" pointers are read by the CPU during the call and may be reused
 *     as soon as it returns; "device" pointers are HIP device memory.
 *   - The caller owns every buffer.  The library performs no device memory
 *     allocation.  It keeps a small reusable pinned host staging ring per
 *     device for uploading the per-call schedule.
 *   - All device work is enqueued on `stream` (a hipStream_t; NULL means the
 *     default stream); calls return before it completes.
 *   - HIP graph capture: an rnnt_loss_fused / rnnt_loss_padded call with
 *     B <= 64 enqueues kernels only (its schedule travels as kernel
 *     arguments), so it can be captured and replayed; a replay recomputes
 *     the same lengths, pointers and sizes it was captured with.  Calls that
 *     copy their schedule from the host (B > 64, and every
 *     rnnt_multiblank_loss call) return RNNT_INVALID_VALUE on a capturing
 *     stream, before enqueuing anything.  Kernel timing must be off while
 *     capturing.
 *   - Host-detectable argument errors return a non-zero rnnt_status before
 *     anything is enqueued; outputs are then untouched.  Problems only the
 *     device can see set bits in a status word kept in the workspace (see
 *     rnnt_loss_fused_check).  No entry point aborts or throws.
 */
#ifndef RNNT_H_
#define RNNT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *rnnt_stream_t; /* a hipStream_t */

/*
 * Each enum below carries two reserved enumerators at the ends of the int32
 * range, so that every int32 value is a valid value of the type: a code the
 * library does not know is refused with RNNT_INVALID_VALUE (or described as
 * "unknown status") instead of being undefined in the C++ implementation.
 */

/* Element type of logits and grad (README parameter table: float32 / float16). */
typedef enum {
    RNNT_F32 = 0,
    RNNT_F16 = 1,
    RNNT_DTYPE_RESERVED_MIN_ = -0x7fffffff - 1,
    RNNT_DTYPE_RESERVED_MAX_ = 0x7fffffff
} rnnt_dtype;

/* Reduction of the per-sample losses (README usage example). */
typedef enum {
    RNNT_REDUCTION_NONE = 0,
    RNNT_REDUCTION_MEAN = 1,
    RNNT_REDUCTION_SUM = 2,
    RNNT_REDUCTION_RESERVED_MIN_ = -0x7fffffff - 1,
    RNNT_REDUCTION_RESERVED_MAX_ = 0x7fffffff
} rnnt_reduction;

/* Return status of every entry point (the ESPnet GPURNNT page's RNNTStatus:
 * success or a failure code; its RNNT_STATUS_INVALID_VALUE for bad inputs). */
typedef enum {
    RNNT_SUCCESS = 0,
    RNNT_INVALID_VALUE = 1,       /* an argument violates the constraints below */
    RNNT_WORKSPACE_TOO_SMALL = 2, /* workspace_bytes below what _workspace_size reported */
    RNNT_MEMOPS_FAILED = 3,       /* a HIP copy or host staging allocation failed */
    RNNT_EXECUTION_FAILED = 4,    /* a kernel launch failed */
    RNNT_STATUS_RESERVED_MIN_ = -0x7fffffff - 1,
    RNNT_STATUS_RESERVED_MAX_ = 0x7fffffff
} rnnt_status;

/* Bits of the device status word (read back by rnnt_loss_fused_check). */
enum {
    RNNT_DEV_LOSS_MISMATCH = 1u, /* |L_alpha - L_beta| > 1e-4 * max(1, |L_beta|) for some sample */
    RNNT_DEV_BAD_TARGET = 2u     /* a label y_u lies outside [0, V) or equals a blank */
};

/*
 * Bytes of device workspace rnnt_loss_fused needs for this batch.
 *
 *   B                 number of samples, >= 1.
 *   V                 classes per row (blank included), >= 1.
 *   N                 rows of the packed logits; must equal sum_i T_i*(U_i+1).
 *   dtype             RNNT_F32 or RNNT_F16.
 *   logit_lengths     host int32[B]: T_i >= 1.
 *   target_lengths    host int32[B]: 0 <= U_i <= 2047 (U_i+1 is the lattice
 *                     width; the alpha/beta kernels keep a whole anti-diagonal
 *                     of up to 2048 nodes in registers: one wavefront's up to
 *                     1024 columns, a workgroup of up to eight above).
 *   workspace_bytes   out: required size; the caller allocates it (any
 *                     alignment of 256 bytes or more) and passes it back.
 * Runs every host-side check of rnnt_loss_fused that does not need the
 * other pointers, so invalid lengths fail here first.  Touches no GPU.
 */
rnnt_status rnnt_loss_fused_workspace_size(int32_t B, int32_t V, int64_t N, rnnt_dtype dtype,
                                           const int32_t *logit_lengths, const int32_t *target_lengths,
                                           size_t *workspace_bytes);

/*
 * Fused loss and gradient (README "Architecture": one call produces both).
 *
 *   logits            device (N, V) row-major, dtype; the packed layout above.
 *   targets           device int32 (B, S) row-major; row i holds y_1..y_{U_i}
 *                     in its first U_i entries; the rest is never read.  May
 *                     be NULL only when every U_i is 0.
 *   S                 row stride of targets, >= max_i U_i.
 *   logit_lengths, target_lengths   host int32[B], as for _workspace_size.
 *   blank             in [-V, V-1]; a negative value counts from the end
 *                     (-1 is V-1, -V is 0).
 *   clamp             > 0 clips each per-sample gradient element to
 *                     [-clamp, clamp]; <= 0 disables clipping.
 *   fastemit_lambda   FastEmit regularisation weight, finite and >= 0 (the
 *                     fastemit_lambda of the GPURNNT parameter list on the
 *                     ESPnet multi-blank utilities page, defined by the
 *                     FastEmit paper it refers to): the gradient with
 *                     respect to every label-emission log-probability is
 *                     multiplied by (1 + fastemit_lambda) before the
 *                     log_softmax chain rule and the clamp; blank emissions
 *                     and the loss value are unchanged.  0: the plain loss.
 *   fused_log_softmax non-zero: apply log_softmax over V at each node.
 *   reduction         RNNT_REDUCTION_NONE / _MEAN / _SUM.
 *   loss              device float[B]: per-sample loss -log P(y|x) (beta
 *                     path), always fp32 whatever dtype is.
 *   loss_reduced      device float[1] or NULL: sum (SUM) or sum/B (MEAN) of
 *                     loss; ignored for NONE.
 *   grad              device (N, V) of dtype, or NULL to skip the gradient.
 *                     Receives d(reduced loss)/d(logits) for a unit upstream
 *                     gradient: the clamped per-sample gradient, times 1/B
 *                     for MEAN.  Every element is written; no zero fill is
 *                     needed.  grad may equal logits exactly (in place);
 *                     any other overlap is RNNT_INVALID_VALUE.
 *   workspace         device, workspace_bytes >= the _workspace_size value.
 *   stream            hipStream_t for all device work.
 * Returns RNNT_INVALID_VALUE for a NULL required pointer, bad dtype or
 * reduction, V < 1, B < 1, blank out of range, fastemit_lambda negative or not
 * finite, T_i < 1, U_i < 0, U_i > 2047, U_i > S, a sample with
 * (T_i + U_i) * max(8 * U1p_i, 16 * (U_i + 1)) >= 2^31 (U1p_i = 64 for
 * U_i < 64, 128 for U_i < 128, else U_i + 1 rounded up to a multiple of
 * 256: the recursions
 * address one sample's tables with 32-bit offsets; T_i + U_i up to 131071
 * at any width), sum_i T_i*(U_i+1) != N or partial overlap of grad and logits;
 * RNNT_WORKSPACE_TOO_SMALL; RNNT_MEMOPS_FAILED; RNNT_EXECUTION_FAILED.
 * Invalid label values are only visible on the device: they set
 * RNNT_DEV_BAD_TARGET.  A label outside [0, V) or equal to blank is no
 * symbol an alignment can emit (warp-transducer build post, section 5.2:
 * the labels exclude blank), so its sample has no alignment: loss +inf and
 * a zero gradient for that sample; the other samples are unaffected.
 * Numerics: the recursions run in fp64 probabilities scaled by a power of
 * two per block of anti-diagonals.  A sample takes the log domain instead
 * when one of its edge log-probabilities lies outside [-80, 80], or when
 * the forward-backward identity (alpha * beta summed over an anti-diagonal
 * is P(y|x)) fails by more than 4e-6 in log2 on one of 16 checked
 * diagonals: nodes carrying alignment mass fell out of fp64's range; the
 * sample is then recomputed in the log domain within the same call.
 */
rnnt_status rnnt_loss_fused(const void *logits, rnnt_dtype dtype, int64_t N, int32_t V,
                            const int32_t *targets, int32_t S,
                            const int32_t *logit_lengths, const int32_t *target_lengths, int32_t B,
                            int64_t blank, float clamp, float fastemit_lambda, int fused_log_softmax,
                            rnnt_reduction reduction, float *loss, float *loss_reduced, void *grad,
                            void *workspace, size_t workspace_bytes, rnnt_stream_t stream);

/*
 * Multiply the gradient written by rnnt_loss_fused by an upstream gradient
 * kept in device memory (the backward step of the reduction, README
 * "Architecture": reduction is handled above the kernel).
 *
 *   grad, dtype, N, V, logit_lengths, target_lengths, B   as passed to the
 *                 rnnt_loss_fused call that wrote grad.
 *   scale         device float[1] (per_sample = 0) or float[B] (per_sample =
 *                 1, for reduction NONE: the rows of sample i are scaled by
 *                 scale[i]).
 *   workspace     the workspace of that call, not reused by another call on
 *                 a different batch in between (its schedule tables are read).
 * Rows whose factor is exactly 1 are left untouched, so a unit upstream
 * gradient costs no memory traffic.  Returns RNNT_INVALID_VALUE for NULL
 * pointers or inconsistent sizes.
 */
rnnt_status rnnt_grad_scale(void *grad, rnnt_dtype dtype, int64_t N, int32_t V, const int32_t *logit_lengths,
                            const int32_t *target_lengths, int32_t B, const float *scale, int per_sample,
                            const void *workspace, size_t workspace_bytes, rnnt_stream_t stream);

/*
 * The same loss and gradient for logits in the padded (B, max_T, max_U1, V)
 * layout that warp-transducer / GPURNNT style pipelines hand over (GPURNNT
 * API page: activations of shape [B, T, U, V+1], T and U the batch maxima):
 * node (t, u) of sample i is row (i*max_T + t)*max_U1 + u of a row-major
 * (B*max_T*max_U1, V) matrix; rows with t >= T_i or u > U_i are padding.
 *
 *   max_T, max_U1     the padded extents: T_i <= max_T and U_i + 1 <= max_U1
 *                     for every sample, else RNNT_INVALID_VALUE.
 *   logits, grad      device (B*max_T*max_U1, V) of dtype.  Padding rows of
 *                     logits never enter a result (where rows are no multiple
 *                     of 16 bytes, a few of their bytes next to a lattice row
 *                     are loaded with it and ignored).  Every element of grad is
 *                     written: the rows of each lattice as by rnnt_loss_fused,
 *                     the padding rows with zeros (no zero fill is needed
 *                     beforehand, unlike GPURNNT's grads).  grad may equal
 *                     logits exactly; any other overlap is RNNT_INVALID_VALUE.
 *   everything else   as for rnnt_loss_fused; the workspace size comes from
 *                     rnnt_loss_padded_workspace_size with the same extents.
 */
rnnt_status rnnt_loss_padded_workspace_size(int32_t B, int32_t V, int32_t max_T, int32_t max_U1, rnnt_dtype dtype,
                                            const int32_t *logit_lengths, const int32_t *target_lengths,
                                            size_t *workspace_bytes);
rnnt_status rnnt_loss_padded(const void *logits, rnnt_dtype dtype, int32_t max_T, int32_t max_U1, int32_t V,
                             const int32_t *targets, int32_t S, const int32_t *logit_lengths,
                             const int32_t *target_lengths, int32_t B, int64_t blank, float clamp,
                             float fastemit_lambda, int fused_log_softmax, rnnt_reduction reduction, float *loss,
                             float *loss_reduced, void *grad, void *workspace, size_t workspace_bytes,
                             rnnt_stream_t stream);

/*
 * rnnt_grad_scale for a gradient written by rnnt_loss_padded (all
 * B*max_T*max_U1 rows are scaled; padding rows stay zero).
 */
rnnt_status rnnt_grad_scale_padded(void *grad, rnnt_dtype dtype, int32_t max_T, int32_t max_U1, int32_t V,
                                   const int32_t *logit_lengths, const int32_t *target_lengths, int32_t B,
                                   const float *scale, int per_sample, const void *workspace,
                                   size_t workspace_bytes, rnnt_stream_t stream);

/*
 * rnnt_loss_fused without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory during the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The workspace is a fixed device array inside the library, 128 MiB
 * (RNNT_NOALLOC_SCRATCH_BYTES) per device, held by every device that loads
 * the library until the process ends.  The call makes no device, pinned or
 * host heap allocation and uses no plan cache; its address is looked up
 * once per device on the first call made with that device current.
 *
 *   Arguments as for rnnt_loss_fused (packed layout), minus the workspace,
 *   plus:
 *   dev_status        device uint32, or NULL: receives the device status
 *                     word of this call (RNNT_DEV_* bits), which
 *                     rnnt_loss_fused_check would read from a workspace.
 * Returns what rnnt_loss_fused returns, and RNNT_INVALID_VALUE for B > 64
 * (the schedule travels as kernel arguments; larger batches would need the
 * host staging copy, which allocates), RNNT_WORKSPACE_TOO_SMALL when the
 * batch needs more than RNNT_NOALLOC_SCRATCH_BYTES of workspace (the size
 * rnnt_loss_fused_workspace_size reports), RNNT_MEMOPS_FAILED when the
 * scratch address cannot be obtained.
 * Every call on one device shares that device's scratch and leaves its
 * contents behind (the next call rewrites what it reads; the status word is
 * cleared at the start of each call): calls that overlap in time on one
 * device, from several streams or threads, race and give undefined
 * results.  Serialise them (one stream, or events between streams).
 */
#define RNNT_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
rnnt_status rnnt_loss_fused_noalloc(const void *logits, rnnt_dtype dtype, int64_t N, int32_t V,
                                    const int32_t *targets, int32_t S, const int32_t *logit_lengths,
                                    const int32_t *target_lengths, int32_t B, int64_t blank, float clamp,
                                    float fastemit_lambda, int fused_log_softmax, rnnt_reduction reduction,
                                    float *loss, float *loss_reduced, void *grad, uint32_t *dev_status,
                                    rnnt_stream_t stream);

/*
 * Multi-blank transducer loss and gradient (the ESPnet
 * compute_multiblank_grad_kernel page: activations over the labels, the
 * standard blank and num_big_blanks big blanks; each big blank has a
 * duration; sigma is the logit under-normalisation hyper-parameter; the page
 * defers the mathematics to the multi-blank transducer paper).  Reading
 * taken: from node (t,u) the standard blank moves to (t+1,u), big blank i to
 * (t + big_blank_durations[i], u) and the next label to (t,u+1); every
 * emission's log-probability is lowered by sigma; an alignment ends when a
 * blank of any kind reaches t = T exactly at u = U.  The loss is -log of the
 * summed alignment probability, the gradient its derivative (with the
 * FastEmit weight on the label emissions).  With no big blank and sigma = 0
 * this is rnnt_loss_fused's loss.
 *
 *   Packed layout only; logits, targets, S, lengths, blank, clamp,
 *   fastemit_lambda, fused_log_softmax, reduction, loss, loss_reduced, grad
 *   (NULL: loss only) and stream as for rnnt_loss_fused.
 *   num_big_blanks    0..4.
 *   big_blank_ids     host int32[num_big_blanks]: the class of each big blank,
 *                     in [0, V), distinct, none equal to the standard blank.
 *   big_blank_durations  host int32[num_big_blanks], each in [1, 16].
 *   sigma             finite; subtracted from every emission's log-probability.
 *   workspace         device, >= rnnt_multiblank_workspace_size bytes, 256-byte
 *                     aligned.
 * Returns RNNT_INVALID_VALUE for the conditions of rnnt_loss_fused, a U_i
 * above 1023 (its sweep keeps an anti-diagonal of up to 1024 nodes in one
 * wavefront), a bad big blank list, a non-finite sigma, a batch whose widest lattice and longest
 * duration need more than 64 KiB of ring per sweep, i.e. R * U1p * 8 bytes
 * > 64 KiB with R the power of two above the longest duration and U1p the
 * widest U_i + 1 rounded up to 128 times a power of two (at U1p = 1024 the
 * longest duration is 7, at 512 it is 15), or a sample with
 * (T_i + U_i) * U1p * 8 >= 2^31.  A label equal to blank or to a big
 * blank, or outside [0, V), sets RNNT_DEV_BAD_TARGET (read with
 * rnnt_loss_fused_check) and leaves its sample without an alignment (loss
 * +inf, zero gradient), as in rnnt_loss_fused.
 * The recursion runs in fp64 probabilities renormalised per anti-diagonal;
 * when the identity that every alignment emits each label once (the sum
 * over t of alpha(t,u) P(label) beta(t,u+1) is P(y|x)) fails by more than
 * 4e-6 in log2 on one of 16 checked columns, nodes carrying alignment mass
 * fell out of fp64's range and the sample is recomputed in the log domain
 * within the same call.  The edge weights are kept as fp64 probabilities,
 * so an edge whose log-probability (less sigma) is below about -745 counts
 * as probability zero in either domain.
 */
rnnt_status rnnt_multiblank_workspace_size(int32_t B, int32_t V, int64_t N, rnnt_dtype dtype,
                                           const int32_t *logit_lengths, const int32_t *target_lengths,
                                           int32_t num_big_blanks, const int32_t *big_blank_durations,
                                           size_t *workspace_bytes);
rnnt_status rnnt_multiblank_loss(const void *logits, rnnt_dtype dtype, int64_t N, int32_t V,
                                 const int32_t *targets, int32_t S, const int32_t *logit_lengths,
                                 const int32_t *target_lengths, int32_t B, int64_t blank, int32_t num_big_blanks,
                                 const int32_t *big_blank_ids, const int32_t *big_blank_durations, float sigma,
                                 float clamp, float fastemit_lambda, int fused_log_softmax,
                                 rnnt_reduction reduction, float *loss, float *loss_reduced, void *grad,
                                 void *workspace, size_t workspace_bytes, rnnt_stream_t stream);

/*
 * The multi-blank loss for logits in the padded (B, max_T, max_U1, V) layout
 * (the compute_multiblank_grad_kernel page's activations [B, T, U, V + 1 +
 * num_big_blanks]): node (t, u) of sample i is row (i*max_T + t)*max_U1 + u;
 * padding rows of logits never enter a result and get a zero gradient
 * (written by the gradient pass itself).  Arguments and limits as for
 * rnnt_multiblank_loss, with max_T >= T_i and max_U1 >= U_i + 1 for every
 * sample, and the workspace sized by rnnt_multiblank_padded_workspace_size.
 */
rnnt_status rnnt_multiblank_padded_workspace_size(int32_t B, int32_t V, int32_t max_T, int32_t max_U1,
                                                  rnnt_dtype dtype, const int32_t *logit_lengths,
                                                  const int32_t *target_lengths, int32_t num_big_blanks,
                                                  const int32_t *big_blank_durations, size_t *workspace_bytes);
rnnt_status rnnt_multiblank_loss_padded(const void *logits, rnnt_dtype dtype, int32_t max_T, int32_t max_U1,
                                        int32_t V, const int32_t *targets, int32_t S,
                                        const int32_t *logit_lengths, const int32_t *target_lengths, int32_t B,
                                        int64_t blank, int32_t num_big_blanks, const int32_t *big_blank_ids,
                                        const int32_t *big_blank_durations, float sigma, float clamp,
                                        float fastemit_lambda, int fused_log_softmax, rnnt_reduction reduction,
                                        float *loss, float *loss_reduced, void *grad, void *workspace,
                                        size_t workspace_bytes, rnnt_stream_t stream);

/*
 * rnnt_grad_scale for a gradient written by rnnt_multiblank_loss (same
 * arguments; the workspace is that call's), and for one written by
 * rnnt_multiblank_loss_padded (all B*max_T*max_U1 rows are scaled; padding
 * rows stay zero).
 */
rnnt_status rnnt_multiblank_grad_scale(void *grad, rnnt_dtype dtype, int64_t N, int32_t V,
                                       const int32_t *logit_lengths, const int32_t *target_lengths, int32_t B,
                                       const float *scale, int per_sample, const void *workspace,
                                       size_t workspace_bytes, rnnt_stream_t stream);
rnnt_status rnnt_multiblank_grad_scale_padded(void *grad, rnnt_dtype dtype, int32_t max_T, int32_t max_U1,
                                              int32_t V, const int32_t *logit_lengths,
                                              const int32_t *target_lengths, int32_t B, const float *scale,
                                              int per_sample, const void *workspace, size_t workspace_bytes,
                                              rnnt_stream_t stream);

/*
 * Synchronises `stream`, then copies into *dev_flags the device status word
 * (RNNT_DEV_* bits) of the most recent rnnt_loss_fused call that used
 * `workspace`; every rnnt_loss_fused call clears it when it starts.  The
 * status codes follow the ESPnet GPURNNT page's RNNTStatus (success, or a
 * failure such as RNNT_STATUS_INVALID_VALUE); the per-sample problems only
 * the device can see (README "Value" section 3: the alpha and beta losses
 * must agree; the build post's section 5.2: labels exclude blank) come back
 * as these bits.  RNNT_INVALID_VALUE for a NULL workspace or dev_flags;
 * RNNT_MEMOPS_FAILED if the copy or the synchronisation fails.
 */
rnnt_status rnnt_loss_fused_check(void *workspace, rnnt_stream_t stream, uint32_t *dev_flags);

/* Static English description of a status code (the ESPnet GPURNNT page's
 * RNNTStatus codes as numbered above); "unknown status" for any other value.
 * Never NULL; the string is owned by the library. */
const char *rnnt_status_string(rnnt_status s);

/*
 * Host-side schedule of a batch, for inspection and tests; touches no GPU.
 * Fills up to `cap` entries of each array (any may be NULL):
 *   sample_order  int32[B]: samples by decreasing lattice area T*(U+1)
 *                 (ties: larger T+U first, then lower index) -- the order in
 *                 which the alpha/beta work of each sample is started
 *                 (README "Operator features": largest tasks first).
 *   chunk_sample, chunk_row_begin, chunk_row_count   int32[n_chunks]: the
 *                 runs of lattice nodes the row passes hand to one
 *                 workgroup each, in issue order; each lies inside one
 *                 sample.  Kernels that take several short rows per
 *                 wavefront walk a run in row order: sample-local rows
 *                 chunk_row_begin .. +chunk_row_count-1.
 *   chunk_diag, chunk_col   int32[n_chunks]: kernels that take one row per
 *                 wavefront walk the same number of nodes in anti-diagonal
 *                 order (diagonal n = t+u, then column u), from node
 *                 (n, u) = (chunk_diag, chunk_col); both orders cut every
 *                 sample after the same node counts.
 *   n_chunks      out: total number of chunks (may exceed cap).
 * Returns RNNT_INVALID_VALUE under the same length checks as _workspace_size.
 */
rnnt_status rnnt_plan_describe(int32_t B, int32_t V, rnnt_dtype dtype,
                               const int32_t *logit_lengths, const int32_t *target_lengths,
                               int32_t cap, int32_t *sample_order, int32_t *chunk_sample,
                               int32_t *chunk_row_begin, int32_t *chunk_row_count,
                               int32_t *chunk_diag, int32_t *chunk_col, int32_t *n_chunks);

/*
 * Per-kernel timing for measurement.  While enabled, every rnnt_loss_fused
 * call brackets each of its kernels with HIP events on its own stream.
 * rnnt_timing_read synchronises on the recorded events and returns, for
 * each kernel, the summed device milliseconds and the number of launches
 * since timing was enabled (index 0 rowstats / gather, 1 alpha_beta,
 * 2 grad, 3 reduce); ms and launches are arrays of 4, either may be NULL.
 * rnnt_timing_enable(0) stops recording and discards what was recorded.
 * Not for concurrent use from several threads.
 */
rnnt_status rnnt_timing_enable(int on);
rnnt_status rnnt_timing_read(double *ms, int32_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* RNNT_H_ */
