/*
 * vwc.h -- selected-token log-probabilities, entropy and the logit gradient
 * from LM-head logits, on one AMD Instinct MI355X (gfx950).
 *
 * For each row r of a logits matrix x and a temperature tau, with z = x / tau:
 *   lse[r]     = log sum_j exp(z[r, j])
 *   logprob[r] = z[r, t_r] - lse[r]            (= log_softmax(z)[t_r])
 *   entropy[r] = -sum_j p_rj log p_rj,  p_rj = exp(z[r, j] - lse[r])
 *   grad[r, j] = g_r * ([j == t_r] - p_rj) / tau
 * No [rows, V] float32 log-softmax or probability tensor is ever formed: each
 * call streams the logits once and keeps O(rows) state.
 *
 * Sources (web pages, cited by title and section):
 *  [A] "[RL][Performance] Avoid full-vocabulary TP gather for selected-token
 *      logprobs" -- "Proposed solution": the selected log-probability equals
 *      minus the token cross entropy; "Prototype correctness": masked positions
 *      get exactly zero gradient; "Problem": only one selected token per
 *      position is needed, not the full-vocabulary tensor.
 *  [B] "fix: chunk target logprobs without tensor parallelism (long-context
 *      OOM)" -- "Changes": forward = float32 logsumexp + gather of the target
 *      logit, saving only the logits (own dtype) and targets; backward =
 *      recompute the softmax and write (onehot - softmax) * grad_output into a
 *      buffer of the logits' dtype; "Verification": zero-length sequences.
 *  [C] "[megatron] feat: add memory-efficient chunked top-k KL computation" --
 *      "Design & Code Changes": the backward keeps the low-precision logits
 *      and a per-token fp32 logZ and recomputes probabilities.
 *  [D] "[Bug] Training/log-prob forward materializes full-vocab fp32 logits
 *      over the entire packed sequence ..." -- maintainer comment: compute
 *      log-prob and entropy on the compact loss-mask rows, scatter scalars
 *      back; empty masks.
 *  [E] "feat: Reduce reference model memory with with parallel logprob
 *      computation" -- "Implementation": vocabulary shards merge a max, a sum
 *      of exp(x - max) and the target logit held by its owning shard.
 *
 * Conventions for every entry point:
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except
 *    where stated.  The library allocates nothing, keeps no pointer after the
 *    call returns and holds no state between calls; the one exception is the
 *    fixed scratch array of vwc_selected_logprob_fwd_noalloc.
 *  - Calls are asynchronous on `stream` (0 = the null stream) and never
 *    synchronize the host.  Results are ready when the stream reaches them.
 *  - Logits are row-major: element (r, j) sits at logits + (r * ld + j) * e,
 *    e = 2 (bf16) or 4 (fp32), 0 <= j < vocab <= ld.  The logits pointer must
 *    be aligned to e bytes; rows may start anywhere else.  Every row is read
 *    in 16-byte vectors from its first 16-byte boundary on, the few elements
 *    before it and past the last whole vector one by one.  A backward keeps
 *    16-byte stores when each row's boundary is also one of its gradient row
 *    (same layout, in place, or both strides whole multiples of 16 bytes with
 *    matching bases) and otherwise writes element by element (same results,
 *    slower).
 *  - logprob / lse / entropy are float32, one per output row.  Gradients are
 *    written in grad_dt (bf16 rounded to nearest-even, or fp32).
 *  - Row sets: the dense calls cover rows 0..n_rows-1.  The `_rows` calls
 *    cover rows row_idx[0..m) (int32 row ids in [0, n_rows); any order,
 *    duplicates allowed), and their per-row outputs are COMPACT: output i
 *    belongs to row row_idx[i].  targets are always indexed by ROW ID
 *    (length n_rows).
 *  - Results are deterministic: no floating-point atomics; the reduction
 *    order of a row depends only on vocab, dtype and the row's alignment, so a
 *    row gives bit-identical results through the dense and the `_rows` calls.
 *  - Errors: every argument check runs on the host before any HIP call; a
 *    failing check returns a status and launches nothing.  n_rows == 0 or
 *    m == 0 returns VWC_OK without a launch.  Data errors cannot be seen on
 *    the host: a target outside [0, vocab) gives logprob = NaN in that row
 *    (dense and `_rows`), and -infinity through the split-vocabulary calls
 *    when no slice owns it.  A row id outside [0, n_rows) gives NaN outputs
 *    (a partial with NaN s, t and w) and reads nothing.  NaN logits propagate
 *    to that row's outputs.
 *  - Detail for the last failure on the calling thread: vwc_last_error().
 */
#ifndef VWC_H
#define VWC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VWC_ABI_VERSION 1

typedef enum vwc_status {
    VWC_OK = 0,
    VWC_ERR_INVALID_ARG = 1, /* a null required pointer, a negative size, ld < vocab, ... */
    VWC_ERR_UNSUPPORTED = 2, /* a valid request the library does not handle (e.g. misaligned dtype) */
    VWC_ERR_HIP = 3,         /* a HIP launch failed; see vwc_last_error() */
    VWC_STATUS_INT_RANGE_LO_ = -0x7fffffff - 1, /* (these two make every int a value */
    VWC_STATUS_INT_RANGE_HI_ = 0x7fffffff       /*  of the type: callers pass ints) */
} vwc_status;

typedef enum vwc_dtype {
    VWC_BF16 = 0, /* bfloat16, stored as its 16-bit pattern */
    VWC_FP32 = 1, /* IEEE binary32 */
    VWC_DTYPE_INT_RANGE_LO_ = -0x7fffffff - 1, /* every int is a value; others are refused */
    VWC_DTYPE_INT_RANGE_HI_ = 0x7fffffff
} vwc_dtype;

typedef enum vwc_grad_layout {
    VWC_GRAD_COMPACT = 0, /* gradient row i of a [m, ld_grad] buffer */
    VWC_GRAD_SCATTER = 1, /* gradient row row_idx[i] of a [n_rows, ld_grad] buffer */
    VWC_GRAD_LAYOUT_INT_RANGE_LO_ = -0x7fffffff - 1, /* every int is a value; others are refused */
    VWC_GRAD_LAYOUT_INT_RANGE_HI_ = 0x7fffffff
} vwc_grad_layout;

/*
 * Partial of one vocabulary slice of one row ([E] "Implementation"; the
 * entropy term w is this library's addition so the merge also yields the
 * entropy).  With columns j of the slice and z = x / tau:
 *   m  a logit of the slice used as the reference point: m <= max_j x_j and
 *      (max_j x_j - m) / tau <= 44 (so s stays far from overflow);
 *      -infinity when the slice is empty.
 *   s  sum_j exp((x_j - m) / tau)                              (>= 1)
 *   t  the raw target logit x_t if the slice owns the target column, else
 *      -infinity (NaN when the dense calls see an out-of-range target)
 *   w  sum_j exp((x_j - m) / tau) * (x_j - m) / tau            (nats)
 * Merging k partials of the same row with M = max_k m_k, d_k = (m_k - M)/tau:
 *   S = sum_k s_k e^{d_k},  W = sum_k e^{d_k} (w_k + d_k s_k),  T = max_k t_k
 *   lse = M / tau + ln S,  logprob = (T - M) / tau - ln S,  H = ln S - W / S
 * Partials only merge with partials made at the same temperature.
 */
typedef struct vwc_partial {
    float m, s, t, w;
} vwc_partial;

/* Bytes of workspace the forward, entropy and partial calls need for `rows`
   output rows of a `vocab`-wide row (or slice) of dtype dt.  A row is cut into
   ceil(vocab * e / 128 KiB) segments (e = 2 for bf16, 4 for fp32).  Rows of up
   to 3 segments are reduced and merged inside one workgroup and need none;
   longer rows need 16 bytes per row per segment.  Never O(rows * vocab). */
size_t vwc_workspace_bytes(int64_t rows, int64_t vocab, vwc_dtype dt);

/*
 * Forward over every row ([A] "Proposed solution", [B] "Changes").
 *  logits   [n_rows, ld] of dt.
 *  targets  int32[n_rows], the selected token of each row.
 *  logprob  float[n_rows] (nullable), lse float[n_rows] (nullable; the fp32
 *           logZ the backward reads, [C]), entropy float[n_rows] (nullable).
 *  workspace / workspace_bytes: at least vwc_workspace_bytes(n_rows, vocab,
 *           dt) bytes, 16-byte aligned (nullable when that is 0).
 * At least one output must be non-null.
 */
vwc_status vwc_selected_logprob_fwd(const void *logits, vwc_dtype dt, int64_t n_rows,
                                    int64_t vocab, int64_t ld, const int32_t *targets,
                                    float temperature, float *logprob, float *lse,
                                    float *entropy, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * vwc_selected_logprob_fwd without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Results are bit-identical to
 * vwc_selected_logprob_fwd.  Rows whose forward needs segment partials
 * (vwc_workspace_bytes(n_rows, vocab, dt) > 0) keep them in a device array of
 * VWC_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (its address is looked up on the first such call on
 * a device, with that device current).  A call needing more returns
 * VWC_ERR_UNSUPPORTED before any launch: at most 65536 bf16 rows of 248320
 * columns (4 segments of 16 bytes each per row) or 32768 such fp32 rows per
 * call.  The call allocates nothing, never calls hipMalloc/hipFree, and needs
 * no clearing of the array (each call writes every partial it reads).  Calls
 * that overlap on one GPU (several streams or host threads) share that array
 * and race: serialise them.  Other arguments as vwc_selected_logprob_fwd.
 */
#define VWC_NOALLOC_SCRATCH_BYTES (4u << 20)

vwc_status vwc_selected_logprob_fwd_noalloc(const void *logits, vwc_dtype dt, int64_t n_rows,
                                            int64_t vocab, int64_t ld, const int32_t *targets,
                                            float temperature, float *logprob, float *lse,
                                            float *entropy, hipStream_t stream);

/*
 * Forward over the compact row set row_idx[0..m) ([D] maintainer comment).
 * Outputs are float[m]; workspace sized by vwc_workspace_bytes(m, vocab, dt).
 */
vwc_status vwc_selected_logprob_fwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                         int64_t vocab, int64_t ld, const int32_t *targets,
                                         const int32_t *row_idx, int64_t m, float temperature,
                                         float *logprob, float *lse, float *entropy,
                                         void *workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/* Entropy of softmax(x / tau) per row, no target ([D] "Bug Description":
   log-probs and entropy from the same logits).  entropy float[n_rows]
   required, lse nullable. */
vwc_status vwc_entropy(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                       int64_t ld, float temperature, float *entropy, float *lse,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Entropy over the compact row set row_idx[0..m); outputs float[m]. */
vwc_status vwc_entropy_rows(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                            int64_t ld, const int32_t *row_idx, int64_t m, float temperature,
                            float *entropy, float *lse, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * Backward with softmax recompute over every row ([B] "Changes", [C] "Design &
 * Code Changes", [A] "Prototype correctness").
 *  lse           float[n_rows] as written by the forward at the same temperature.
 *  grad_logprob  float[n_rows], the incoming gradient g_r of logprob[r].
 *  grad_logits   [n_rows, ld_grad] of grad_dt (ld_grad >= vocab); columns
 *                [vocab, ld_grad) are not touched.  Rows with g_r == 0 are
 *                written as +0.0 without reading their logits or lse.
 * grad_logits either is exactly logits (same pointer, dtype and ld: the
 * gradient replaces the logits in place, saving the second [rows, vocab]
 * buffer) or does not overlap them (VWC_ERR_INVALID_ARG when the address
 * ranges intersect otherwise).  In place, every element is read and then
 * written by the same thread, so no row sees another row's gradient; the
 * logits are gone afterwards.  The same rule holds for every backward call;
 * in place the `_rows` calls need VWC_GRAD_SCATTER and distinct row ids, and
 * vwc_topk_kl_bwd needs rows on 16 bytes and k <= 256 (VWC_ERR_UNSUPPORTED
 * otherwise).
 */
vwc_status vwc_selected_logprob_bwd(const void *logits, vwc_dtype dt, int64_t n_rows,
                                    int64_t vocab, int64_t ld, const int32_t *targets,
                                    float temperature, const float *lse,
                                    const float *grad_logprob, void *grad_logits,
                                    vwc_dtype grad_dt, int64_t ld_grad, hipStream_t stream);

/*
 * Forward and backward in one call, for a loss whose per-row weight g_r is
 * known before the forward (a fixed-weight loss: token-mean cross-entropy, a
 * policy-gradient step whose importance ratio is still 1).  The results are
 * those of vwc_selected_logprob_fwd followed by vwc_selected_logprob_bwd with
 * the lse it wrote ([B] "Changes": the gradient (onehot - softmax) * g in the
 * logits' dtype; [C] "Design & Code Changes": from the logits and the fp32
 * logZ).  lse (float[n_rows]) is required; logprob and entropy are nullable.
 * The other arguments are as in those two calls, and grad_logits follows the
 * same in-place rule.  When a row fits on chip (at most 31744 16-byte vectors:
 * 253952 bf16 or 126976 fp32 columns) and the gradient has the logits' dtype
 * and 16-byte phase, one workgroup per row reads the row once, reduces it,
 * and writes the gradient from the held values (HBM traffic: one read and one
 * write of the rows instead of two reads and one write).  Otherwise the two
 * calls run in turn (`workspace` as for the forward).  Each row's lse and
 * entropy may differ from the separate forward's in the last bits (another
 * reduction order); every result meets the same bounds.
 */
vwc_status vwc_selected_logprob_fwd_bwd(const void *logits, vwc_dtype dt, int64_t n_rows,
                                        int64_t vocab, int64_t ld, const int32_t *targets,
                                        float temperature, const float *grad_logprob,
                                        float *logprob, float *lse, float *entropy,
                                        void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/*
 * The same over the row set row_idx[0..m) ([D] maintainer comment: compute on
 * the loss-mask rows only): grad_logprob, logprob, lse and entropy are compact
 * float[m]; targets are indexed by row id; layout places the gradient as in
 * vwc_selected_logprob_bwd_rows (VWC_GRAD_SCATTER: rows row_idx[i] of
 * [n_rows, ld_grad], other rows untouched, duplicate ids race; in place needs
 * scatter and distinct ids).  Row ids outside [0, n_rows) give NaN outputs and
 * no gradient.  A compact gradient keeps the on-chip path only when every row
 * has the same 16-byte phase as its gradient row (strides of whole 16-byte
 * multiples); otherwise the two `_rows` calls run.
 */
vwc_status vwc_selected_logprob_fwd_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                             int64_t vocab, int64_t ld, const int32_t *targets,
                                             const int32_t *row_idx, int64_t m,
                                             float temperature, const float *grad_logprob,
                                             float *logprob, float *lse, float *entropy,
                                             void *grad_logits, vwc_dtype grad_dt,
                                             int64_t ld_grad, vwc_grad_layout layout,
                                             void *workspace, size_t workspace_bytes,
                                             hipStream_t stream);

/*
 * Backward over the compact row set row_idx[0..m).  lse and grad_logprob are
 * float[m] (compact, as the `_rows` forward writes them).  layout selects
 * where gradient row i goes: VWC_GRAD_COMPACT -> row i of [m, ld_grad];
 * VWC_GRAD_SCATTER -> row row_idx[i] of [n_rows, ld_grad], other rows
 * untouched (the caller clears them: [D] maintainer comment, the results of
 * rows off the loss mask are left to the caller).  With VWC_GRAD_SCATTER,
 * duplicate row ids race.
 */
vwc_status vwc_selected_logprob_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                         int64_t vocab, int64_t ld, const int32_t *targets,
                                         const int32_t *row_idx, int64_t m, float temperature,
                                         const float *lse, const float *grad_logprob,
                                         void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                                         vwc_grad_layout layout, hipStream_t stream);

/*
 * Backward of a loss that uses both forward outputs of a row,
 *   L = sum_r g_r * logprob_r + h_r * entropy_r,
 * fused into the same single pass over the logits:
 *   grad[r, j] = (g_r ([j == t_r] - p_rj) - h_r p_rj (z_rj - lse_r + H_r)) / tau,
 * since dH/dz_j = -p_j (log p_j + H).  The pages' RL losses consume both the
 * log-probabilities and the entropy of the same logits ([D] "Bug
 * Description": get_log_probs_and_entropy; maintainer comment).
 *  lse, entropy   float[n_rows] from the forward at the same temperature
 *                 (entropy may be NULL when grad_entropy is NULL).
 *  grad_logprob   float[n_rows] (g) or NULL (g = 0; targets may then be NULL).
 *  grad_entropy   float[n_rows] (h) or NULL (h = 0: same result as
 *                 vwc_selected_logprob_bwd).  At least one must be non-NULL.
 * Rows with g == 0 and h == 0 are written as +0.0 without reading the logits.
 * Other arguments as vwc_selected_logprob_bwd.
 */
vwc_status vwc_logprob_entropy_bwd(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                                   int64_t ld, const int32_t *targets, float temperature,
                                   const float *lse, const float *entropy,
                                   const float *grad_logprob, const float *grad_entropy,
                                   void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                                   hipStream_t stream);

/* The same over the compact row set row_idx[0..m): lse, entropy,
   grad_logprob and grad_entropy are float[m]; layout as in
   vwc_selected_logprob_bwd_rows. */
vwc_status vwc_logprob_entropy_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                        int64_t vocab, int64_t ld, const int32_t *targets,
                                        const int32_t *row_idx, int64_t m, float temperature,
                                        const float *lse, const float *entropy,
                                        const float *grad_logprob, const float *grad_entropy,
                                        void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                                        vwc_grad_layout layout, hipStream_t stream);

/*
 * Forward and the logprob + entropy backward in one call, for a loss
 *   L = sum_r g_r * logprob_r + h_r * entropy_r
 * whose weights g (grad_logprob, nullable: 0) and h (grad_entropy, required)
 * are known before the forward ("[Bug] Training/log-prob forward materializes
 * full-vocab fp32 logits ..." section "Bug Description": RL losses that use the
 * log-probabilities and the entropy of the same logits, e.g. an entropy bonus
 * with a token-mean weight).  The results are those of vwc_selected_logprob_fwd
 * with the entropy, followed by vwc_logprob_entropy_bwd with the lse and entropy
 * it wrote: lse and entropy (float[n_rows]) are required outputs, logprob is
 * nullable; targets may be NULL when neither grad_logprob nor logprob is given.
 * When a row fits on chip (as for vwc_selected_logprob_fwd_bwd) one workgroup
 * per row reads it once and writes its gradient from the held values;
 * otherwise the two calls run in turn.  lse, entropy and logprob may differ from
 * the separate forward's in the last bits (another reduction order); the
 * gradient is the separate backward's from these outputs, bit for bit.  Rows
 * with g == 0 and h == 0 get +0.0.  In place (grad_logits == logits) as for
 * the backward.  Other arguments and errors as vwc_selected_logprob_fwd_bwd.
 */
vwc_status vwc_logprob_entropy_fwd_bwd(const void *logits, vwc_dtype dt, int64_t n_rows,
                                       int64_t vocab, int64_t ld, const int32_t *targets,
                                       float temperature, const float *grad_logprob,
                                       const float *grad_entropy, float *logprob, float *lse,
                                       float *entropy, void *grad_logits, vwc_dtype grad_dt,
                                       int64_t ld_grad, void *workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* The same over the row set row_idx[0..m): grad_logprob, grad_entropy and the
   outputs are float[m] (compact); layout, bad row ids and the in-place rule as
   for vwc_selected_logprob_fwd_bwd_rows. */
vwc_status vwc_logprob_entropy_fwd_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                            int64_t vocab, int64_t ld, const int32_t *targets,
                                            const int32_t *row_idx, int64_t m, float temperature,
                                            const float *grad_logprob, const float *grad_entropy,
                                            float *logprob, float *lse, float *entropy,
                                            void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                                            vwc_grad_layout layout, void *workspace,
                                            size_t workspace_bytes, hipStream_t stream);

typedef enum vwc_kl_mode {
    VWC_KL_TRUNCATED = 0, /* sum over the teacher top-k, clamped at 0 */
    VWC_KL_TAIL = 1,      /* K+1 categories: the top-k plus one aggregate tail */
    VWC_KL_MODE_INT_RANGE_LO_ = -0x7fffffff - 1, /* every int is a value; others are refused */
    VWC_KL_MODE_INT_RANGE_HI_ = 0x7fffffff
} vwc_kl_mode;

/*
 * Top-k forward KL of a teacher payload against the student softmax, from the
 * verl top-k KL pages ("[megatron] feat: add memory-efficient chunked top-k KL
 * computation"; its commit text of the tail-aware top-k KL change, "What does
 * this PR do?" and "Design & Code Changes").  Per row r, T_r =
 * topk_idx[r*k .. r*k+k) (distinct student columns, int32), teacher
 * log-probs a_n = teacher_logprob[r*k + n] (float), p_n = exp(a_n),
 * q_j = softmax(x_r / tau)_j, P = sum p_n, Q = sum q_{T_n},
 * S = sum p_n (a_n - log q_{T_n}):
 *   VWC_KL_TRUNCATED: loss = max(0, S)
 *   VWC_KL_TAIL:      loss = S + p_tail (log p_tail - log max(1 - Q, eps)),
 *                     p_tail = max(0, 1 - P), 0 log 0 = 0
 * Outputs float[n_rows]: loss, student_mass (Q), teacher_mass (P), topk_sum
 * (S, before any clamp) and lse; each nullable except lse and the ones the
 * backward needs (it reads lse, student_mass, teacher_mass, topk_sum).
 * tail_mass_eps must lie in (0, 1) for VWC_KL_TAIL (the page's default is
 * 1e-6).  A column id outside [0, vocab) gives NaN outputs for its row.
 * workspace: vwc_workspace_bytes(n_rows, vocab, dt).
 */
vwc_status vwc_topk_kl_fwd(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                           int64_t ld, const int32_t *topk_idx, const float *teacher_logprob,
                           int32_t k, vwc_kl_mode mode, float tail_mass_eps, float temperature,
                           float *loss, float *student_mass, float *teacher_mass, float *topk_sum,
                           float *lse, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Top-k KL over the row set row_idx[0..m) (the loss-mask rows, as for the
 * other `_rows` calls).  topk_idx and teacher_logprob are [m, k] (one payload
 * per listed row, in list order); the outputs are float[m].  A row id outside
 * [0, n_rows) gives NaN outputs for its entry.  Each listed row gets the bits
 * of the dense call's row.  workspace: vwc_workspace_bytes(m, vocab, dt).
 */
vwc_status vwc_topk_kl_fwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                                int64_t ld, const int32_t *row_idx, int64_t m,
                                const int32_t *topk_idx, const float *teacher_logprob, int32_t k,
                                vwc_kl_mode mode, float tail_mass_eps, float temperature,
                                float *loss, float *student_mass, float *teacher_mass,
                                float *topk_sum, float *lse, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Gradient of sum_r g_r loss_r with respect to the student logits, in one
 * streaming pass that also writes the k payload columns (rows on 16 bytes and
 * k <= 256; otherwise a second launch rewrites those columns) (the page's
 * analytic form: q_j - p_j inside the top-k and q_j (P - Q)/(1 - Q) outside
 * for the tail objective; q_j P - p_j [j in T] for the truncated one, and 0
 * for a clamped truncated row or while the eps guard is active on the tail
 * term's q_tail; all divided by tau).  lse, student_mass, teacher_mass and
 * topk_sum come from vwc_topk_kl_fwd; grad_loss is float[n_rows].  Rows with
 * g == 0 or a clamped truncated loss are written as +0.0 without reading the
 * logits.  Other arguments as vwc_selected_logprob_bwd.
 */
vwc_status vwc_topk_kl_bwd(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                           int64_t ld, const int32_t *topk_idx, const float *teacher_logprob,
                           int32_t k, vwc_kl_mode mode, float tail_mass_eps, float temperature,
                           const float *lse, const float *student_mass, const float *teacher_mass,
                           const float *topk_sum, const float *grad_loss, void *grad_logits,
                           vwc_dtype grad_dt, int64_t ld_grad, hipStream_t stream);

/*
 * Backward over the row set row_idx[0..m): the payload, lse, student_mass,
 * teacher_mass, topk_sum and grad_loss are the `_rows` forward's, indexed by
 * list position.  layout as for vwc_selected_logprob_bwd_rows: gradient row i
 * at row i of [m, ld_grad] (VWC_GRAD_COMPACT) or at row row_idx[i] of
 * [n_rows, ld_grad] (VWC_GRAD_SCATTER, other rows untouched; duplicate ids
 * race).  Rows with an id outside [0, n_rows) are not written.
 */
vwc_status vwc_topk_kl_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                                int64_t ld, const int32_t *row_idx, int64_t m,
                                const int32_t *topk_idx, const float *teacher_logprob, int32_t k,
                                vwc_kl_mode mode, float tail_mass_eps, float temperature,
                                const float *lse, const float *student_mass,
                                const float *teacher_mass, const float *topk_sum,
                                const float *grad_loss, void *grad_logits, vwc_dtype grad_dt,
                                int64_t ld_grad, vwc_grad_layout layout, hipStream_t stream);

/*
 * Top-k KL forward and backward in one call, for a distillation loss whose
 * per-row weight g_r (grad_loss, float[n_rows]) is known before the forward,
 * e.g. a token mean.  The results are those of vwc_topk_kl_fwd followed by
 * vwc_topk_kl_bwd with the lse, student_mass, teacher_mass and topk_sum it
 * wrote (the chunked top-k KL of "[megatron] feat: add memory-efficient
 * chunked top-k KL computation": keep the logits and the per-row logZ,
 * recompute the student softmax in the backward).  lse, student_mass,
 * teacher_mass and topk_sum (float[n_rows]) are required, loss is nullable;
 * the payload, mode, tail_mass_eps and the in-place rule are as in those two
 * calls.  When a row fits on chip (as for vwc_selected_logprob_fwd_bwd), the
 * gradient has the logits' dtype and 16-byte phase, and k <= 256, one
 * workgroup per row reads the row once, reduces it, sums the payload, and
 * writes the gradient (payload columns included) from the held values: one
 * read and one write of the rows instead of two reads and one write.
 * Otherwise the two calls run in turn (`workspace` as for vwc_topk_kl_fwd).
 * lse, student_mass, teacher_mass, topk_sum and loss may differ from the
 * separate forward's in the last bits (another reduction order); every
 * result meets the same bounds, and the gradient is the separate backward's
 * from these outputs.
 */
vwc_status vwc_topk_kl_fwd_bwd(const void *logits, vwc_dtype dt, int64_t n_rows, int64_t vocab,
                               int64_t ld, const int32_t *topk_idx, const float *teacher_logprob,
                               int32_t k, vwc_kl_mode mode, float tail_mass_eps,
                               float temperature, const float *grad_loss, float *loss,
                               float *student_mass, float *teacher_mass, float *topk_sum,
                               float *lse, void *grad_logits, vwc_dtype grad_dt, int64_t ld_grad,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The same over the row set row_idx[0..m): the payload, grad_loss and the
 * outputs are indexed by list position (as for vwc_topk_kl_fwd_rows), layout
 * as for vwc_topk_kl_bwd_rows (compact: gradient row i is list entry i;
 * scatter: row id r of a [n_rows, ld_grad] buffer, other rows untouched,
 * duplicate ids race).  Each listed row gets the dense call's bits.  A row id
 * outside [0, n_rows) gives NaN outputs and leaves its gradient row unwritten.
 * In place (grad_logits == logits) needs VWC_GRAD_SCATTER, else
 * VWC_ERR_INVALID_ARG before anything runs, and distinct ids (not checked).
 */
vwc_status vwc_topk_kl_fwd_bwd_rows(const void *logits, vwc_dtype dt, int64_t n_rows,
                                    int64_t vocab, int64_t ld, const int32_t *row_idx, int64_t m,
                                    const int32_t *topk_idx, const float *teacher_logprob,
                                    int32_t k, vwc_kl_mode mode, float tail_mass_eps,
                                    float temperature, const float *grad_loss, float *loss,
                                    float *student_mass, float *teacher_mass, float *topk_sum,
                                    float *lse, void *grad_logits, vwc_dtype grad_dt,
                                    int64_t ld_grad, vwc_grad_layout layout, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/*
 * Partial of one vocabulary slice ([E] "Implementation", steps 1-3 in one
 * pass).  logits_slice points at global column v_start of row 0; the slice is
 * columns [0, v_local) of each row, rows ld elements apart.  targets hold
 * GLOBAL column ids (int32[n_rows], nullable: then every t is -infinity);
 * the slice owns t when v_start <= t < v_start + v_local.  row_idx is
 * nullable (then m must equal n_rows).  out is vwc_partial[m].
 * workspace: vwc_workspace_bytes(m, v_local, dt) bytes.
 */
vwc_status vwc_vocab_partial(const void *logits_slice, vwc_dtype dt, int64_t n_rows,
                             int64_t v_local, int64_t ld, int64_t v_start,
                             const int32_t *targets, const int32_t *row_idx, int64_t m,
                             float temperature, vwc_partial *out, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Merge k slice partials per row ([E] "Implementation", step 4; the merge
 * formulas are in the vwc_partial comment).  parts is vwc_partial[k][rows]
 * (slice-major: slice q's partial of row i at parts[q * rows + i]), merged in
 * slice order.  Outputs float[rows], each nullable (at least one non-null).
 */
vwc_status vwc_partial_combine(const vwc_partial *parts, int32_t k, int64_t rows,
                               float temperature, float *logprob, float *lse, float *entropy,
                               hipStream_t stream);

/*
 * Row-set selection ([D] maintainer comment: keep the loss-mask rows).
 * Writes the ascending ids of the nonzero entries of mask[0..n) to
 * row_idx[0..count) and the count to *count (device int32).  row_idx must
 * hold n entries.  n <= INT32_MAX.
 */
vwc_status vwc_mask_to_index(const uint8_t *mask, int64_t n, int32_t *row_idx, int32_t *count,
                             hipStream_t stream);

/*
 * The same for long masks (the packed and context-parallel sequences of [B]
 * "Verification" and [D] "Bug Description" run to 64k-160k tokens and more),
 * spread over the whole GPU: the mask is cut into tiles of 4096 entries, each
 * tile's nonzeros are counted, one workgroup turns the counts into offsets, and
 * every tile writes its ids from its offset; the ids equal the one-workgroup
 * call's.  Masks of at most 65536 entries take the one-workgroup scan (one
 * launch) and need no workspace; longer ones need
 * vwc_mask_to_index_workspace_bytes(n) bytes (4 per tile), 4-byte aligned,
 * whose contents on entry do not matter.  Other arguments as
 * vwc_mask_to_index.
 */
size_t vwc_mask_to_index_workspace_bytes(int64_t n);

vwc_status vwc_mask_to_index_ws(const uint8_t *mask, int64_t n, int32_t *row_idx, int32_t *count,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Fused LM head ([D] maintainer comment: keep the loss-mask rows of the final
 * hidden state before the vocabulary projection and compute log-prob and
 * entropy on those rows only; [A] "Alternatives considered": a fused
 * LM-head / cross-entropy kernel; the merge of [E] "Implementation" joins the
 * vocabulary segments).  For output i with row r = row_idx ? row_idx[i] : i:
 *   x_j = sum_{k<d} hidden[r, k] * weight[j, k]      (bf16 x bf16, fp32 sum)
 * and then lse / logprob / entropy of x as above.  The logits exist only in
 * registers: nothing of size rows x vocab is ever written.
 *  hidden   bf16 [n_rows, ldh], the final hidden states (after the last norm).
 *  weight   bf16 [vocab, ldw], the output layer, one row per vocabulary entry.
 *  d        the hidden size: columns [0, d) of both are used; d <= ldh, ldw.
 *  targets  int32[n_rows] by row id (required when logprob is requested).
 *  row_idx  int32[m] kept row ids (nullable: then m must equal n_rows).
 *  logprob, lse, entropy  float[m], compact, each nullable (one required).
 *  workspace  16-byte aligned, at least vwc_lmhead_workspace_bytes(m, vocab, d)
 *           bytes with row_idx (16 bytes per row per segment of 1024
 *           vocabulary entries, then the m kept rows compacted, m * d * 2
 *           bytes rounded up to 16); without row_idx the partials alone.
 * Layout limits (VWC_ERR_UNSUPPORTED otherwise): hidden and weight 16-byte
 * aligned, d, ldh and ldw multiples of 8, ldh and ldw below 2^22, m at most
 * INT32_MAX (and m * d / 8 below 2^39 with row_idx).  m > 0 needs
 * n_rows >= 1.  A row id
 * outside [0, n_rows) gives NaN outputs; a target outside [0, vocab) gives a
 * NaN logprob.  The reduction order of a row depends only on vocab and d,
 * so a row gives bit-identical results whatever row set it is computed in.
 */
size_t vwc_lmhead_workspace_bytes(int64_t rows, int64_t vocab, int64_t d);

vwc_status vwc_lmhead_logprob_fwd(const void *hidden, int64_t n_rows, int64_t ldh,
                                  const void *weight, int64_t vocab, int64_t ldw, int64_t d,
                                  const int32_t *targets, const int32_t *row_idx, int64_t m,
                                  float temperature, float *logprob, float *lse, float *entropy,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code (host pointer, never NULL). */
const char *vwc_status_string(vwc_status status);

/* Detail of the last failure on the calling thread ("" if none; host pointer,
   valid until the next call on this thread). */
const char *vwc_last_error(void);

/* VWC_ABI_VERSION of the loaded library. */
int vwc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VWC_H */
