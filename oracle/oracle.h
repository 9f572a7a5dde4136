/*
 * oracle.h -- plain fp64 CPU oracle for selected-token log-probabilities,
 * entropy and the logit gradient.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code; only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or helper with the
 * HIP library: it has its own bf16 decode and its own bf16 rounding.
 *
 * Every function works in double precision on the definition itself:
 *   z_j   = x_j / tau                               (tau widened to double)
 *   LSE   = M + log(sum_j exp(z_j - M)),  M = max_j z_j
 *   lp    = z_t - LSE                               (log_softmax(z)[t])
 *   H     = -sum_j p_j * log p_j,   p_j = exp(z_j - LSE)
 *   grad_j = g * ([j == t] - p_j) / tau             (+0.0 when g == 0)
 *
 * Sources (web pages, cited by title and section):
 *  - "[RL][Performance] Avoid full-vocabulary TP gather for selected-token
 *    logprobs", section "Proposed solution": the selected log-probability equals
 *    minus the token cross entropy (label smoothing 0); section "Prototype
 *    correctness": masked positions receive exactly zero gradient.
 *  - "fix: chunk target logprobs without tensor parallelism (long-context OOM)",
 *    section "Changes": the forward is a float32 per-chunk logsumexp plus a
 *    gather of the target logit; the backward recomputes the softmax and writes
 *    (onehot - softmax) * grad_output; a non-positive chunk size is an error.
 *    Section "Behavior change and trade-off": chunking only reassociates the
 *    reduction.
 *  - "[megatron] feat: add memory-efficient chunked top-k KL computation",
 *    section "Design & Code Changes": the backward keeps the logits and a
 *    per-token fp32 logZ and recomputes probabilities from them.
 *  - "feat: Reduce reference model memory with with parallel logprob
 *    computation", section "Implementation": a vocabulary-sharded
 *    log-softmax merges per-shard max, per-shard sum of exp(x - max) and the
 *    target logit held only by the shard that owns it.
 *  - "[Bug] Training/log-prob forward materializes full-vocab fp32 logits over
 *    the entire packed sequence ...", the maintainer comment: log-probability
 *    and entropy are computed on the compact set of loss-mask rows only.
 *
 * Return codes: 0 ok, -1 invalid argument, -2 target out of range,
 * -3 row index out of range, -4 out of memory.
 */
#ifndef VWC_ORACLE_H
#define VWC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_BF16 0 /* logits are raw bf16 bit patterns (uint16) */
#define ORACLE_FP32 1 /* logits are IEEE binary32 */
#define ORACLE_FP64 2 /* logits are IEEE binary64 (the LM-head oracle's own logits) */

/*
 * Forward over a row set.  logits is a host buffer [n_rows, ld] of `dtype`.
 * rows == NULL selects rows 0..m-1 (m must equal n_rows); otherwise rows[i]
 * (0 <= rows[i] < n_rows) is the row of output i.  targets is indexed by row id
 * (length n_rows) and may be NULL when logprob is NULL.  Rows are visited in
 * chunks of row_chunk rows (row_chunk <= 0 is an error).  Each output pointer
 * ([m] doubles) may be NULL.
 */
int oracle_forward(const void *logits, int dtype, int64_t n_rows, int64_t vocab,
                   int64_t ld, const int32_t *targets, const int32_t *rows,
                   int64_t m, double tau, int64_t row_chunk, double *logprob,
                   double *lse, double *entropy);

/*
 * Backward over a row set: grad[i * vocab + j] for output i and column j, the
 * gradient of logprob_i with respect to the logits, scaled by grad_out[i].
 * grad_out is float (the dtype the caller's loss hands over), length m.
 */
int oracle_backward(const void *logits, int dtype, int64_t n_rows,
                    int64_t vocab, int64_t ld, const int32_t *targets,
                    const int32_t *rows, int64_t m, double tau,
                    const float *grad_out, double *grad);

/*
 * Backward of a loss that uses both outputs of a row:
 *   L = sum_i g_i * logprob_i + h_i * entropy_i
 * grad[i * vocab + j] = dL/dx_j
 *                     = (g_i ([j == t] - p_j) - h_i p_j (z_j - LSE + H)) / tau,
 * since dH/dz_j = -p_j (log p_j + H) and log p_j = z_j - LSE.  grad_logprob
 * and grad_entropy are float[m] and each may be NULL (treated as 0); targets
 * may be NULL when grad_logprob is.  Rows where both are 0 get +0.0.
 */
int oracle_backward_entropy(const void *logits, int dtype, int64_t n_rows,
                            int64_t vocab, int64_t ld, const int32_t *targets,
                            const int32_t *rows, int64_t m, double tau,
                            const float *grad_logprob,
                            const float *grad_entropy, double *grad);

/*
 * Top-k forward KL of a teacher payload against the student softmax
 * ("[megatron] feat: add memory-efficient chunked top-k KL computation",
 * commit text of the tail-aware top-k KL change, "What does this PR do?").
 * Per row i: T = topk_idx[i*k .. i*k+k) (distinct student columns), teacher
 * log-probs a_n = teacher_logprob[i*k + n], p_n = exp(a_n), student
 * q_j = exp(z_j - LSE).  P = sum_n p_n, Q = sum_n q_{T_n},
 *   truncated:  L = max(0, sum_n p_n (a_n - log q_{T_n}))
 *   tail:       L = sum_n p_n (a_n - log q_{T_n})
 *                   + (1 - P) (log(1 - P) - log(max(1 - Q, eps)))
 * with 0 log 0 = 0, and 1 - P read as max(0, 1 - P) (a payload whose fp32
 * log-probs sum above 1 has an empty tail).  Outputs (each nullable) loss[i], student_mass[i] = Q,
 * teacher_mass[i] = P.  mode: 0 truncated, 1 tail.
 */
int oracle_topk_kl_forward(const void *logits, int dtype, int64_t n_rows,
                           int64_t vocab, int64_t ld, const int32_t *topk_idx,
                           const float *teacher_logprob, int64_t k, int mode,
                           double tail_eps, double tau, double *loss,
                           double *student_mass, double *teacher_mass);

/*
 * Gradient of sum_i g_i L_i with respect to the student logits, from the
 * definition: L as a function of log q_{T_n} and, in tail mode, of
 * log max(1 - Q, eps) (whose derivative is 0 while the guard is active), with
 * d log q_i / dz_j = [i == j] - q_j and dQ/dz_j = q_j [j in T] - q_j Q; then
 * d/dx = d/dz / tau.  A truncated row whose loss is clamped gets 0.
 * grad is [n_rows][vocab]; grad_loss is float[n_rows].
 */
int oracle_topk_kl_backward(const void *logits, int dtype, int64_t n_rows,
                            int64_t vocab, int64_t ld, const int32_t *topk_idx,
                            const float *teacher_logprob, int64_t k, int mode,
                            double tail_eps, double tau, const float *grad_loss,
                            double *grad);

/*
 * Partial of one vocabulary slice: the slice's columns are
 * [v_start, v_start + v_local) of the full vocabulary; logits_slice points at
 * column v_start of row 0 and rows are ld elements apart.  Per output i:
 *   pm[i] = max_j z_j over the slice
 *   ps[i] = sum_j exp(z_j - pm[i])
 *   pw[i] = sum_j exp(z_j - pm[i]) * (z_j - pm[i])
 *   pt[i] = z_t if v_start <= t < v_start + v_local, else -infinity
 * targets are global column ids and may be NULL (then pt is not written).
 */
int oracle_slice_partial(const void *logits_slice, int dtype, int64_t n_rows,
                         int64_t v_local, int64_t ld, int64_t v_start,
                         const int32_t *targets, const int32_t *rows, int64_t m,
                         double tau, double *pm, double *ps, double *pw,
                         double *pt);

/*
 * Merge k slice partials per row; partial arrays are laid out [k][m].
 * Any output pointer may be NULL.
 */
int oracle_combine(int64_t k, int64_t m, const double *pm, const double *ps,
                   const double *pw, const double *pt, double *logprob,
                   double *lse, double *entropy);

/*
 * Forward computed through vocabulary chunks of vchunk columns (the last one
 * ragged), each reduced to a slice partial and merged with oracle_combine.
 */
int oracle_forward_vchunk(const void *logits, int dtype, int64_t n_rows,
                          int64_t vocab, int64_t ld, const int32_t *targets,
                          const int32_t *rows, int64_t m, double tau,
                          int64_t vchunk, double *logprob, double *lse,
                          double *entropy);

/*
 * LM-head logits of a row set ("[Bug] Training/log-prob forward materializes
 * full-vocab fp32 logits ...", maintainer comment: keep the loss-mask rows of
 * the final hidden state before the vocabulary projection; "[RL][Performance]
 * Avoid full-vocabulary TP gather ...", "Alternatives considered": a fused
 * LM-head / cross-entropy kernel).  hidden is bf16 bits [n_rows, ldh], weight
 * is bf16 bits [vocab, ldw] (one row per vocabulary entry, as the output
 * layer stores it).  For output i with row r = rows ? rows[i] : i:
 *   x[i * vocab + j] = sum_{k=0}^{d-1} hidden[r, k] * weight[j, k]
 * summed in ascending k in double (every bf16 product is exact in double).
 * abs_sum (nullable) gets sum_k |hidden[r, k] * weight[j, k]| at the same
 * index, the scale of the rounding error of any finite-precision evaluation.
 */
int oracle_lmhead_logits(const uint16_t *hidden, int64_t n_rows, int64_t ldh,
                         const uint16_t *weight, int64_t vocab, int64_t ldw,
                         int64_t d, const int32_t *rows, int64_t m, double *x,
                         double *abs_sum);

/*
 * Forward of the fused LM head: the logits above followed by oracle_forward's
 * definitions (z_j = x_j / tau; lse, logprob = z_t - lse, entropy), computed
 * row_chunk rows at a time.  targets is indexed by row id (length n_rows) and
 * may be NULL when logprob is NULL.  err_scale (nullable, [m]) gets
 * (A_t + max_j A_j) / tau with A_j the abs_sum of column j and t the target
 * (max_j A_j / tau alone when targets is NULL): the bound on how far an
 * evaluation with logit errors |dx_j| <= eps * A_j can move logprob.
 */
int oracle_lmhead_forward(const uint16_t *hidden, int64_t n_rows, int64_t ldh,
                          const uint16_t *weight, int64_t vocab, int64_t ldw,
                          int64_t d, const int32_t *targets, const int32_t *rows,
                          int64_t m, double tau, int64_t row_chunk,
                          double *logprob, double *lse, double *entropy,
                          double *err_scale);

/* Round a double to the nearest bf16 (ties to even); returns the bit pattern. */
uint16_t oracle_bf16_rne(double v);

/* Round n doubles to bf16 bit patterns. */
void oracle_bf16_rne_array(const double *v, uint16_t *out, int64_t n);

/* Number of OpenMP threads the oracle runs on. */
int oracle_num_threads(void);

/* Run later calls on n threads (n > 0; ignored otherwise). */
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif

#endif /* VWC_ORACLE_H */
