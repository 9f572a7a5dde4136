/*
 * oracle.c -- plain fp64 CPU oracle (TEST INFRASTRUCTURE ONLY; see oracle.h).
 *
 * Written for a reader who checks it against the definition by eye: every row
 * is handled on its own in a few sequential passes over its columns, in double
 * precision, with no blocking, fusion or reordering beyond the definition.
 * OpenMP only distributes whole rows over host threads.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the upper half of an IEEE binary32: widen by shifting 16 bits up. */
static double decode_bf16(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Logit x[row, col] widened to double. */
static double logit_at(const void *logits, int dtype, int64_t ld, int64_t row,
                       int64_t col) {
    int64_t off = row * ld + col;
    if (dtype == ORACLE_BF16) return decode_bf16(((const uint16_t *)logits)[off]);
    if (dtype == ORACLE_FP64) return ((const double *)logits)[off];
    return (double)((const float *)logits)[off];
}

static int dtype_ok(int dtype) {
    return dtype == ORACLE_BF16 || dtype == ORACLE_FP32 || dtype == ORACLE_FP64;
}

static int tau_ok(double tau) { return isfinite(tau) && tau > 0.0; }

/* Row id of output i. */
static int64_t row_of(const int32_t *rows, int64_t i) {
    return rows ? (int64_t)rows[i] : i;
}

static int check_rows(const int32_t *rows, int64_t m, int64_t n_rows) {
    if (!rows) return m == n_rows ? 0 : -1;
    for (int64_t i = 0; i < m; ++i)
        if (rows[i] < 0 || (int64_t)rows[i] >= n_rows) return -3;
    return 0;
}

static int check_targets(const int32_t *targets, const int32_t *rows, int64_t m,
                         int64_t vocab) {
    for (int64_t i = 0; i < m; ++i) {
        int64_t t = targets[row_of(rows, i)];
        if (t < 0 || t >= vocab) return -2;
    }
    return 0;
}

/*
 * Log-sum-exp of z_j = x[row, c0 + j] / tau over j in [0, n):
 *   M = max z_j;  S = sum exp(z_j - M);  LSE = M + log S.
 * Two passes, columns in ascending order.
 */
/* exp(z - M), with exp(-inf) = 0 even when M is -inf too (a row or slice of
   -inf logits: masked vocabulary entries have probability 0). */
static double exp_shifted(double z, double M) {
    return z == -INFINITY ? 0.0 : exp(z - M);
}

/* p * a for a term of probability p: 0 when p is 0, whatever a is (the limit
   0 log 0 = 0 of -p log p; a is -inf there).  NaN p stays NaN. */
static double p_times(double p, double a) { return p == 0.0 ? 0.0 : p * a; }

static void row_max_sum(const void *logits, int dtype, int64_t ld, int64_t row,
                        int64_t c0, int64_t n, double tau, double *M_out,
                        double *S_out) {
    double M = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double z = logit_at(logits, dtype, ld, row, c0 + j) / tau;
        if (z > M) M = z;
    }
    double S = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double z = logit_at(logits, dtype, ld, row, c0 + j) / tau;
        S += exp_shifted(z, M);
    }
    *M_out = M;
    *S_out = S;
}

/* Entropy -sum_j p_j log p_j with p_j = exp(z_j - LSE) and log p_j = z_j - LSE. */
static double row_entropy(const void *logits, int dtype, int64_t ld,
                          int64_t row, int64_t vocab, double tau, double LSE) {
    double H = 0.0;
    for (int64_t j = 0; j < vocab; ++j) {
        double z = logit_at(logits, dtype, ld, row, j) / tau;
        double p = exp_shifted(z, LSE);
        H -= p_times(p, z - LSE);
    }
    return H;
}

int oracle_forward(const void *logits, int dtype, int64_t n_rows, int64_t vocab,
                   int64_t ld, const int32_t *targets, const int32_t *rows,
                   int64_t m, double tau, int64_t row_chunk, double *logprob,
                   double *lse, double *entropy) {
    /* Non-positive chunk sizes are rejected, as in the chunked local kernel
       described in "fix: chunk target logprobs without tensor parallelism",
       section "Changes". */
    if (row_chunk <= 0) return -1;
    if (!logits || !dtype_ok(dtype) || n_rows < 0 || m < 0 || vocab <= 0 ||
        ld < vocab || !tau_ok(tau))
        return -1;
    if (logprob && !targets) return -1;
    int rc = check_rows(rows, m, n_rows);
    if (rc) return rc;
    if (logprob && (rc = check_targets(targets, rows, m, vocab))) return rc;

    for (int64_t c0 = 0; c0 < m; c0 += row_chunk) {
        int64_t c1 = c0 + row_chunk < m ? c0 + row_chunk : m;
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t i = c0; i < c1; ++i) {
            int64_t r = row_of(rows, i);
            double M, S;
            row_max_sum(logits, dtype, ld, r, 0, vocab, tau, &M, &S);
            double LSE = M + log(S);
            if (lse) lse[i] = LSE;
            if (logprob) {
                /* log_softmax(z)[t] = z_t - LSE, which is -cross_entropy(z, t). */
                double zt = logit_at(logits, dtype, ld, r, targets[r]) / tau;
                logprob[i] = zt - LSE;
            }
            if (entropy)
                entropy[i] = row_entropy(logits, dtype, ld, r, vocab, tau, LSE);
        }
    }
    return 0;
}

int oracle_backward(const void *logits, int dtype, int64_t n_rows,
                    int64_t vocab, int64_t ld, const int32_t *targets,
                    const int32_t *rows, int64_t m, double tau,
                    const float *grad_out, double *grad) {
    if (!logits || !dtype_ok(dtype) || n_rows < 0 || m < 0 || vocab <= 0 ||
        ld < vocab || !tau_ok(tau) || !targets || !grad_out || (m && !grad))
        return -1;
    int rc = check_rows(rows, m, n_rows);
    if (rc) return rc;
    if ((rc = check_targets(targets, rows, m, vocab))) return rc;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        int64_t r = row_of(rows, i);
        double *gi = grad + i * vocab;
        double g = (double)grad_out[i];
        if (g == 0.0) {
            /* Rows without loss get an exact +0.0 gradient ("Avoid
               full-vocabulary TP gather ...", section "Prototype correctness"). */
            for (int64_t j = 0; j < vocab; ++j) gi[j] = 0.0;
            continue;
        }
        /* The logZ is recomputed here from the logits; nothing comes from the
           forward of the code under test. */
        double M, S;
        row_max_sum(logits, dtype, ld, r, 0, vocab, tau, &M, &S);
        double LSE = M + log(S);
        int64_t t = targets[r];
        for (int64_t j = 0; j < vocab; ++j) {
            double z = logit_at(logits, dtype, ld, r, j) / tau;
            double p = exp(z - LSE);
            double onehot = (j == t) ? 1.0 : 0.0;
            /* d(z_t - LSE)/dx_j = (onehot_j - p_j) / tau, times the incoming g. */
            gi[j] = g * (onehot - p) / tau;
        }
    }
    return 0;
}

int oracle_backward_entropy(const void *logits, int dtype, int64_t n_rows,
                            int64_t vocab, int64_t ld, const int32_t *targets,
                            const int32_t *rows, int64_t m, double tau,
                            const float *grad_logprob,
                            const float *grad_entropy, double *grad) {
    if (!logits || !dtype_ok(dtype) || n_rows < 0 || m < 0 || vocab <= 0 ||
        ld < vocab || !tau_ok(tau) || (grad_logprob && !targets) ||
        (m && !grad))
        return -1;
    int rc = check_rows(rows, m, n_rows);
    if (rc) return rc;
    if (grad_logprob && (rc = check_targets(targets, rows, m, vocab))) return rc;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        int64_t r = row_of(rows, i);
        double *gi = grad + i * vocab;
        double g = grad_logprob ? (double)grad_logprob[i] : 0.0;
        double h = grad_entropy ? (double)grad_entropy[i] : 0.0;
        if (g == 0.0 && h == 0.0) {
            for (int64_t j = 0; j < vocab; ++j) gi[j] = 0.0;
            continue;
        }
        double M, S;
        row_max_sum(logits, dtype, ld, r, 0, vocab, tau, &M, &S);
        double LSE = M + log(S);
        double H = row_entropy(logits, dtype, ld, r, vocab, tau, LSE);
        int64_t t = grad_logprob ? targets[r] : -1;
        for (int64_t j = 0; j < vocab; ++j) {
            double z = logit_at(logits, dtype, ld, r, j) / tau;
            double p = exp_shifted(z, LSE);
            double onehot = (j == t) ? 1.0 : 0.0;
            /* d logprob / dz_j = onehot_j - p_j;  dH / dz_j = -p_j (z_j - LSE + H). */
            gi[j] = (g * (onehot - p) - h * p_times(p, z - LSE + H)) / tau;
        }
    }
    return 0;
}

/* 0 log 0 = 0 */
static double xlogx_term(double a, double log_a) { return a == 0.0 ? 0.0 : a * log_a; }

static int topk_args_ok(const void *logits, int dtype, int64_t n_rows, int64_t vocab,
                        int64_t ld, const int32_t *topk_idx,
                        const float *teacher_logprob, int64_t k, int mode,
                        double tail_eps, double tau) {
    if (!logits || !dtype_ok(dtype) || n_rows < 0 || vocab <= 0 || ld < vocab ||
        !tau_ok(tau) || k <= 0 || k > vocab || (mode != 0 && mode != 1))
        return -1;
    if (n_rows > 0 && (!topk_idx || !teacher_logprob)) return -1;
    if (mode == 1 && !(tail_eps > 0.0 && tail_eps < 1.0)) return -1;
    for (int64_t i = 0; i < n_rows * k; ++i)
        if (topk_idx[i] < 0 || (int64_t)topk_idx[i] >= vocab) return -2;
    return 0;
}

/* Per-row pieces of the top-k KL: LSE, P, Q and the loss. */
static void topk_row(const void *logits, int dtype, int64_t ld, int64_t i,
                     int64_t vocab, const int32_t *idx, const float *tlp,
                     int64_t k, int mode, double tail_eps, double tau,
                     double *LSE_out, double *P_out, double *Q_out,
                     double *L_out) {
    double M, S;
    row_max_sum(logits, dtype, ld, i, 0, vocab, tau, &M, &S);
    double LSE = M + log(S);
    double P = 0.0, Q = 0.0, L = 0.0;
    for (int64_t n = 0; n < k; ++n) {
        double a = (double)tlp[n];
        double p = exp(a);
        double logq = logit_at(logits, dtype, ld, i, idx[n]) / tau - LSE;
        P += p;
        Q += exp(logq);
        L += p * (a - logq);
    }
    if (mode == 0) {
        if (L < 0.0) L = 0.0; /* clamp_min(0) of the truncated objective */
    } else {
        /* A payload whose fp32 log-probs sum above 1 has an empty tail. */
        double pt = P < 1.0 ? 1.0 - P : 0.0;
        double qt = 1.0 - Q;
        if (qt < tail_eps) qt = tail_eps;
        L += xlogx_term(pt, log(pt)) - (pt == 0.0 ? 0.0 : pt * log(qt));
    }
    *LSE_out = LSE;
    *P_out = P;
    *Q_out = Q;
    *L_out = L;
}

int oracle_topk_kl_forward(const void *logits, int dtype, int64_t n_rows,
                           int64_t vocab, int64_t ld, const int32_t *topk_idx,
                           const float *teacher_logprob, int64_t k, int mode,
                           double tail_eps, double tau, double *loss,
                           double *student_mass, double *teacher_mass) {
    int rc = topk_args_ok(logits, dtype, n_rows, vocab, ld, topk_idx,
                          teacher_logprob, k, mode, tail_eps, tau);
    if (rc) return rc;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        double LSE, P, Q, L;
        topk_row(logits, dtype, ld, i, vocab, topk_idx + i * k,
                 teacher_logprob + i * k, k, mode, tail_eps, tau, &LSE, &P, &Q, &L);
        if (loss) loss[i] = L;
        if (student_mass) student_mass[i] = Q;
        if (teacher_mass) teacher_mass[i] = P;
    }
    return 0;
}

int oracle_topk_kl_backward(const void *logits, int dtype, int64_t n_rows,
                            int64_t vocab, int64_t ld, const int32_t *topk_idx,
                            const float *teacher_logprob, int64_t k, int mode,
                            double tail_eps, double tau, const float *grad_loss,
                            double *grad) {
    int rc = topk_args_ok(logits, dtype, n_rows, vocab, ld, topk_idx,
                          teacher_logprob, k, mode, tail_eps, tau);
    if (rc) return rc;
    if (n_rows > 0 && (!grad_loss || !grad)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int32_t *idx = topk_idx + i * k;
        const float *tlp = teacher_logprob + i * k;
        double *gi = grad + i * vocab;
        double LSE, P, Q, L;
        topk_row(logits, dtype, ld, i, vocab, idx, tlp, k, mode, tail_eps, tau,
                 &LSE, &P, &Q, &L);
        double g = (double)grad_loss[i];
        /* the truncated loss before its clamp: a clamped row has no gradient */
        double Lraw = 0.0;
        for (int64_t n = 0; n < k; ++n) {
            double a = (double)tlp[n];
            Lraw += exp(a) * (a - (logit_at(logits, dtype, ld, i, idx[n]) / tau - LSE));
        }
        int row_dead = (mode == 0 && Lraw < 0.0) || g == 0.0;
        /* dL/d log q_{T_n} = -p_n;  tail: dL/d log qtail = -(1 - P), active guard: 0 */
        double dl_dlogqt = 0.0;
        if (mode == 1 && 1.0 - Q >= tail_eps) dl_dlogqt = -(P < 1.0 ? 1.0 - P : 0.0);
        for (int64_t j = 0; j < vocab; ++j) {
            if (row_dead) {
                gi[j] = 0.0;
                continue;
            }
            double qj = exp(logit_at(logits, dtype, ld, i, j) / tau - LSE);
            double in_t = 0.0;
            double d = 0.0;
            for (int64_t n = 0; n < k; ++n) {
                double p = exp((double)tlp[n]);
                double dlogq = (idx[n] == j ? 1.0 : 0.0) - qj; /* d log q_{T_n} / dz_j */
                d += -p * dlogq;
                if (idx[n] == j) in_t = 1.0;
            }
            /* d log qtail / dz_j = -(q_j [j in T] - q_j Q) / (1 - Q) */
            if (dl_dlogqt != 0.0)
                d += dl_dlogqt * (-(qj * in_t - qj * Q) / (1.0 - Q));
            gi[j] = g * d / tau;
        }
    }
    return 0;
}

int oracle_slice_partial(const void *logits_slice, int dtype, int64_t n_rows,
                         int64_t v_local, int64_t ld, int64_t v_start,
                         const int32_t *targets, const int32_t *rows, int64_t m,
                         double tau, double *pm, double *ps, double *pw,
                         double *pt) {
    if (!logits_slice || !dtype_ok(dtype) || n_rows < 0 || m < 0 ||
        v_local <= 0 || ld < v_local || v_start < 0 || !tau_ok(tau) ||
        (m && (!pm || !ps || !pw)) || (pt && !targets))
        return -1;
    int rc = check_rows(rows, m, n_rows);
    if (rc) return rc;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        int64_t r = row_of(rows, i);
        double M, S;
        row_max_sum(logits_slice, dtype, ld, r, 0, v_local, tau, &M, &S);
        double W = 0.0;
        for (int64_t j = 0; j < v_local; ++j) {
            double z = logit_at(logits_slice, dtype, ld, r, j) / tau;
            W += p_times(exp_shifted(z, M), z - M);
        }
        pm[i] = M;
        ps[i] = S;
        pw[i] = W;
        if (pt) {
            /* Only the slice that owns the target contributes its logit
               ("Reduce reference model memory ...", section "Implementation"). */
            int64_t t = targets[r];
            if (t >= v_start && t < v_start + v_local)
                pt[i] = logit_at(logits_slice, dtype, ld, r, t - v_start) / tau;
            else
                pt[i] = -INFINITY;
        }
    }
    return 0;
}

int oracle_combine(int64_t k, int64_t m, const double *pm, const double *ps,
                   const double *pw, const double *pt, double *logprob,
                   double *lse, double *entropy) {
    if (k <= 0 || m < 0 || (m && (!pm || !ps || !pw)) || (logprob && !pt))
        return -1;
    for (int64_t i = 0; i < m; ++i) {
        /* Global max over the slices. */
        double M = -INFINITY;
        for (int64_t q = 0; q < k; ++q)
            if (pm[q * m + i] > M) M = pm[q * m + i];
        /* Sum of exp(z - M): each slice's sum rescaled from its own max. */
        double S = 0.0, W = 0.0, T = -INFINITY;
        for (int64_t q = 0; q < k; ++q) {
            if (pt && pt[q * m + i] > T) T = pt[q * m + i];
            /* A slice whose logits are all -inf has S = 0 and adds nothing. */
            if (ps[q * m + i] == 0.0) continue;
            double d = pm[q * m + i] - M;
            double f = exp(d);
            S += ps[q * m + i] * f;
            /* sum exp(z - M)(z - M) = sum exp(z - M_q) e^d ((z - M_q) + d) */
            W += f * (pw[q * m + i] + d * ps[q * m + i]);
        }
        double LSE = M + log(S);
        if (lse) lse[i] = LSE;
        if (logprob) logprob[i] = T - LSE;
        /* H = LSE - E_p[z] = log S - W / S. */
        if (entropy) entropy[i] = log(S) - W / S;
    }
    return 0;
}

int oracle_forward_vchunk(const void *logits, int dtype, int64_t n_rows,
                          int64_t vocab, int64_t ld, const int32_t *targets,
                          const int32_t *rows, int64_t m, double tau,
                          int64_t vchunk, double *logprob, double *lse,
                          double *entropy) {
    if (vchunk <= 0) return -1;
    if (!logits || !dtype_ok(dtype) || n_rows < 0 || m < 0 || vocab <= 0 ||
        ld < vocab || !tau_ok(tau) || (logprob && !targets))
        return -1;
    int rc = check_rows(rows, m, n_rows);
    if (rc) return rc;
    if (logprob && (rc = check_targets(targets, rows, m, vocab))) return rc;
    if (m == 0) return 0;

    int64_t k = (vocab + vchunk - 1) / vchunk;
    size_t n = (size_t)(k * m);
    double *pm = malloc(n * sizeof(double)), *ps = malloc(n * sizeof(double));
    double *pw = malloc(n * sizeof(double)), *pt = malloc(n * sizeof(double));
    if (!pm || !ps || !pw || !pt) {
        free(pm); free(ps); free(pw); free(pt);
        return -4;
    }
    const size_t esize = dtype == ORACLE_BF16 ? 2 : 4;
    for (int64_t q = 0; q < k; ++q) {
        int64_t v0 = q * vchunk;
        int64_t vl = v0 + vchunk <= vocab ? vchunk : vocab - v0;
        const char *slice = (const char *)logits + (size_t)v0 * esize;
        rc = oracle_slice_partial(slice, dtype, n_rows, vl, ld, v0,
                                  logprob ? targets : NULL, rows, m, tau,
                                  pm + q * m, ps + q * m, pw + q * m,
                                  logprob ? pt + q * m : NULL);
        if (rc) break;
    }
    if (!rc)
        rc = oracle_combine(k, m, pm, ps, pw, logprob ? pt : NULL, logprob, lse,
                            entropy);
    free(pm); free(ps); free(pw); free(pt);
    return rc;
}

/* ------------------------------------------------------------ LM head */

static int lmhead_args_ok(const uint16_t *hidden, int64_t n_rows, int64_t ldh,
                          const uint16_t *weight, int64_t vocab, int64_t ldw,
                          int64_t d, int64_t m) {
    return hidden && weight && n_rows >= 0 && m >= 0 && vocab > 0 && d > 0 &&
           ldh >= d && ldw >= d;
}

int oracle_lmhead_logits(const uint16_t *hidden, int64_t n_rows, int64_t ldh,
                         const uint16_t *weight, int64_t vocab, int64_t ldw,
                         int64_t d, const int32_t *rows, int64_t m, double *x,
                         double *abs_sum) {
    if (!lmhead_args_ok(hidden, n_rows, ldh, weight, vocab, ldw, d, m) || (m && !x))
        return -1;
    int rc = check_rows(rows, m, n_rows);
    if (rc) return rc;
    for (int64_t i = 0; i < m; ++i) {
        const uint16_t *h = hidden + row_of(rows, i) * ldh;
        /* Columns are independent dot products; threads split the columns. */
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < vocab; ++j) {
            const uint16_t *w = weight + j * ldw;
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < d; ++k) {
                double p = decode_bf16(h[k]) * decode_bf16(w[k]);
                s += p;
                a += fabs(p);
            }
            x[i * vocab + j] = s;
            if (abs_sum) abs_sum[i * vocab + j] = a;
        }
    }
    return 0;
}

int oracle_lmhead_forward(const uint16_t *hidden, int64_t n_rows, int64_t ldh,
                          const uint16_t *weight, int64_t vocab, int64_t ldw,
                          int64_t d, const int32_t *targets, const int32_t *rows,
                          int64_t m, double tau, int64_t row_chunk,
                          double *logprob, double *lse, double *entropy,
                          double *err_scale) {
    if (row_chunk <= 0 || !tau_ok(tau) ||
        !lmhead_args_ok(hidden, n_rows, ldh, weight, vocab, ldw, d, m))
        return -1;
    if (logprob && !targets) return -1;
    int rc = check_rows(rows, m, n_rows);
    if (rc) return rc;
    if (logprob && (rc = check_targets(targets, rows, m, vocab))) return rc;
    if (m == 0) return 0;

    int64_t cap = row_chunk < m ? row_chunk : m;
    double *x = malloc((size_t)(cap * vocab) * sizeof(double));
    double *a = err_scale ? malloc((size_t)(cap * vocab) * sizeof(double)) : NULL;
    int32_t *sub_rows = malloc((size_t)cap * sizeof(int32_t));
    int32_t *sub_targets = malloc((size_t)cap * sizeof(int32_t));
    if (!x || (err_scale && !a) || !sub_rows || !sub_targets) {
        free(x);
        free(a);
        free(sub_rows);
        free(sub_targets);
        return -4;
    }
    for (int64_t c0 = 0; c0 < m && rc == 0; c0 += cap) {
        int64_t n = c0 + cap < m ? cap : m - c0;
        for (int64_t i = 0; i < n; ++i) {
            sub_rows[i] = (int32_t)row_of(rows, c0 + i);
            sub_targets[i] = targets ? targets[sub_rows[i]] : 0;
        }
        rc = oracle_lmhead_logits(hidden, n_rows, ldh, weight, vocab, ldw, d, sub_rows,
                                  n, x, a);
        /* The chunk's logits are rows 0..n-1 of an fp64 matrix; targets follow. */
        if (rc == 0)
            rc = oracle_forward(x, ORACLE_FP64, n, vocab, vocab, targets ? sub_targets : NULL,
                                NULL, n, tau, n, logprob ? logprob + c0 : NULL,
                                lse ? lse + c0 : NULL, entropy ? entropy + c0 : NULL);
        if (rc == 0 && err_scale) {
            for (int64_t i = 0; i < n; ++i) {
                const double *ai = a + i * vocab;
                double amax = 0.0;
                for (int64_t j = 0; j < vocab; ++j)
                    if (ai[j] > amax) amax = ai[j];
                err_scale[c0 + i] = ((targets ? ai[sub_targets[i]] : 0.0) + amax) / tau;
            }
        }
    }
    free(x);
    free(a);
    free(sub_rows);
    free(sub_targets);
    return rc;
}

/*
 * Nearest bf16 to v, ties to even, straight from the double (no detour through
 * float, which would round twice).  bf16 has fp32's exponent range and 8
 * significant bits; below 2^-126 its spacing is the fixed 2^-133.  Dividing by
 * the spacing is exact (a power of two), rint() rounds to nearest-even in the
 * default rounding mode, and the product is exactly representable in float.
 */
uint16_t oracle_bf16_rne(double v) {
    if (isnan(v)) return 0x7FC0;
    if (isinf(v)) return v > 0 ? 0x7F80 : 0xFF80;
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    int e;
    frexp(v, &e); /* |v| = f * 2^e with f in [0.5, 1): the leading bit is 2^(e-1) */
    int lead = e - 1;
    int q_exp = lead < -126 ? -133 : lead - 7;
    double q = ldexp(1.0, q_exp);
    double r = rint(v / q) * q;
    if (fabs(r) >= ldexp(1.0, 128)) return v > 0 ? 0x7F80 : 0xFF80;
    float f = (float)r; /* exact */
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    if (r == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    return (uint16_t)(w >> 16);
}

void oracle_bf16_rne_array(const double *v, uint16_t *out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_rne(v[i]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
