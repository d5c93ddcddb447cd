/*
 * la2_oracle.c -- CPU oracle for causal linear attention (test infrastructure only).
 *
 * This file is the slow, plain, fp64 definition that the GPU kernels are checked
 * against.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load it; the product path never does.  It shares no code, header or
 * constant with the HIP library.
 *
 * What it computes (page "Lightning Attention", lizeman.github.io llm-arch-kb,
 * section 1 "Premise", the numerator of the output equation and the prefix-sum
 * recurrence S_t = S_{t-1} + phi(k_t) v_t^T):
 *   - the feature map phi is the identity (same page, section 2, where the
 *     default configuration is said to use identity phi);
 *   - no denominator: only the numerator recurrence is computed;
 *   - an optional per-head decay lam in (0, 1] multiplies the past state:
 *         S_t = lam * S_{t-1} + k_t v_t^T,      o_t = S_t^T q_t,
 *     which for lam = 1 is exactly the page's prefix sum.
 *
 * Backward (derived from the forward by the chain rule; the pages only state
 * that the backward is tiled as well -- Lightning Attention-2 abstract, arXiv
 * 2401.04658 card):
 *   dq_t = S_t do_t                                  (forward sweep, same S_t)
 *   R_t  = lam * R_{t+1} + q_t do_t^T,  R_{T+1} = 0  (reverse sweep)
 *   dk_t = R_t v_t,   dv_t = R_t^T k_t
 *
 * la2_oracle_backward_state is the backward of la2_oracle_forward_state: the gradients of
 * <o, do> + <state_out, ds_out>, the carried-in state's among them (ds_in = lam R_0), so that a
 * sequence trained in chunks gets the same gradients as trained whole.
 *
 * la2_oracle_forward_normalized is the full output of the same section 1, numerator
 * over denominator, with a feature map phi (identity, or elu + 1) and the decay
 * applied to the denominator's prefix sum z_t = lam z_{t-1} + phi(k_t) as to S;
 * la2_oracle_backward_normalized is its backward, by the chain rule through the ratio.
 *
 * The *_rows entry points evaluate the same quantities one output row at a
 * time from the closed sums
 *   o_t  = sum_{s<=t} lam^{t-s} (q_t . k_s) v_s
 *   dq_t = sum_{s<=t} lam^{t-s} (do_t . v_s) k_s
 *   dk_t = sum_{s>=t} lam^{s-t} (do_s . v_t) q_s
 *   dv_t = sum_{s>=t} lam^{s-t} (q_s . k_t) do_s
 * so that single rows of very long sequences can be checked without running
 * the whole recurrence.
 *
 * Layout: every tensor is a contiguous array of chains, each chain a row-major
 * [T, d] (q, k, dq, dk) or [T, dv] (v, o, do, dv) block of doubles.  lam holds
 * one decay per chain.  All arithmetic is IEEE fp64; no fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- whole-sequence recurrences --------------------------------------- */

/* The recurrence carried in from and out to a state, the summary of everything before the
 * sequence (same page, section 2, "Memory footprint": the only state that persists across tiles
 * is the d x dv matrix S).  s_in, s_out: [n_chains][d][dv] or NULL.  The sequence starts from
 * S_{-1} = s_in (0 when NULL), so its first step is S_0 = lam * s_in + k_0 v_0^T, and S_{T-1} is
 * written to s_out.  Splitting a sequence at any t and carrying S_{t-1} over gives the same o. */
void la2_oracle_forward_state(int64_t n_chains, int64_t T, int64_t d, int64_t dv,
                              const double *lam, const double *q, const double *k,
                              const double *v, const double *s_in, double *o, double *s_out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < n_chains; ++c) {
        const double *qc = q + c * T * d;
        const double *kc = k + c * T * d;
        const double *vc = v + c * T * dv;
        double *oc = o + c * T * dv;
        const double l = lam[c];
        double *S = (double *)calloc((size_t)(d * dv), sizeof(double)); /* S[i][j], i < d, j < dv */
        if (s_in)
            for (int64_t i = 0; i < d; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] = s_in[c * d * dv + i * dv + j];
        for (int64_t t = 0; t < T; ++t) {
            const double *kt = kc + t * d, *vt = vc + t * dv, *qt = qc + t * d;
            /* S_t = lam * S_{t-1} + k_t v_t^T */
            for (int64_t i = 0; i < d; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] = l * S[i * dv + j] + kt[i] * vt[j];
            /* o_t = S_t^T q_t */
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < d; ++i)
                    acc += S[i * dv + j] * qt[i];
                oc[t * dv + j] = acc;
            }
        }
        if (s_out)
            for (int64_t i = 0; i < d; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    s_out[c * d * dv + i * dv + j] = S[i * dv + j];
        free(S);
    }
}

void la2_oracle_forward(int64_t n_chains, int64_t T, int64_t d, int64_t dv,
                        const double *lam, const double *q, const double *k,
                        const double *v, double *o)
{
    la2_oracle_forward_state(n_chains, T, d, dv, lam, q, k, v, NULL, o, NULL);
}

/* ---- normalized form with a feature map ------------------------------- */

/* The feature map phi applied elementwise: 0 = identity (the default configuration named on the
 * "Lightning Attention" page, section 2), 1 = elu(x) + 1 (x + 1 for x > 0, e^x otherwise), a
 * strictly positive map as in the linear-transformer lineage that page builds on (section 1). */
static double feature(double x, int fmap)
{
    if (fmap == 1)
        return x > 0.0 ? x + 1.0 : exp(x);
    return x;
}

/* Normalized output of the same page, section 1 (numerator over denominator, both prefix sums of
 * phi(k)), with the decay applied to both recurrences:
 *   S_t = lam S_{t-1} + phi(k_t) v_t^T,   z_t = lam z_{t-1} + phi(k_t),
 *   o_t = (S_t^T phi(q_t)) / (z_t . phi(q_t)).
 * No epsilon: with a strictly positive phi the denominator is positive. */
void la2_oracle_forward_normalized(int64_t n_chains, int64_t T, int64_t d, int64_t dv,
                                   const double *lam, const double *q, const double *k,
                                   const double *v, int fmap, double *o)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < n_chains; ++c) {
        const double l = lam[c];
        double *S = (double *)calloc((size_t)(d * dv), sizeof(double));
        double *z = (double *)calloc((size_t)d, sizeof(double));
        double *pq = (double *)malloc((size_t)d * sizeof(double));
        double *pk = (double *)malloc((size_t)d * sizeof(double));
        for (int64_t t = 0; t < T; ++t) {
            const double *qt = q + (c * T + t) * d, *kt = k + (c * T + t) * d, *vt = v + (c * T + t) * dv;
            for (int64_t i = 0; i < d; ++i) {
                pq[i] = feature(qt[i], fmap);
                pk[i] = feature(kt[i], fmap);
            }
            double den = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                z[i] = l * z[i] + pk[i];
                den += z[i] * pq[i];
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] = l * S[i * dv + j] + pk[i] * vt[j];
            }
            for (int64_t j = 0; j < dv; ++j) {
                double num = 0.0;
                for (int64_t i = 0; i < d; ++i)
                    num += S[i * dv + j] * pq[i];
                o[(c * T + t) * dv + j] = num / den;
            }
        }
        free(S);
        free(z);
        free(pq);
        free(pk);
    }
}

/* Backward of the forward carried in from s_in and out to state_out = S_{T-1} (fp64 [d, dv] per
 * chain, as la2_oracle_forward_state), for the loss <o, dout> + <state_out, ds_out>.  By the chain
 * rule through the recurrence:
 *   dq_t = S_t do_t                       (the forward sweep from S_{-1} = s_in)
 *   R_{T-1} = q_{T-1} do_{T-1}^T + ds_out,   R_t = lam R_{t+1} + q_t do_t^T
 *   dk_t = R_t v_t,   dv_t = R_t^T k_t,   ds_in = lam R_0
 * s_in, ds_out: NULL for zero; ds_in: NULL when not wanted. */
/* Derivative of the feature map: 1 for the identity, 1 above 0 and e^x at or below for elu + 1. */
static double feature_deriv(double x, int fmap)
{
    if (fmap == 1)
        return x > 0.0 ? 1.0 : exp(x);
    return 1.0;
}

/* Backward of la2_oracle_forward_normalized for the loss <o, dout>, by the chain rule through
 * o_t = n_t / den_t, n_t = S_t^T pq_t, den_t = z_t . pq_t (pq = phi(q), pk = phi(k)):
 *   dn_t = do_t / den_t,   dden_t = -(do_t . o_t) / den_t
 *   d pq_t = S_t dn_t + dden_t z_t
 *   R_t = lam R_{t+1} + pq_t dn_t^T,   y_t = lam y_{t+1} + dden_t pq_t     (reverse sweep)
 *   d pk_t = R_t v_t + y_t,   dv_t = R_t^T pk_t
 *   dq = d pq (.) phi'(q),   dk = d pk (.) phi'(k). */
void la2_oracle_backward_normalized(int64_t n_chains, int64_t T, int64_t d, int64_t dv,
                                    const double *lam, const double *q, const double *k,
                                    const double *v, const double *dout, int fmap, double *dq,
                                    double *dk, double *dvo)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < n_chains; ++c) {
        const double l = lam[c];
        const double *qc = q + c * T * d, *kc = k + c * T * d, *vc = v + c * T * dv, *gc = dout + c * T * dv;
        double *dqc = dq + c * T * d, *dkc = dk + c * T * d, *dvc = dvo + c * T * dv;
        double *S = (double *)calloc((size_t)(d * dv), sizeof(double));
        double *z = (double *)calloc((size_t)d, sizeof(double));
        double *pq = (double *)malloc((size_t)(T * d) * sizeof(double));
        double *pk = (double *)malloc((size_t)(T * d) * sizeof(double));
        double *dn = (double *)malloc((size_t)(T * dv) * sizeof(double));
        double *dden = (double *)malloc((size_t)T * sizeof(double));
        for (int64_t e = 0; e < T * d; ++e) {
            pq[e] = feature(qc[e], fmap);
            pk[e] = feature(kc[e], fmap);
        }
        /* forward sweep: S_t, z_t, the output, then d pq_t */
        for (int64_t t = 0; t < T; ++t) {
            const double *pqt = pq + t * d, *pkt = pk + t * d, *vt = vc + t * dv, *gt = gc + t * dv;
            double den = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                z[i] = l * z[i] + pkt[i];
                den += z[i] * pqt[i];
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] = l * S[i * dv + j] + pkt[i] * vt[j];
            }
            double go = 0.0;
            for (int64_t j = 0; j < dv; ++j) {
                double num = 0.0;
                for (int64_t i = 0; i < d; ++i)
                    num += S[i * dv + j] * pqt[i];
                go += gt[j] * (num / den);
                dn[t * dv + j] = gt[j] / den;
            }
            dden[t] = -go / den;
            for (int64_t i = 0; i < d; ++i) {
                double acc = dden[t] * z[i];
                for (int64_t j = 0; j < dv; ++j)
                    acc += S[i * dv + j] * dn[t * dv + j];
                dqc[t * d + i] = acc * feature_deriv(qc[t * d + i], fmap);
            }
        }
        /* reverse sweep: R_t, y_t, then d pk_t and dv_t */
        double *R = S, *y = z;
        memset(R, 0, sizeof(double) * (size_t)(d * dv));
        memset(y, 0, sizeof(double) * (size_t)d);
        for (int64_t t = T - 1; t >= 0; --t) {
            const double *pqt = pq + t * d, *pkt = pk + t * d, *vt = vc + t * dv;
            for (int64_t i = 0; i < d; ++i) {
                y[i] = l * y[i] + dden[t] * pqt[i];
                for (int64_t j = 0; j < dv; ++j)
                    R[i * dv + j] = l * R[i * dv + j] + pqt[i] * dn[t * dv + j];
            }
            for (int64_t i = 0; i < d; ++i) {
                double acc = y[i];
                for (int64_t j = 0; j < dv; ++j)
                    acc += vt[j] * R[i * dv + j];
                dkc[t * d + i] = acc * feature_deriv(kc[t * d + i], fmap);
            }
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < d; ++i)
                    acc += R[i * dv + j] * pkt[i];
                dvc[t * dv + j] = acc;
            }
        }
        free(S);
        free(z);
        free(pq);
        free(pk);
        free(dn);
        free(dden);
    }
}

void la2_oracle_backward_state(int64_t n_chains, int64_t T, int64_t d, int64_t dv,
                               const double *lam, const double *q, const double *k,
                               const double *v, const double *dout, const double *s_in,
                               const double *ds_out, double *dq, double *dk, double *dvo,
                               double *ds_in)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < n_chains; ++c) {
        const double *qc = q + c * T * d;
        const double *kc = k + c * T * d;
        const double *vc = v + c * T * dv;
        const double *gc = dout + c * T * dv;
        double *dqc = dq + c * T * d;
        double *dkc = dk + c * T * d;
        double *dvc = dvo + c * T * dv;
        const double l = lam[c];
        double *S = (double *)calloc((size_t)(d * dv), sizeof(double));
        if (s_in)
            for (int64_t e = 0; e < d * dv; ++e)
                S[e] = s_in[c * d * dv + e];
        /* forward sweep: dq_t = S_t do_t */
        for (int64_t t = 0; t < T; ++t) {
            const double *kt = kc + t * d, *vt = vc + t * dv, *gt = gc + t * dv;
            for (int64_t i = 0; i < d; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] = l * S[i * dv + j] + kt[i] * vt[j];
            for (int64_t i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j)
                    acc += S[i * dv + j] * gt[j];
                dqc[t * d + i] = acc;
            }
        }
        /* reverse sweep: R_t = lam R_{t+1} + q_t do_t^T (+ ds_out at the last position);
         * dk_t = R_t v_t; dv_t = R_t^T k_t */
        double *R = S;
        memset(R, 0, sizeof(double) * (size_t)(d * dv));
        for (int64_t t = T - 1; t >= 0; --t) {
            const double *qt = qc + t * d, *gt = gc + t * dv;
            const double *kt = kc + t * d, *vt = vc + t * dv;
            for (int64_t i = 0; i < d; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    R[i * dv + j] = l * R[i * dv + j] + qt[i] * gt[j];
            if (ds_out && t == T - 1)
                for (int64_t e = 0; e < d * dv; ++e)
                    R[e] += ds_out[c * d * dv + e];
            for (int64_t i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int64_t j = 0; j < dv; ++j)
                    acc += R[i * dv + j] * vt[j];
                dkc[t * d + i] = acc;
            }
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < d; ++i)
                    acc += R[i * dv + j] * kt[i];
                dvc[t * dv + j] = acc;
            }
        }
        /* ds_in: S_t depends on s_in through lam^(t+1) */
        if (ds_in)
            for (int64_t e = 0; e < d * dv; ++e)
                ds_in[c * d * dv + e] = l * R[e];
        free(S);
    }
}

void la2_oracle_backward(int64_t n_chains, int64_t T, int64_t d, int64_t dv,
                         const double *lam, const double *q, const double *k,
                         const double *v, const double *dout, double *dq,
                         double *dk, double *dvo)
{
    la2_oracle_backward_state(n_chains, T, d, dv, lam, q, k, v, dout, NULL, NULL, dq, dk, dvo, NULL);
}

/* ---- single rows from the closed sums (one chain) ---------------------- */

static double dot(const double *a, const double *b, int64_t n)
{
    double acc = 0.0;
    for (int64_t i = 0; i < n; ++i)
        acc += a[i] * b[i];
    return acc;
}

/* o rows: out[r, :] = o_{rows[r]} for the chain (q, k, v) with decay lam. */
void la2_oracle_forward_rows(int64_t T, int64_t d, int64_t dv, double lam,
                             const double *q, const double *k, const double *v,
                             int64_t n_rows, const int64_t *rows, double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t t = rows[r];
        double *y = out + r * dv;
        for (int64_t j = 0; j < dv; ++j)
            y[j] = 0.0;
        if (t < 0 || t >= T)
            continue;
        for (int64_t s = 0; s <= t; ++s) {
            const double w = pow(lam, (double)(t - s)) * dot(q + t * d, k + s * d, d);
            for (int64_t j = 0; j < dv; ++j)
                y[j] += w * v[s * dv + j];
        }
    }
}

/* dq, dk, dv rows for the chain; each output row block is [n_rows, width]. */
void la2_oracle_backward_rows(int64_t T, int64_t d, int64_t dv, double lam,
                              const double *q, const double *k, const double *v,
                              const double *dout, int64_t n_rows,
                              const int64_t *rows, double *dq_rows,
                              double *dk_rows, double *dv_rows)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t t = rows[r];
        double *gq = dq_rows + r * d, *gk = dk_rows + r * d, *gv = dv_rows + r * dv;
        for (int64_t i = 0; i < d; ++i)
            gq[i] = gk[i] = 0.0;
        for (int64_t j = 0; j < dv; ++j)
            gv[j] = 0.0;
        if (t < 0 || t >= T)
            continue;
        /* dq_t = sum_{s<=t} lam^{t-s} (do_t . v_s) k_s */
        for (int64_t s = 0; s <= t; ++s) {
            const double w = pow(lam, (double)(t - s)) * dot(dout + t * dv, v + s * dv, dv);
            for (int64_t i = 0; i < d; ++i)
                gq[i] += w * k[s * d + i];
        }
        /* dk_t = sum_{s>=t} lam^{s-t} (do_s . v_t) q_s ; dv_t = sum_{s>=t} lam^{s-t} (q_s . k_t) do_s */
        for (int64_t s = t; s < T; ++s) {
            const double p = pow(lam, (double)(s - t));
            const double wk = p * dot(dout + s * dv, v + t * dv, dv);
            const double wv = p * dot(q + s * d, k + t * d, d);
            for (int64_t i = 0; i < d; ++i)
                gk[i] += wk * q[s * d + i];
            for (int64_t j = 0; j < dv; ++j)
                gv[j] += wv * dout[s * dv + j];
        }
    }
}

int la2_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following oracle calls (timing only; results do not depend on it). */
void la2_oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
