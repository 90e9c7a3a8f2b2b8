/*
 * la_oracle.c -- plain, slow, fp64 CPU oracle for linear attention with the
 * feature map phi(x) = elu(x) + 1.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no source with the HIP library.
 *
 * Every routine is the plain definition written out, one token at a time, in
 * double precision, in the order the pages state it:
 *
 *   - Feature map: "Transformers are RNNs" blog digest (irregular6612), section
 *     "Methods" and "Method / key components 1)"; velog review, section 3.3
 *     "Feature Maps and Computational Cost"; itwiki "Linear attention"
 *     (선형 어텐션), section "Formulas".  phi(x) = elu(x) + 1 with the ELU
 *     slope alpha = 1, i.e. x + 1 for x > 0 and exp(x) otherwise.
 *   - Causal form: blog digest, "Method / key components 3) and 4)"; velog
 *     review sections 3.4 "Causal Masking" and 3.6 "Transformers and RNNs";
 *     itwiki "Linear attention", section "Causal masking and the recurrent
 *     form".  S_i = S_{i-1} + phi(k_i) v_i^T, z_i = z_{i-1} + phi(k_i),
 *     out_i = phi(q_i)^T S_i / phi(q_i)^T z_i: the state is updated with
 *     token i first, then read (the prefix sum includes j = i).
 *   - Non-causal form: blog digest "Method / key components 2)"; velog review
 *     section 3.2 "Linearized Attention"; itwiki "Formulas / reordering by
 *     associativity".  The same sums taken over all N tokens.
 *   - Gradient: velog review section 3.5 "Gradient Computation" states only
 *     that the gradient is itself written as cumulative sums so that memory
 *     stays linear; the formulas are not printed.  The routine below is the
 *     exact gradient of out_i = num_i / den_i, written as one forward and one
 *     reverse cumulative sum over an augmented value vector [v, 1].
 *
 * Layouts (row-major, contiguous): sequences [B][H][N][d], state S
 * [B][H][d_k][d_v], normaliser z [B][H][d_k], per-token den [B][H][N].
 * OpenMP, when enabled at build time, parallelises over the independent
 * (batch, head) pairs only; the arithmetic inside each pair is sequential.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* phi(x) = elu(x) + 1 with alpha = 1. */
static double phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* d phi / dx: 1 for x > 0, exp(x) otherwise (continuous at 0). */
static double dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }

/* Number of threads OpenMP would use for the (batch, head) loop. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Causal forward, recurrent form.  For every (b, h): S = 0, z = 0; for each
 * token i in order, add phi(k_i) v_i^T to S and phi(k_i) to z, then
 * den_i = phi(q_i) . z and out_i = phi(q_i)^T S / den_i.
 * `den` may be NULL.
 */
void oracle_fwd_causal_f64(const double *q, const double *k, const double *v,
                           double *o, double *den,
                           int B, int H, int N, int dk, int dv)
{
    long BH = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        const double *qb = q + bh * (long)N * dk;
        const double *kb = k + bh * (long)N * dk;
        const double *vb = v + bh * (long)N * dv;
        double *ob = o + bh * (long)N * dv;
        double *S = calloc((size_t)dk * dv, sizeof(double));
        double *z = calloc((size_t)dk, sizeof(double));
        double *fq = malloc((size_t)dk * sizeof(double));
        for (int i = 0; i < N; ++i) {
            const double *ki = kb + (long)i * dk;
            const double *vi = vb + (long)i * dv;
            const double *qi = qb + (long)i * dk;
            for (int e = 0; e < dk; ++e) {
                double fk = phi(ki[e]);
                z[e] += fk;
                for (int c = 0; c < dv; ++c) S[(long)e * dv + c] += fk * vi[c];
            }
            double d = 0.0;
            for (int e = 0; e < dk; ++e) {
                fq[e] = phi(qi[e]);
                d += fq[e] * z[e];
            }
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int e = 0; e < dk; ++e) num += fq[e] * S[(long)e * dv + c];
                ob[(long)i * dv + c] = num / d;
            }
            if (den) den[bh * (long)N + i] = d;
        }
        free(S);
        free(z);
        free(fq);
    }
}

/*
 * Non-causal forward: S = sum_j phi(k_j) v_j^T and z = sum_j phi(k_j) over all
 * N tokens, then out_i = phi(q_i)^T S / phi(q_i) . z for every i.
 */
void oracle_fwd_noncausal_f64(const double *q, const double *k, const double *v,
                              double *o, int B, int H, int N, int dk, int dv)
{
    long BH = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        const double *qb = q + bh * (long)N * dk;
        const double *kb = k + bh * (long)N * dk;
        const double *vb = v + bh * (long)N * dv;
        double *ob = o + bh * (long)N * dv;
        double *S = calloc((size_t)dk * dv, sizeof(double));
        double *z = calloc((size_t)dk, sizeof(double));
        double *fq = malloc((size_t)dk * sizeof(double));
        for (int j = 0; j < N; ++j) {
            for (int e = 0; e < dk; ++e) {
                double fk = phi(kb[(long)j * dk + e]);
                z[e] += fk;
                for (int c = 0; c < dv; ++c) S[(long)e * dv + c] += fk * vb[(long)j * dv + c];
            }
        }
        for (int i = 0; i < N; ++i) {
            double d = 0.0;
            for (int e = 0; e < dk; ++e) {
                fq[e] = phi(qb[(long)i * dk + e]);
                d += fq[e] * z[e];
            }
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int e = 0; e < dk; ++e) num += fq[e] * S[(long)e * dv + c];
                ob[(long)i * dv + c] = num / d;
            }
        }
        free(S);
        free(z);
        free(fq);
    }
}

/*
 * One recurrent decode step on a persistent state: for every (b, h),
 * S += phi(k) v^T, z += phi(k), then out = phi(q)^T S / phi(q) . z.
 * S [B][H][dk][dv] and z [B][H][dk] are read and written in place;
 * q, k [B][H][dk], v and out [B][H][dv].
 */
void oracle_decode_step_f64(double *S, double *z, const double *q, const double *k,
                            const double *v, double *o, int B, int H, int dk, int dv)
{
    long BH = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < BH; ++bh) {
        double *Sb = S + bh * (long)dk * dv;
        double *zb = z + bh * (long)dk;
        const double *qb = q + bh * (long)dk;
        const double *kb = k + bh * (long)dk;
        const double *vb = v + bh * (long)dv;
        double *ob = o + bh * (long)dv;
        for (int e = 0; e < dk; ++e) {
            double fk = phi(kb[e]);
            zb[e] += fk;
            for (int c = 0; c < dv; ++c) Sb[(long)e * dv + c] += fk * vb[c];
        }
        double d = 0.0;
        for (int e = 0; e < dk; ++e) d += phi(qb[e]) * zb[e];
        for (int c = 0; c < dv; ++c) {
            double num = 0.0;
            for (int e = 0; e < dk; ++e) num += phi(qb[e]) * Sb[(long)e * dv + c];
            ob[c] = num / d;
        }
    }
}

/*
 * Cumulative-sum backward of the causal form.
 *
 * Given the upstream gradient g_i = dL/dout_i, with num_i = phi(q_i)^T S_i and
 * den_i = phi(q_i) . z_i:
 *   dL/dnum_i = g_i / den_i                      (call it gh_i, length dv)
 *   dL/dden_i = -(g_i . out_i) / den_i           (call it eps_i, a scalar)
 * Writing V'_j = [v_j, 1] and G'_i = [gh_i, eps_i], the pair (num_i, den_i)
 * equals phi(q_i)^T S'_i with S'_i = sum_{j<=i} phi(k_j) V'_j^T, so
 *   dL/dphi(q_i) = S'_i G'_i                      (forward cumulative sum)
 *   dL/dphi(k_j) = R'_j V'_j,   R'_j = sum_{i>=j} phi(q_i) G'_i^T
 *   dL/dv_j      = R_j^T phi(k_j), R_j = the first dv columns of R'_j
 *                                                 (reverse cumulative sum)
 * and the chain rule through phi gives dq = dL/dphi(q) * phi'(q),
 * dk = dL/dphi(k) * phi'(k).  Only d x (dv + 1) running sums are kept: no
 * per-token state is stored.  out_i and den_i are recomputed here in fp64.
 */
void oracle_bwd_causal_f64(const double *q, const double *k, const double *v,
                           const double *g, double *dq, double *dk_out, double *dv_out,
                           int B, int H, int N, int dk, int dv)
{
    long BH = (long)B * H;
    int dv1 = dv + 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        const double *qb = q + bh * (long)N * dk;
        const double *kb = k + bh * (long)N * dk;
        const double *vb = v + bh * (long)N * dv;
        const double *gb = g + bh * (long)N * dv;
        double *dqb = dq + bh * (long)N * dk;
        double *dkb = dk_out + bh * (long)N * dk;
        double *dvb = dv_out + bh * (long)N * dv;

        double *o = malloc((size_t)N * dv * sizeof(double));
        double *den = malloc((size_t)N * sizeof(double));
        double *Gp = malloc((size_t)N * dv1 * sizeof(double)); /* G'_i */
        double *Sp = calloc((size_t)dk * dv1, sizeof(double));  /* S' or R' */

        /* Forward pass for out and den (same recurrence as the forward). */
        for (int i = 0; i < N; ++i) {
            for (int e = 0; e < dk; ++e) {
                double fk = phi(kb[(long)i * dk + e]);
                for (int c = 0; c < dv; ++c) Sp[(long)e * dv1 + c] += fk * vb[(long)i * dv + c];
                Sp[(long)e * dv1 + dv] += fk;
            }
            double d = 0.0;
            for (int e = 0; e < dk; ++e) d += phi(qb[(long)i * dk + e]) * Sp[(long)e * dv1 + dv];
            den[i] = d;
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int e = 0; e < dk; ++e) num += phi(qb[(long)i * dk + e]) * Sp[(long)e * dv1 + c];
                o[(long)i * dv + c] = num / d;
            }
        }

        /* G'_i = [g_i / den_i, -(g_i . out_i) / den_i]. */
        for (int i = 0; i < N; ++i) {
            double go = 0.0;
            for (int c = 0; c < dv; ++c) {
                Gp[(long)i * dv1 + c] = gb[(long)i * dv + c] / den[i];
                go += gb[(long)i * dv + c] * o[(long)i * dv + c];
            }
            Gp[(long)i * dv1 + dv] = -go / den[i];
        }

        /* Forward cumulative sum: S'_i, then dq_i = (S'_i G'_i) * phi'(q_i). */
        memset(Sp, 0, (size_t)dk * dv1 * sizeof(double));
        for (int i = 0; i < N; ++i) {
            for (int e = 0; e < dk; ++e) {
                double fk = phi(kb[(long)i * dk + e]);
                for (int c = 0; c < dv; ++c) Sp[(long)e * dv1 + c] += fk * vb[(long)i * dv + c];
                Sp[(long)e * dv1 + dv] += fk;
            }
            for (int e = 0; e < dk; ++e) {
                double acc = 0.0;
                for (int c = 0; c < dv1; ++c) acc += Sp[(long)e * dv1 + c] * Gp[(long)i * dv1 + c];
                dqb[(long)i * dk + e] = acc * dphi(qb[(long)i * dk + e]);
            }
        }

        /* Reverse cumulative sum: R'_j, then dk_j and dv_j. */
        memset(Sp, 0, (size_t)dk * dv1 * sizeof(double));
        for (int j = N - 1; j >= 0; --j) {
            for (int e = 0; e < dk; ++e) {
                double fq = phi(qb[(long)j * dk + e]);
                for (int c = 0; c < dv1; ++c) Sp[(long)e * dv1 + c] += fq * Gp[(long)j * dv1 + c];
            }
            for (int e = 0; e < dk; ++e) {
                double acc = Sp[(long)e * dv1 + dv]; /* times V'_j[dv] = 1 */
                for (int c = 0; c < dv; ++c) acc += Sp[(long)e * dv1 + c] * vb[(long)j * dv + c];
                dkb[(long)j * dk + e] = acc * dphi(kb[(long)j * dk + e]);
            }
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int e = 0; e < dk; ++e) acc += Sp[(long)e * dv1 + c] * phi(kb[(long)j * dk + e]);
                dvb[(long)j * dv + c] = acc;
            }
        }
        free(o);
        free(den);
        free(Gp);
        free(Sp);
    }
}

/*
 * Gradient of the non-causal form (blog digest "Method / key components 2)";
 * velog review sections 3.2 and 3.5).  The pages give no formula; this is the
 * exact gradient of out_i = num_i / den_i with num_i = phi(q_i)^T S and
 * den_i = phi(q_i) . z, S and z summed over all N tokens.  With the same
 * augmented vectors as the causal gradient, V'_j = [v_j, 1] and
 * G'_i = [g_i / den_i, -(g_i . out_i) / den_i]:
 *   S' = sum_j phi(k_j) V'_j^T,   dL/dphi(q_i) = S' G'_i
 *   R' = sum_i phi(q_i) G'_i^T,   dL/dphi(k_j) = R' V'_j,  dL/dv_j = R^T phi(k_j)
 * (R = the first dv columns of R'), then dq = dL/dphi(q) * phi'(q) and
 * dk = dL/dphi(k) * phi'(k).  The sums are full sums, not running ones.
 */
void oracle_bwd_noncausal_f64(const double *q, const double *k, const double *v,
                              const double *g, double *dq, double *dk_out, double *dv_out,
                              int B, int H, int N, int dk, int dv)
{
    long BH = (long)B * H;
    int dv1 = dv + 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        const double *qb = q + bh * (long)N * dk;
        const double *kb = k + bh * (long)N * dk;
        const double *vb = v + bh * (long)N * dv;
        const double *gb = g + bh * (long)N * dv;
        double *dqb = dq + bh * (long)N * dk;
        double *dkb = dk_out + bh * (long)N * dk;
        double *dvb = dv_out + bh * (long)N * dv;
        double *Sp = calloc((size_t)dk * dv1, sizeof(double)); /* S' */
        double *Rp = calloc((size_t)dk * dv1, sizeof(double)); /* R' */
        double *Gi = malloc((size_t)dv1 * sizeof(double));      /* G'_i */

        /* S' over all tokens. */
        for (int j = 0; j < N; ++j) {
            for (int e = 0; e < dk; ++e) {
                double fk = phi(kb[(long)j * dk + e]);
                for (int c = 0; c < dv; ++c) Sp[(long)e * dv1 + c] += fk * vb[(long)j * dv + c];
                Sp[(long)e * dv1 + dv] += fk;
            }
        }
        /* Per query: den_i, out_i, G'_i; dq_i = (S' G'_i) * phi'(q_i); R' += phi(q_i) G'_i^T. */
        for (int i = 0; i < N; ++i) {
            double d = 0.0;
            for (int e = 0; e < dk; ++e) d += phi(qb[(long)i * dk + e]) * Sp[(long)e * dv1 + dv];
            double go = 0.0;
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int e = 0; e < dk; ++e) num += phi(qb[(long)i * dk + e]) * Sp[(long)e * dv1 + c];
                go += gb[(long)i * dv + c] * (num / d);
                Gi[c] = gb[(long)i * dv + c] / d;
            }
            Gi[dv] = -go / d;
            for (int e = 0; e < dk; ++e) {
                double acc = 0.0;
                for (int c = 0; c < dv1; ++c) acc += Sp[(long)e * dv1 + c] * Gi[c];
                dqb[(long)i * dk + e] = acc * dphi(qb[(long)i * dk + e]);
                double fq = phi(qb[(long)i * dk + e]);
                for (int c = 0; c < dv1; ++c) Rp[(long)e * dv1 + c] += fq * Gi[c];
            }
        }
        /* Per key: dk_j = (R' V'_j) * phi'(k_j), dv_j = R^T phi(k_j). */
        for (int j = 0; j < N; ++j) {
            for (int e = 0; e < dk; ++e) {
                double acc = Rp[(long)e * dv1 + dv]; /* times V'_j[dv] = 1 */
                for (int c = 0; c < dv; ++c) acc += Rp[(long)e * dv1 + c] * vb[(long)j * dv + c];
                dkb[(long)j * dk + e] = acc * dphi(kb[(long)j * dk + e]);
            }
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int e = 0; e < dk; ++e) acc += Rp[(long)e * dv1 + c] * phi(kb[(long)j * dk + e]);
                dvb[(long)j * dv + c] = acc;
            }
        }
        free(Sp);
        free(Rp);
        free(Gi);
    }
}

/*
 * Causal forward with a fixed per-head decay gamma (the itwiki article's table
 * of later variants, RetNet row: S_t = gamma S_{t-1} + ...).  The feature map
 * and the normaliser of the base method are kept, and both running sums decay:
 *   S_i = gamma_h S_{i-1} + phi(k_i) v_i^T,   z_i = gamma_h z_{i-1} + phi(k_i),
 *   out_i = phi(q_i)^T S_i / phi(q_i) . z_i,
 * with gamma_h = gamma[h] for head h of the (b, h) pair.  gamma = 1 is the
 * causal form above.  `den` may be NULL.
 */
void oracle_fwd_causal_decay_f64(const double *q, const double *k, const double *v, const double *gamma,
                                 double *o, double *den, int B, int H, int N, int dk, int dv)
{
    long BH = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        const double g = gamma[bh % H];
        const double *qb = q + bh * (long)N * dk;
        const double *kb = k + bh * (long)N * dk;
        const double *vb = v + bh * (long)N * dv;
        double *ob = o + bh * (long)N * dv;
        double *S = calloc((size_t)dk * dv, sizeof(double));
        double *z = calloc((size_t)dk, sizeof(double));
        double *fq = malloc((size_t)dk * sizeof(double));
        for (int i = 0; i < N; ++i) {
            const double *ki = kb + (long)i * dk;
            const double *vi = vb + (long)i * dv;
            const double *qi = qb + (long)i * dk;
            for (int e = 0; e < dk; ++e) {
                double fk = phi(ki[e]);
                z[e] = g * z[e] + fk;
                for (int c = 0; c < dv; ++c) S[(long)e * dv + c] = g * S[(long)e * dv + c] + fk * vi[c];
            }
            double d = 0.0;
            for (int e = 0; e < dk; ++e) {
                fq[e] = phi(qi[e]);
                d += fq[e] * z[e];
            }
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int e = 0; e < dk; ++e) num += fq[e] * S[(long)e * dv + c];
                ob[(long)i * dv + c] = num / d;
            }
            if (den) den[bh * (long)N + i] = d;
        }
        free(S);
        free(z);
        free(fq);
    }
}

/*
 * One decode step with the per-head decay: S = gamma_h S + phi(k) v^T,
 * z = gamma_h z + phi(k), then out = phi(q)^T S / phi(q) . z.
 */
void oracle_decode_step_decay_f64(double *S, double *z, const double *q, const double *k,
                                  const double *v, const double *gamma, double *o,
                                  int B, int H, int dk, int dv)
{
    long BH = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < BH; ++bh) {
        const double g = gamma[bh % H];
        double *Sb = S + bh * (long)dk * dv;
        double *zb = z + bh * (long)dk;
        const double *qb = q + bh * (long)dk;
        const double *kb = k + bh * (long)dk;
        const double *vb = v + bh * (long)dv;
        double *ob = o + bh * (long)dv;
        for (int e = 0; e < dk; ++e) {
            double fk = phi(kb[e]);
            zb[e] = g * zb[e] + fk;
            for (int c = 0; c < dv; ++c) Sb[(long)e * dv + c] = g * Sb[(long)e * dv + c] + fk * vb[c];
        }
        double d = 0.0;
        for (int e = 0; e < dk; ++e) d += phi(qb[e]) * zb[e];
        for (int c = 0; c < dv; ++c) {
            double num = 0.0;
            for (int e = 0; e < dk; ++e) num += phi(qb[e]) * Sb[(long)e * dv + c];
            ob[c] = num / d;
        }
    }
}

/*
 * Gradient of the causal form with the per-head decay (the itwiki variants
 * table, RetNet row; the pages print no gradient).  It is the cumulative-sum
 * gradient above with both running sums decayed by gamma_h per token:
 *   S'_i = gamma S'_{i-1} + phi(k_i) V'_i^T      dL/dphi(q_i) = S'_i G'_i
 *   R'_j = gamma R'_{j+1} + phi(q_j) G'_j^T      dL/dphi(k_j) = R'_j V'_j,
 *                                                dL/dv_j = R_j^T phi(k_j),
 * with V'_j = [v_j, 1], G'_i = [g_i / den_i, -(g_i . out_i) / den_i] and the
 * decayed den_i, out_i of oracle_fwd_causal_decay_f64; then the chain rule
 * through phi.  gamma = 1 is oracle_bwd_causal_f64.
 */
void oracle_bwd_causal_decay_f64(const double *q, const double *k, const double *v, const double *g,
                                 const double *gamma, double *dq, double *dk_out, double *dv_out,
                                 int B, int H, int N, int dk, int dv)
{
    long BH = (long)B * H;
    int dv1 = dv + 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        const double gm = gamma[bh % H];
        const double *qb = q + bh * (long)N * dk;
        const double *kb = k + bh * (long)N * dk;
        const double *vb = v + bh * (long)N * dv;
        const double *gb = g + bh * (long)N * dv;
        double *dqb = dq + bh * (long)N * dk;
        double *dkb = dk_out + bh * (long)N * dk;
        double *dvb = dv_out + bh * (long)N * dv;
        double *Gp = malloc((size_t)N * dv1 * sizeof(double));
        double *Sp = calloc((size_t)dk * dv1, sizeof(double));

        /* Forward sweep: decayed S', out_i and den_i, G'_i, then dq_i = (S'_i G'_i) phi'(q_i). */
        for (int i = 0; i < N; ++i) {
            for (int e = 0; e < dk; ++e) {
                double fk = phi(kb[(long)i * dk + e]);
                for (int c = 0; c < dv; ++c)
                    Sp[(long)e * dv1 + c] = gm * Sp[(long)e * dv1 + c] + fk * vb[(long)i * dv + c];
                Sp[(long)e * dv1 + dv] = gm * Sp[(long)e * dv1 + dv] + fk;
            }
            double d = 0.0;
            for (int e = 0; e < dk; ++e) d += phi(qb[(long)i * dk + e]) * Sp[(long)e * dv1 + dv];
            double go = 0.0;
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int e = 0; e < dk; ++e) num += phi(qb[(long)i * dk + e]) * Sp[(long)e * dv1 + c];
                go += gb[(long)i * dv + c] * (num / d);
                Gp[(long)i * dv1 + c] = gb[(long)i * dv + c] / d;
            }
            Gp[(long)i * dv1 + dv] = -go / d;
            for (int e = 0; e < dk; ++e) {
                double acc = 0.0;
                for (int c = 0; c < dv1; ++c) acc += Sp[(long)e * dv1 + c] * Gp[(long)i * dv1 + c];
                dqb[(long)i * dk + e] = acc * dphi(qb[(long)i * dk + e]);
            }
        }

        /* Reverse sweep: decayed R', then dk_j and dv_j. */
        memset(Sp, 0, (size_t)dk * dv1 * sizeof(double));
        for (int j = N - 1; j >= 0; --j) {
            for (int e = 0; e < dk; ++e) {
                double fq = phi(qb[(long)j * dk + e]);
                for (int c = 0; c < dv1; ++c)
                    Sp[(long)e * dv1 + c] = gm * Sp[(long)e * dv1 + c] + fq * Gp[(long)j * dv1 + c];
            }
            for (int e = 0; e < dk; ++e) {
                double acc = Sp[(long)e * dv1 + dv]; /* times V'_j[dv] = 1 */
                for (int c = 0; c < dv; ++c) acc += Sp[(long)e * dv1 + c] * vb[(long)j * dv + c];
                dkb[(long)j * dk + e] = acc * dphi(kb[(long)j * dk + e]);
            }
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int e = 0; e < dk; ++e) acc += Sp[(long)e * dv1 + c] * phi(kb[(long)j * dk + e]);
                dvb[(long)j * dv + c] = acc;
            }
        }
        free(Gp);
        free(Sp);
    }
}

/*
 * ---------------------------------------------------------------------------
 * Pluggable feature map (itwiki "선형 어텐션", section "특징 사상 선택"
 * (choice of feature map), which lists elu + 1, Performer's positive
 * orthogonal random features and the identity; blog digest "Digest" (open
 * questions: better feature maps such as Performer's random features)).
 *
 * kind 0, elu + 1:  phi(x) = elu(x) + 1 as above, m = dk.
 * kind 1, identity: phi(x) = x, m = dk (the caller supplies features that
 *                   keep the denominators positive).
 * kind 2, positive random features approximating the softmax kernel
 *                   exp(q . k) without bias:
 *                   phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(m),  r < m,
 *                   with w_r the r-th of m random directions of dimension dk,
 *                   W[h][r][e] for head h (drawn by the caller).
 *                   Then E_w[phi(q) . phi(k)] = exp(q . k) for w ~ N(0, I).
 * The attention itself is unchanged: the state has m rows instead of dk.
 * ---------------------------------------------------------------------------
 */
static void fm_feature(int kind, const double *Wh, int m, const double *x, int dk, double *out)
{
    if (kind == 0) {
        for (int e = 0; e < dk; ++e) out[e] = phi(x[e]);
    } else if (kind == 1) {
        for (int e = 0; e < dk; ++e) out[e] = x[e];
    } else {
        double nx = 0.0;
        for (int e = 0; e < dk; ++e) nx += x[e] * x[e];
        for (int r = 0; r < m; ++r) {
            double a = 0.0;
            for (int e = 0; e < dk; ++e) a += Wh[(long)r * dk + e] * x[e];
            out[r] = exp(a - 0.5 * nx) / sqrt((double)m);
        }
    }
}

/* dx = J^T dphi, J the Jacobian of the feature map at x:
 * elu + 1: diag(phi'(x)); identity: I; random features:
 * d phi_r / d x_e = phi_r(x) (w_re - x_e). */
static void fm_feature_vjp(int kind, const double *Wh, int m, const double *x, int dk, const double *dphi_in,
                           double *dx)
{
    if (kind == 0) {
        for (int e = 0; e < dk; ++e) dx[e] = dphi_in[e] * dphi(x[e]);
    } else if (kind == 1) {
        for (int e = 0; e < dk; ++e) dx[e] = dphi_in[e];
    } else {
        double *f = malloc((size_t)m * sizeof(double));
        fm_feature(kind, Wh, m, x, dk, f);
        for (int e = 0; e < dk; ++e) dx[e] = 0.0;
        for (int r = 0; r < m; ++r) {
            double u = dphi_in[r] * f[r];
            for (int e = 0; e < dk; ++e) dx[e] += u * (Wh[(long)r * dk + e] - x[e]);
        }
        free(f);
    }
}

/* Feature dimension of a map (m for random features, dk otherwise). */
static int fm_dim(int kind, int m, int dk) { return kind == 2 ? m : dk; }

/* The feature map alone: phi of every row of x [B][H][N][dk] into out [B][H][N][m']. */
void oracle_fm_features_f64(const double *x, int kind, const double *W, int m, double *out,
                            int B, int H, int N, int dk)
{
    long BH = (long)B * H;
    int mf = fm_dim(kind, m, dk);
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < BH; ++bh) {
        const double *Wh = kind == 2 ? W + (bh % H) * (long)m * dk : NULL;
        for (int i = 0; i < N; ++i)
            fm_feature(kind, Wh, m, x + (bh * N + i) * (long)dk, dk, out + (bh * N + i) * (long)mf);
    }
}

/* Causal forward with a feature map: the recurrent form of
 * oracle_fwd_causal_f64 with phi replaced by the map (state S [m'][dv]). */
void oracle_fwd_causal_fm_f64(const double *q, const double *k, const double *v, int kind, const double *W,
                              int m, double *o, double *den, int B, int H, int N, int dk, int dv)
{
    long BH = (long)B * H;
    int mf = fm_dim(kind, m, dk);
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        const double *Wh = kind == 2 ? W + (bh % H) * (long)m * dk : NULL;
        double *S = calloc((size_t)mf * dv, sizeof(double));
        double *z = calloc((size_t)mf, sizeof(double));
        double *fq = malloc((size_t)mf * sizeof(double));
        double *fk = malloc((size_t)mf * sizeof(double));
        for (int i = 0; i < N; ++i) {
            const double *vi = v + (bh * N + i) * (long)dv;
            fm_feature(kind, Wh, m, k + (bh * N + i) * (long)dk, dk, fk);
            for (int e = 0; e < mf; ++e) {
                z[e] += fk[e];
                for (int c = 0; c < dv; ++c) S[(long)e * dv + c] += fk[e] * vi[c];
            }
            fm_feature(kind, Wh, m, q + (bh * N + i) * (long)dk, dk, fq);
            double d = 0.0;
            for (int e = 0; e < mf; ++e) d += fq[e] * z[e];
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int e = 0; e < mf; ++e) num += fq[e] * S[(long)e * dv + c];
                o[(bh * N + i) * (long)dv + c] = num / d;
            }
            if (den) den[bh * (long)N + i] = d;
        }
        free(S);
        free(z);
        free(fq);
        free(fk);
    }
}

/* Non-causal forward with a feature map (sums over all N tokens). */
void oracle_fwd_noncausal_fm_f64(const double *q, const double *k, const double *v, int kind, const double *W,
                                 int m, double *o, int B, int H, int N, int dk, int dv)
{
    long BH = (long)B * H;
    int mf = fm_dim(kind, m, dk);
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        const double *Wh = kind == 2 ? W + (bh % H) * (long)m * dk : NULL;
        double *S = calloc((size_t)mf * dv, sizeof(double));
        double *z = calloc((size_t)mf, sizeof(double));
        double *f = malloc((size_t)mf * sizeof(double));
        for (int j = 0; j < N; ++j) {
            fm_feature(kind, Wh, m, k + (bh * N + j) * (long)dk, dk, f);
            for (int e = 0; e < mf; ++e) {
                z[e] += f[e];
                for (int c = 0; c < dv; ++c) S[(long)e * dv + c] += f[e] * v[(bh * N + j) * (long)dv + c];
            }
        }
        for (int i = 0; i < N; ++i) {
            fm_feature(kind, Wh, m, q + (bh * N + i) * (long)dk, dk, f);
            double d = 0.0;
            for (int e = 0; e < mf; ++e) d += f[e] * z[e];
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int e = 0; e < mf; ++e) num += f[e] * S[(long)e * dv + c];
                o[(bh * N + i) * (long)dv + c] = num / d;
            }
        }
        free(S);
        free(z);
        free(f);
    }
}

/* One decode step with a feature map: S [B][H][m'][dv], z [B][H][m'] in place. */
void oracle_decode_step_fm_f64(double *S, double *z, const double *q, const double *k, const double *v, int kind,
                               const double *W, int m, double *o, int B, int H, int dk, int dv)
{
    long BH = (long)B * H;
    int mf = fm_dim(kind, m, dk);
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < BH; ++bh) {
        const double *Wh = kind == 2 ? W + (bh % H) * (long)m * dk : NULL;
        double *Sb = S + bh * (long)mf * dv;
        double *zb = z + bh * (long)mf;
        double *fq = malloc((size_t)mf * sizeof(double));
        double *fk = malloc((size_t)mf * sizeof(double));
        fm_feature(kind, Wh, m, k + bh * (long)dk, dk, fk);
        fm_feature(kind, Wh, m, q + bh * (long)dk, dk, fq);
        for (int e = 0; e < mf; ++e) {
            zb[e] += fk[e];
            for (int c = 0; c < dv; ++c) Sb[(long)e * dv + c] += fk[e] * v[bh * (long)dv + c];
        }
        double d = 0.0;
        for (int e = 0; e < mf; ++e) d += fq[e] * zb[e];
        for (int c = 0; c < dv; ++c) {
            double num = 0.0;
            for (int e = 0; e < mf; ++e) num += fq[e] * Sb[(long)e * dv + c];
            o[bh * (long)dv + c] = num / d;
        }
        free(fq);
        free(fk);
    }
}

/*
 * Gradient of the causal form with a feature map: the cumulative-sum gradient
 * of oracle_bwd_causal_f64 taken with respect to the features, phi_q = phi(q_i)
 * and phi_k = phi(k_j), then carried back through the map (fm_feature_vjp).
 */
void oracle_bwd_causal_fm_f64(const double *q, const double *k, const double *v, const double *g, int kind,
                              const double *W, int m, double *dq, double *dk_out, double *dv_out,
                              int B, int H, int N, int dk, int dv)
{
    long BH = (long)B * H;
    int dv1 = dv + 1;
    int mf = fm_dim(kind, m, dk);
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < BH; ++bh) {
        const double *Wh = kind == 2 ? W + (bh % H) * (long)m * dk : NULL;
        const double *qb = q + bh * (long)N * dk;
        const double *kb = k + bh * (long)N * dk;
        const double *vb = v + bh * (long)N * dv;
        const double *gb = g + bh * (long)N * dv;
        double *FQ = malloc((size_t)N * mf * sizeof(double));
        double *FK = malloc((size_t)N * mf * sizeof(double));
        double *Gp = malloc((size_t)N * dv1 * sizeof(double));
        double *Sp = calloc((size_t)mf * dv1, sizeof(double));
        double *df = malloc((size_t)mf * sizeof(double));
        for (int i = 0; i < N; ++i) {
            fm_feature(kind, Wh, m, qb + (long)i * dk, dk, FQ + (long)i * mf);
            fm_feature(kind, Wh, m, kb + (long)i * dk, dk, FK + (long)i * mf);
        }
        /* Forward sweep: S'_i, out_i and den_i, G'_i, then dphi_q(i) = S'_i G'_i. */
        for (int i = 0; i < N; ++i) {
            const double *fk = FK + (long)i * mf, *fq = FQ + (long)i * mf;
            for (int e = 0; e < mf; ++e) {
                for (int c = 0; c < dv; ++c) Sp[(long)e * dv1 + c] += fk[e] * vb[(long)i * dv + c];
                Sp[(long)e * dv1 + dv] += fk[e];
            }
            double d = 0.0;
            for (int e = 0; e < mf; ++e) d += fq[e] * Sp[(long)e * dv1 + dv];
            double go = 0.0;
            for (int c = 0; c < dv; ++c) {
                double num = 0.0;
                for (int e = 0; e < mf; ++e) num += fq[e] * Sp[(long)e * dv1 + c];
                go += gb[(long)i * dv + c] * (num / d);
                Gp[(long)i * dv1 + c] = gb[(long)i * dv + c] / d;
            }
            Gp[(long)i * dv1 + dv] = -go / d;
            for (int e = 0; e < mf; ++e) {
                double acc = 0.0;
                for (int c = 0; c < dv1; ++c) acc += Sp[(long)e * dv1 + c] * Gp[(long)i * dv1 + c];
                df[e] = acc;
            }
            fm_feature_vjp(kind, Wh, m, qb + (long)i * dk, dk, df, dq + (bh * N + i) * (long)dk);
        }
        /* Reverse sweep: R'_j, then dphi_k(j) = R'_j V'_j and dv_j = R_j^T phi_k(j). */
        memset(Sp, 0, (size_t)mf * dv1 * sizeof(double));
        for (int j = N - 1; j >= 0; --j) {
            const double *fk = FK + (long)j * mf, *fq = FQ + (long)j * mf;
            for (int e = 0; e < mf; ++e)
                for (int c = 0; c < dv1; ++c) Sp[(long)e * dv1 + c] += fq[e] * Gp[(long)j * dv1 + c];
            for (int e = 0; e < mf; ++e) {
                double acc = Sp[(long)e * dv1 + dv];
                for (int c = 0; c < dv; ++c) acc += Sp[(long)e * dv1 + c] * vb[(long)j * dv + c];
                df[e] = acc;
            }
            fm_feature_vjp(kind, Wh, m, kb + (long)j * dk, dk, df, dk_out + (bh * N + j) * (long)dk);
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int e = 0; e < mf; ++e) acc += Sp[(long)e * dv1 + c] * fk[e];
                dv_out[(bh * N + j) * (long)dv + c] = acc;
            }
        }
        free(FQ);
        free(FK);
        free(Gp);
        free(Sp);
        free(df);
    }
}
