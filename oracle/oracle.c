/*
 * oracle.c -- plain fp64 CPU oracle of the causal dot product of linear
 * attention.  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * CPU-baseline leg of the benchmark call it; the product library never links,
 * loads or calls anything here, and nothing here is shared with the HIP code.
 *
 * Method.  The opening post of "Dot Product Computes Wrong Values"
 * (github.com/triton-lang/triton issue 217) names the computation: the causal
 * dot product of "Transformers are RNNs" (Algorithm 1), a batch-parallel O(n)
 * for-loop computing a prefix sum.  Per (n, h) slice, with q_i, k_i in R^E and
 * v_i in R^M:
 *     S_i   = S_{i-1} + k_i v_i^T          (E x M running state, S_{-1} = 0)
 *     out_i = q_i^T S_i                    (M-vector)
 * The later comment on the same page with the author's loop excerpt adds the
 * current row to the state before the output row is read, so the sum is
 * inclusive: out_i = sum_{j<=i} (q_i . k_j) v_j.
 *
 * The normalised form (linear attention proper) divides by
 *     den_i = phi(q_i) . z_i + eps,   z_i = sum_{j<=i} phi(k_j),
 * with phi = elu + 1 (alpha = 1): phi(x) = x + 1 for x > 0, exp(x) otherwise.
 *
 * Carried state.  A slice may start from a given state instead of zero:
 * S_{-1} = S0 (and z_{-1} = z0 in the normalised form), so that a sequence can
 * be processed in segments, each starting from the final state of the one
 * before (the loop of the opening post keeps that state explicitly).  Then
 * out_i = q_i^T (S0 + sum_{j<=i} k_j v_j^T), and the gradient of
 * f = sum_i out_i . dO_i with respect to S0 is sum_i q_i dO_i^T.  S0, z0 are
 * [NH][E][M] and [NH][E] floats; NULL means zero.  Final states are written
 * to [NH][E][M] (and [NH][E]) double arrays when the pointer is not NULL.
 *
 * Layout: Q, K are [NH][L][E] and V, dO are [NH][L][M], row-major, contiguous,
 * given as float (fp32 values, or bf16 values widened exactly to fp32).  All
 * arithmetic is double precision.  Outputs are double arrays of the same
 * shapes.  Every function loops over the NH slices independently (OpenMP over
 * slices); within a slice the loops are the plain definitions below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* phi = elu + 1 with alpha = 1 (the feature map of linear attention). */
static double phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* ---------------------------------------------------------------------------
 * Forward, O(L E M) recurrence: S += k_i v_i^T, then out_i = q_i^T S.
 * ------------------------------------------------------------------------- */
void oracle_fwd(const float *Q, const float *K, const float *V, const float *S0, double *Out,
                double *Sfin, int64_t NH, int64_t L, int64_t E, int64_t M) {
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < NH; ++s) {
        const float *q = Q + s * L * E, *k = K + s * L * E, *v = V + s * L * M;
        double *out = Out + s * L * M;
        double *S = (double *)calloc((size_t)(E * M), sizeof(double));
        if (S0)
            for (int64_t x = 0; x < E * M; ++x) S[x] = (double)S0[s * E * M + x];
        for (int64_t i = 0; i < L; ++i) {
            for (int64_t e = 0; e < E; ++e)
                for (int64_t m = 0; m < M; ++m)
                    S[e * M + m] += (double)k[i * E + e] * (double)v[i * M + m];
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t e = 0; e < E; ++e) acc += (double)q[i * E + e] * S[e * M + m];
                out[i * M + m] = acc;
            }
        }
        if (Sfin) memcpy(Sfin + s * E * M, S, (size_t)(E * M) * sizeof(double));
        free(S);
    }
}

/* ---------------------------------------------------------------------------
 * Forward, O(L^2 (E + M)) masked brute force:
 *   out_i = q_i^T S0 + sum_{j<=i} (q_i.k_j) v_j.
 * ------------------------------------------------------------------------- */
void oracle_fwd_brute(const float *Q, const float *K, const float *V, const float *S0, double *Out,
                      int64_t NH, int64_t L, int64_t E, int64_t M) {
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < NH; ++s) {
        const float *q = Q + s * L * E, *k = K + s * L * E, *v = V + s * L * M;
        double *out = Out + s * L * M;
        for (int64_t i = 0; i < L; ++i) {
            for (int64_t m = 0; m < M; ++m) {
                double c = 0.0;
                if (S0)
                    for (int64_t e = 0; e < E; ++e) c += (double)q[i * E + e] * (double)S0[s * E * M + e * M + m];
                out[i * M + m] = c;
            }
            for (int64_t j = 0; j <= i; ++j) {
                double a = 0.0;
                for (int64_t e = 0; e < E; ++e) a += (double)q[i * E + e] * (double)k[j * E + e];
                for (int64_t m = 0; m < M; ++m) out[i * M + m] += a * (double)v[j * M + m];
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Normalised forward, recurrence.  feature_map = 1 applies phi to the raw Q, K
 * values; feature_map = 0 uses Q, K as given.
 *   S += phi(k_i) v_i^T;  z += phi(k_i);
 *   out_i = (phi(q_i)^T S) / (phi(q_i) . z + eps)
 * ------------------------------------------------------------------------- */
void oracle_linattn(const float *Q, const float *K, const float *V, const float *S0, const float *z0,
                    double *Out, double *Sfin, double *zfin, int64_t NH, int64_t L, int64_t E, int64_t M,
                    double eps, int feature_map) {
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < NH; ++s) {
        const float *q = Q + s * L * E, *k = K + s * L * E, *v = V + s * L * M;
        double *out = Out + s * L * M;
        double *S = (double *)calloc((size_t)(E * M), sizeof(double));
        double *z = (double *)calloc((size_t)E, sizeof(double));
        if (S0)
            for (int64_t x = 0; x < E * M; ++x) S[x] = (double)S0[s * E * M + x];
        if (z0)
            for (int64_t e = 0; e < E; ++e) z[e] = (double)z0[s * E + e];
        double *fq = (double *)malloc((size_t)E * sizeof(double));
        double *fk = (double *)malloc((size_t)E * sizeof(double));
        for (int64_t i = 0; i < L; ++i) {
            for (int64_t e = 0; e < E; ++e) {
                fq[e] = feature_map ? phi((double)q[i * E + e]) : (double)q[i * E + e];
                fk[e] = feature_map ? phi((double)k[i * E + e]) : (double)k[i * E + e];
            }
            for (int64_t e = 0; e < E; ++e) {
                z[e] += fk[e];
                for (int64_t m = 0; m < M; ++m) S[e * M + m] += fk[e] * (double)v[i * M + m];
            }
            double den = eps;
            for (int64_t e = 0; e < E; ++e) den += fq[e] * z[e];
            for (int64_t m = 0; m < M; ++m) {
                double num = 0.0;
                for (int64_t e = 0; e < E; ++e) num += fq[e] * S[e * M + m];
                out[i * M + m] = num / den;
            }
        }
        if (Sfin) memcpy(Sfin + s * E * M, S, (size_t)(E * M) * sizeof(double));
        if (zfin) memcpy(zfin + s * E, z, (size_t)E * sizeof(double));
        free(S); free(z); free(fq); free(fk);
    }
}

/* ---------------------------------------------------------------------------
 * Normalised forward, brute force, with c_i = phi(q_i):
 *   out_i = (c_i^T S0 + sum_{j<=i} a_ij v_j) / (c_i . z0 + sum_{j<=i} a_ij + eps),
 *   a_ij = c_i . phi(k_j)
 * ------------------------------------------------------------------------- */
void oracle_linattn_brute(const float *Q, const float *K, const float *V, const float *S0, const float *z0,
                          double *Out, int64_t NH, int64_t L, int64_t E, int64_t M, double eps,
                          int feature_map) {
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < NH; ++s) {
        const float *q = Q + s * L * E, *k = K + s * L * E, *v = V + s * L * M;
        double *out = Out + s * L * M;
        for (int64_t i = 0; i < L; ++i) {
            double den = eps;
            for (int64_t m = 0; m < M; ++m) out[i * M + m] = 0.0;
            for (int64_t e = 0; e < E; ++e) {
                const double c = feature_map ? phi((double)q[i * E + e]) : (double)q[i * E + e];
                if (z0) den += c * (double)z0[s * E + e];
                if (S0)
                    for (int64_t m = 0; m < M; ++m) out[i * M + m] += c * (double)S0[s * E * M + e * M + m];
            }
            for (int64_t j = 0; j <= i; ++j) {
                double a = 0.0;
                for (int64_t e = 0; e < E; ++e) {
                    double fq = feature_map ? phi((double)q[i * E + e]) : (double)q[i * E + e];
                    double fk = feature_map ? phi((double)k[j * E + e]) : (double)k[j * E + e];
                    a += fq * fk;
                }
                den += a;
                for (int64_t m = 0; m < M; ++m) out[i * M + m] += a * (double)v[j * M + m];
            }
            for (int64_t m = 0; m < M; ++m) out[i * M + m] /= den;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Backward of out = causal_product(Q, K, V) (from state S0) for an upstream
 * gradient dO, i.e. the gradient of
 *   f = sum_i [ q_i^T S0 dO_i + sum_{j<=i} (q_i.k_j)(v_j.dO_i) ].
 * Forward sweep:  S = S0;  S += k_i v_i^T;  dq_i = S dO_i.
 * Reverse sweep:  R += q_i dO_i^T (i descending);  dk_i = R v_i;  dv_i = R^T k_i.
 * The gradient of S0 is the final R (sum of all q_i dO_i^T), written to dS0
 * when it is not NULL.
 * ------------------------------------------------------------------------- */
void oracle_bwd(const float *Q, const float *K, const float *V, const float *dO, const float *S0,
                double *dQ, double *dK, double *dV, double *dS0,
                int64_t NH, int64_t L, int64_t E, int64_t M) {
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < NH; ++s) {
        const float *q = Q + s * L * E, *k = K + s * L * E, *v = V + s * L * M;
        const float *go = dO + s * L * M;
        double *dq = dQ + s * L * E, *dk = dK + s * L * E, *dv = dV + s * L * M;
        double *S = (double *)calloc((size_t)(E * M), sizeof(double));
        if (S0)
            for (int64_t x = 0; x < E * M; ++x) S[x] = (double)S0[s * E * M + x];
        for (int64_t i = 0; i < L; ++i) {
            for (int64_t e = 0; e < E; ++e)
                for (int64_t m = 0; m < M; ++m)
                    S[e * M + m] += (double)k[i * E + e] * (double)v[i * M + m];
            for (int64_t e = 0; e < E; ++e) {
                double acc = 0.0;
                for (int64_t m = 0; m < M; ++m) acc += S[e * M + m] * (double)go[i * M + m];
                dq[i * E + e] = acc;
            }
        }
        memset(S, 0, (size_t)(E * M) * sizeof(double));
        double *R = S;
        for (int64_t i = L - 1; i >= 0; --i) {
            for (int64_t e = 0; e < E; ++e)
                for (int64_t m = 0; m < M; ++m)
                    R[e * M + m] += (double)q[i * E + e] * (double)go[i * M + m];
            for (int64_t e = 0; e < E; ++e) {
                double acc = 0.0;
                for (int64_t m = 0; m < M; ++m) acc += R[e * M + m] * (double)v[i * M + m];
                dk[i * E + e] = acc;
            }
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t e = 0; e < E; ++e) acc += R[e * M + m] * (double)k[i * E + e];
                dv[i * M + m] = acc;
            }
        }
        if (dS0) memcpy(dS0 + s * E * M, R, (size_t)(E * M) * sizeof(double));
        free(S);
    }
}

/* ---------------------------------------------------------------------------
 * Backward, brute force from
 *   f = sum_i [ q_i^T S0 dO_i + sum_{j<=i} (q_i.k_j)(v_j.dO_i) ]:
 *   dq_i = S0 dO_i + sum_{j<=i} (dO_i.v_j) k_j
 *   dk_j = sum_{i>=j} (dO_i.v_j) q_i
 *   dv_j = sum_{i>=j} (q_i.k_j) dO_i
 *   dS0[e][m] = sum_i q_i[e] dO_i[m]
 * ------------------------------------------------------------------------- */
void oracle_bwd_brute(const float *Q, const float *K, const float *V, const float *dO, const float *S0,
                      double *dQ, double *dK, double *dV, double *dS0,
                      int64_t NH, int64_t L, int64_t E, int64_t M) {
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < NH; ++s) {
        const float *q = Q + s * L * E, *k = K + s * L * E, *v = V + s * L * M;
        const float *go = dO + s * L * M;
        double *dq = dQ + s * L * E, *dk = dK + s * L * E, *dv = dV + s * L * M;
        for (int64_t x = 0; x < L * E; ++x) { dq[x] = 0.0; dk[x] = 0.0; }
        for (int64_t x = 0; x < L * M; ++x) dv[x] = 0.0;
        for (int64_t i = 0; i < L; ++i) {
            for (int64_t e = 0; e < E; ++e) {
                double c = 0.0;
                if (S0)
                    for (int64_t m = 0; m < M; ++m) c += (double)S0[s * E * M + e * M + m] * (double)go[i * M + m];
                dq[i * E + e] = c;
            }
            if (dS0) {
                double *g0 = dS0 + s * E * M;
                if (i == 0)
                    for (int64_t x = 0; x < E * M; ++x) g0[x] = 0.0;
                for (int64_t e = 0; e < E; ++e)
                    for (int64_t m = 0; m < M; ++m) g0[e * M + m] += (double)q[i * E + e] * (double)go[i * M + m];
            }
            for (int64_t j = 0; j <= i; ++j) {
                double gv = 0.0, qk = 0.0;
                for (int64_t m = 0; m < M; ++m) gv += (double)go[i * M + m] * (double)v[j * M + m];
                for (int64_t e = 0; e < E; ++e) qk += (double)q[i * E + e] * (double)k[j * E + e];
                for (int64_t e = 0; e < E; ++e) {
                    dq[i * E + e] += gv * (double)k[j * E + e];
                    dk[j * E + e] += gv * (double)q[i * E + e];
                }
                for (int64_t m = 0; m < M; ++m) dv[j * M + m] += qk * (double)go[i * M + m];
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Backward of the normalised form out_i = n_i / d_i (from S0, z0) for an
 * upstream gradient dO, with c_i = phi(q_i), f_j = phi(k_j):
 *   n_i = c_i^T S_i,  S_i = S0 + sum_{j<=i} f_j v_j^T,
 *   d_i = c_i . z_i + eps,  z_i = z0 + sum_{j<=i} f_j.
 * The quotient rule gives the gradients of n_i and d_i,
 *   dn_i = dO_i / d_i,   dd_i = -(dO_i . n_i) / d_i^2,
 * and through the two prefix sums
 *   dc_i = S_i dn_i + dd_i z_i,
 *   df_j = R_j v_j + r_j,   R_j = sum_{i>=j} c_i dn_i^T,  r_j = sum_{i>=j} dd_i c_i,
 *   dv_j = R_j^T f_j,
 *   dS0 = R_0,  dz0 = r_0,
 * then through phi: dq = dc * phi'(q), dk = df * phi'(k), with phi' = 1 for
 * x > 0 and exp(x) otherwise (feature_map = 1), or 1 (feature_map = 0).
 * First a forward sweep (S_i, z_i, n_i, d_i, dc_i), then a reverse sweep.
 * Outputs dS0 [NH][E][M] and dz0 [NH][E] are written when not NULL.
 * ------------------------------------------------------------------------- */
static double dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }

void oracle_linattn_bwd(const float *Q, const float *K, const float *V, const float *dO, const float *S0,
                        const float *z0, double *dQ, double *dK, double *dV, double *dS0, double *dz0,
                        int64_t NH, int64_t L, int64_t E, int64_t M, double eps, int feature_map) {
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < NH; ++s) {
        const float *q = Q + s * L * E, *k = K + s * L * E, *v = V + s * L * M;
        const float *go = dO + s * L * M;
        double *dq = dQ + s * L * E, *dk = dK + s * L * E, *dv = dV + s * L * M;
        double *S = (double *)calloc((size_t)(E * M), sizeof(double));
        double *z = (double *)calloc((size_t)E, sizeof(double));
        double *c = (double *)malloc((size_t)(L * E) * sizeof(double));
        double *f = (double *)malloc((size_t)(L * E) * sizeof(double));
        double *dn = (double *)malloc((size_t)(L * M) * sizeof(double));
        double *dd = (double *)malloc((size_t)L * sizeof(double));
        if (S0)
            for (int64_t x = 0; x < E * M; ++x) S[x] = (double)S0[s * E * M + x];
        if (z0)
            for (int64_t e = 0; e < E; ++e) z[e] = (double)z0[s * E + e];
        for (int64_t x = 0; x < L * E; ++x) {
            c[x] = feature_map ? phi((double)q[x]) : (double)q[x];
            f[x] = feature_map ? phi((double)k[x]) : (double)k[x];
        }
        /* forward sweep */
        for (int64_t i = 0; i < L; ++i) {
            for (int64_t e = 0; e < E; ++e) {
                z[e] += f[i * E + e];
                for (int64_t m = 0; m < M; ++m) S[e * M + m] += f[i * E + e] * (double)v[i * M + m];
            }
            double den = eps;
            for (int64_t e = 0; e < E; ++e) den += c[i * E + e] * z[e];
            double gn = 0.0;  /* dO_i . n_i */
            for (int64_t m = 0; m < M; ++m) {
                double num = 0.0;
                for (int64_t e = 0; e < E; ++e) num += c[i * E + e] * S[e * M + m];
                gn += (double)go[i * M + m] * num;
                dn[i * M + m] = (double)go[i * M + m] / den;
            }
            dd[i] = -gn / (den * den);
            for (int64_t e = 0; e < E; ++e) {
                double acc = dd[i] * z[e];
                for (int64_t m = 0; m < M; ++m) acc += S[e * M + m] * dn[i * M + m];
                dq[i * E + e] = acc * (feature_map ? dphi((double)q[i * E + e]) : 1.0);
            }
        }
        /* reverse sweep */
        double *R = S, *r = z;
        memset(R, 0, (size_t)(E * M) * sizeof(double));
        memset(r, 0, (size_t)E * sizeof(double));
        for (int64_t i = L - 1; i >= 0; --i) {
            for (int64_t e = 0; e < E; ++e) {
                r[e] += dd[i] * c[i * E + e];
                for (int64_t m = 0; m < M; ++m) R[e * M + m] += c[i * E + e] * dn[i * M + m];
            }
            for (int64_t e = 0; e < E; ++e) {
                double acc = r[e];
                for (int64_t m = 0; m < M; ++m) acc += R[e * M + m] * (double)v[i * M + m];
                dk[i * E + e] = acc * (feature_map ? dphi((double)k[i * E + e]) : 1.0);
            }
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t e = 0; e < E; ++e) acc += R[e * M + m] * f[i * E + e];
                dv[i * M + m] = acc;
            }
        }
        if (dS0) memcpy(dS0 + s * E * M, R, (size_t)(E * M) * sizeof(double));
        if (dz0) memcpy(dz0 + s * E, r, (size_t)E * sizeof(double));
        free(S); free(z); free(c); free(f); free(dn); free(dd);
    }
}

/* Final running state S_{L-1} = sum_j k_j v_j^T of every slice, [NH][E][M]. */
void oracle_state(const float *K, const float *V, double *S_out,
                  int64_t NH, int64_t L, int64_t E, int64_t M) {
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < NH; ++s) {
        const float *k = K + s * L * E, *v = V + s * L * M;
        double *S = S_out + s * E * M;
        for (int64_t x = 0; x < E * M; ++x) S[x] = 0.0;
        for (int64_t j = 0; j < L; ++j)
            for (int64_t e = 0; e < E; ++e)
                for (int64_t m = 0; m < M; ++m)
                    S[e * M + m] += (double)k[j * E + e] * (double)v[j * M + m];
    }
}
