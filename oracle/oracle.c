/*
 * oracle.c -- float64 CPU oracle for the KL projection onto the Birkhoff
 * polytope, its implicit-differentiation backward pass and the fixed-sweep
 * Sinkhorn-Knopp baseline.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library.  The product path
 * (the HIP library and its Python binding) never calls, links or includes it,
 * and this file includes nothing from the product path.
 *
 * Sources (cited by title and section / equation only):
 *   [P]  "Accelerating Birkhoff Projection for Manifold-Constrained
 *        Hyper-Connections", sections 2.2-4.2, equations (1)-(13).
 *   [B]  the author's blog post "浅谈 DeepSeek mHC 一种可能的加速方案：
 *        小矩阵遇上牛顿法" ("small matrices meet Newton's method"),
 *        section 2.2 (step-size rule and Sinkhorn fallback).
 *
 * Conventions.  H is the n x n logit matrix (the pages' R = -M), so the
 * projected matrix is T = proj_KL(exp(H)).  With eta = 1 and a = b = 1
 * ([P] end of section 2.3) the dual pair (alpha, beta) recovers
 * T_ij = exp(alpha_i + beta_j + H_ij) (eq 4).  beta is always reported in the
 * gauge beta_n = 0 ([P] section 3.1).  Every matrix is row-major, matrices
 * are stored back to back ([B, n, n]).
 *
 * Precision.  Everything is IEEE double; no -ffast-math.  Plain libm exp,
 * log, expm1 and log1p.
 *
 * The oracle_eot_* functions cover the general small entropic OT of [P]
 * section 2.3 (cost M, marginals a and b, regularisation eta, n x m) with the
 * same algorithms: Sinkhorn-Knopp as the block coordinate ascent of eq (7),
 * Newton on eq (8) with the gradient and Hessian of eq (9), eq (13) backward.
 * Their pins: a hand-worked 2 x 2 plan, the 2 x 2 quadratic closed form, the
 * product plan of a separable cost, the optimality certificate of eq (4), a
 * constrained primal solver for eq (3), a library minimiser for eq (8), a
 * finite-difference Newton step, the eta / transpose / marginal-scaling
 * symmetries, the Birkhoff special case, finite differences, shift invariants
 * and unrolled autograd for eq (13).
 *
 * oracle_mix / oracle_mix_bwd are the consumer of the projection: the
 * residual-stream mixing y = H_res x of the mHC layer update ([P] section 2.1)
 * and its backward, pinned against library matmuls, exact properties of
 * doubly stochastic and permutation matrices, autograd, and finite differences
 * through the projection.
 *
 * Parity pins.  Every exported function is pinned by tests that do not call
 * this code for the expected value: the n = 2 closed form, exactly known
 * fixed points (doubly stochastic inputs with row/column shifts), rank-one
 * inputs, a constrained primal solver for eq (1), a library minimiser for
 * eq (8), finite differences and unrolled autograd for eq (13), and hand
 * computed Sinkhorn sweeps for eq (2).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_NMAX 16
/* Sinkhorn-Knopp sweeps that give Newton's starting point (not updates) */
#define START_SWEEPS 3

/* ------------------------------------------------------------------ */
/* small helpers                                                        */
/* ------------------------------------------------------------------ */

/* log(sum_k exp(v[k*s])), k < m, shifted by the maximum.  NaN propagates. */
static double lse(const double *v, int m, int s)
{
    double mx = -INFINITY;
    int nan = 0;
    for (int k = 0; k < m; ++k) {
        double x = v[k * s];
        if (x != x) nan = 1;
        else if (x > mx) mx = x;
    }
    if (nan) return NAN;
    if (mx == -INFINITY || mx == INFINITY) return mx;
    double acc = 0.0;
    for (int k = 0; k < m; ++k) acc += exp(v[k * s] - mx);
    return mx + log(acc);
}

/* eq (5) with M = -H, eta = 1, a = 1:  alpha_i = -log sum_j exp(beta_j + H_ij) */
static void alpha_of_beta(const double *H, int n, const double *beta, double *alpha)
{
    double u[ORACLE_NMAX];
    for (int i = 0; i < n; ++i) {
        for (int j = 0; j < n; ++j) u[j] = H[i * n + j] + beta[j];
        alpha[i] = -lse(u, n, 1);
    }
}

/* eq (6) with M = -H, eta = 1, b = 1:  beta_j = -log sum_i exp(alpha_i + H_ij) */
static void beta_of_alpha(const double *H, int n, const double *alpha, double *beta)
{
    double u[ORACLE_NMAX];
    for (int j = 0; j < n; ++j) {
        for (int i = 0; i < n; ++i) u[i] = H[i * n + j] + alpha[i];
        beta[j] = -lse(u, n, 1);
    }
}

/* primal recovery after eq (4):  T_ij = exp(alpha_i + beta_j + H_ij) */
static void primal(const double *H, int n, const double *alpha, const double *beta, double *T)
{
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) T[i * n + j] = exp(alpha[i] + beta[j] + H[i * n + j]);
}

/* max over rows and columns of |sum - 1| (distance to the marginals of B_n) */
static double marginal_residual(const double *T, int n)
{
    double r = 0.0;
    for (int i = 0; i < n; ++i) {
        double s = 0.0;
        for (int j = 0; j < n; ++j) s += T[i * n + j];
        double e = fabs(s - 1.0);
        if (!(e <= r)) r = e; /* NaN propagates */
    }
    for (int j = 0; j < n; ++j) {
        double s = 0.0;
        for (int i = 0; i < n; ++i) s += T[i * n + j];
        double e = fabs(s - 1.0);
        if (!(e <= r)) r = e;
    }
    return r;
}

static double max_abs_diff(const double *a, const double *b, int len)
{
    double r = 0.0;
    for (int k = 0; k < len; ++k) {
        double e = fabs(a[k] - b[k]);
        if (!(e <= r)) r = e;
    }
    return r;
}

/* Solve A x = b in place (A is m x m row-major, overwritten; x returned in b)
 * by Gaussian elimination with partial pivoting.  Returns 0, or -1 when a
 * pivot is zero or not finite. */
static int solve_gepp(double *A, double *b, int m)
{
    for (int k = 0; k < m; ++k) {
        int p = k;
        double best = fabs(A[k * m + k]);
        for (int r = k + 1; r < m; ++r) {
            double v = fabs(A[r * m + k]);
            if (v > best) { best = v; p = r; }
        }
        if (!(best > 0.0) || !isfinite(best)) return -1;
        if (p != k) {
            for (int c = 0; c < m; ++c) {
                double t = A[k * m + c]; A[k * m + c] = A[p * m + c]; A[p * m + c] = t;
            }
            double t = b[k]; b[k] = b[p]; b[p] = t;
        }
        for (int r = k + 1; r < m; ++r) {
            double f = A[r * m + k] / A[k * m + k];
            if (f == 0.0) continue;
            for (int c = k; c < m; ++c) A[r * m + c] -= f * A[k * m + c];
            b[r] -= f * b[k];
        }
    }
    for (int k = m - 1; k >= 0; --k) {
        double s = b[k];
        for (int c = k + 1; c < m; ++c) s -= A[k * m + c] * b[c];
        b[k] = s / A[k * m + k];
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Sinkhorn-Knopp in log form ([P] eq (2), as the BCA of eq (7))        */
/* ------------------------------------------------------------------ */

/* Sweeps from beta = 0 (v^(0) = 1) until the marginal residual of
 * T = exp(alpha + beta + H) is <= tol, at most cap sweeps.  One sweep is the
 * row update (eq 5) followed by the column update (eq 6).  Returns the number
 * of sweeps; *conv = 1 when the tolerance was met. */
static int sk_to_tol_one(const double *H, int n, double tol, int cap,
                         double *T, double *beta_out, int *conv)
{
    double alpha[ORACLE_NMAX], beta[ORACLE_NMAX];
    for (int j = 0; j < n; ++j) beta[j] = 0.0;
    *conv = 0;
    int k = 0;
    while (k < cap) {
        ++k;
        alpha_of_beta(H, n, beta, alpha);
        beta_of_alpha(H, n, alpha, beta);
        primal(H, n, alpha, beta, T);
        if (marginal_residual(T, n) <= tol) { *conv = 1; break; }
    }
    if (k == 0) { /* cap == 0: report the un-scaled starting point */
        alpha_of_beta(H, n, beta, alpha);
        primal(H, n, alpha, beta, T);
    }
    for (int j = 0; j < n; ++j) beta_out[j] = beta[j] - beta[n - 1];
    return k;
}

/* Exactly K sweeps from beta = 0, then T = diag(u) A diag(v)
 * (after K sweeps the column sums are exact; rows carry the error). */
static void sk_fixed_one(const double *H, int n, int K, double *T)
{
    double alpha[ORACLE_NMAX], beta[ORACLE_NMAX];
    for (int j = 0; j < n; ++j) beta[j] = 0.0;
    for (int k = 0; k < K; ++k) {
        alpha_of_beta(H, n, beta, alpha);
        beta_of_alpha(H, n, alpha, beta);
    }
    primal(H, n, alpha, beta, T);
}

/* ------------------------------------------------------------------ */
/* Newton on the reduced dual ([P] section 3.1, eqs (8)-(9))            */
/* ------------------------------------------------------------------ */

/* T(beta): row i is Softmax(H_i. + beta), evaluated max-shifted as in eq (10);
 * c_j = sum_i T_ij (eq 11). */
static void eval_T(const double *H, int n, const double *beta, double *T, double *c)
{
    for (int i = 0; i < n; ++i) {
        double mu = -INFINITY;
        for (int j = 0; j < n; ++j) {
            double u = H[i * n + j] + beta[j];
            if (u > mu) mu = u;
        }
        double s = 0.0;
        for (int j = 0; j < n; ++j) {
            double e = exp(H[i * n + j] + beta[j] - mu);
            T[i * n + j] = e;
            s += e;
        }
        for (int j = 0; j < n; ++j) T[i * n + j] /= s;
    }
    for (int j = 0; j < n; ++j) {
        double s = 0.0;
        for (int i = 0; i < n; ++i) s += T[i * n + j];
        c[j] = s;
    }
}

static double colsum_residual(const double *c, int n)
{
    double r = 0.0;
    for (int j = 0; j < n; ++j) {
        double e = fabs(c[j] - 1.0);
        if (!(e <= r)) r = e;
    }
    return r;
}

/* Newton's method for min_x f(x), x = beta_{-n} (eq 8), from the dual after
 * START_SWEEPS Sinkhorn-Knopp sweeps from beta = 0 (the pages leave x^(0) open):
 * each sweep scales the columns of the row-normalised T to sum to one,
 *   beta_j <- beta_j - log c_j + log c_n,  c = column sums of T at beta,
 * and the rows are normalised again (T = rows of softmax(H + beta)).  The
 * sweeps are not counted as updates; they stop early if a column sum
 * underflows.
 *   gradient  g = c_{-n} - 1                           (eq 9, a = b = 1)
 *   Hessian   diag(c_{-n}) - T_{-n}^T T_{-n}           (eq 9, eta = 1)
 *   step      x+ = x + gamma d,  d = -Hess^{-1} g
 * Step size ([B] section 2.2): try gamma = 1, 0.5, 0.1, 0.05, 0.01 in turn and
 * take the first one at which both the objective and the gradient are smaller
 * than at x (read as f(x + gamma d) < f(x) and ||g(x + gamma d)||_2 < ||g(x)||_2);
 * when none is taken, do one Sinkhorn-Knopp sweep (eqs 5-7) and re-gauge
 * beta_n = 0.  The objective difference is evaluated through the exact identity
 *   f(x + gamma d) - f(x) = sum_i log(sum_j T_ij e^{gamma d_j}) - gamma sum_j d_j,
 * which follows from f = n + sum_i LSE_i(H_i. + beta) - sum_j beta_j (eq 8 with
 * eq 5), written with log1p / expm1 (rows of T sum to one).
 * Stop when every column sum is within tol of 1 (rows are exact by
 * construction), or after max_iter updates (a trial point is not an update).
 * Returns the number of updates, or -1 when tol was not reached. */
static int newton_one(const double *H, int n, double tol, int max_iter,
                      double *T, double *beta_out)
{
    static const double steps[5] = {1.0, 0.5, 0.1, 0.05, 0.01};
    const int m = n - 1;
    double beta[ORACLE_NMAX] = {0}, c[ORACLE_NMAX] = {0}, g[ORACLE_NMAX], d[ORACLE_NMAX];
    double hess[ORACLE_NMAX * ORACLE_NMAX];
    double bt[ORACLE_NMAX], Tt[ORACLE_NMAX * ORACLE_NMAX], ct[ORACLE_NMAX];
    double alpha[ORACLE_NMAX];
    for (int j = 0; j < n; ++j) beta[j] = 0.0;
    eval_T(H, n, beta, T, c);
    int ok = 1;
    for (int j = 0; j < n; ++j) ok = ok && c[j] > 0.0 && isfinite(c[j]);
    for (int sw = 0; sw < START_SWEEPS && ok; ++sw) {
        const double lcn = log(c[n - 1]);
        for (int j = 0; j < n; ++j) beta[j] += -log(c[j]) + lcn;
        eval_T(H, n, beta, T, c);
        for (int j = 0; j < n; ++j) ok = ok && c[j] > 0.0 && isfinite(c[j]);
    }
    int it = 0, conv = 0;
    for (;;) {
        double res = colsum_residual(c, n);
        if (res != res) break;
        if (res <= tol) { conv = 1; break; }
        if (it >= max_iter) break;

        double gn2 = 0.0;
        for (int j = 0; j < m; ++j) { g[j] = c[j] - 1.0; gn2 += g[j] * g[j]; }
        /* h_jk = [j == k] c_j - sum_i T_ij T_ik (eq 9).  The diagonal is formed
         * as sum_i T_ij (sum_{l != j} T_il): the same number, since every row of
         * T sums to one (eval_T normalises it), without the cancellation of
         * c_j - sum_i T_ij^2, which leaves no correct digit once column j is
         * carried by one entry within 1e-16 of 1 (logit spans beyond ~40). */
        for (int j = 0; j < m; ++j)
            for (int k = 0; k < m; ++k) {
                double p = 0.0;
                if (j == k) {
                    for (int i = 0; i < n; ++i) {
                        double o = 0.0;
                        for (int l = 0; l < n; ++l)
                            if (l != j) o += T[i * n + l];
                        p += T[i * n + j] * o;
                    }
                    hess[j * m + k] = p;
                } else {
                    for (int i = 0; i < n; ++i) p += T[i * n + j] * T[i * n + k];
                    hess[j * m + k] = -p;
                }
            }
        for (int j = 0; j < m; ++j) d[j] = -g[j];
        int accepted = 0;
        if (solve_gepp(hess, d, m) == 0) {
            for (int s = 0; s < 5 && !accepted; ++s) {
                double gam = steps[s];
                double df = 0.0;
                for (int i = 0; i < n; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < m; ++j) acc += T[i * n + j] * expm1(gam * d[j]);
                    df += log1p(acc);
                }
                for (int j = 0; j < m; ++j) df -= gam * d[j];
                for (int j = 0; j < m; ++j) bt[j] = beta[j] + gam * d[j];
                bt[m] = 0.0;
                eval_T(H, n, bt, Tt, ct);
                double gt2 = 0.0;
                for (int j = 0; j < m; ++j) gt2 += (ct[j] - 1.0) * (ct[j] - 1.0);
                if (df < 0.0 && gt2 < gn2) {
                    accepted = 1;
                    memcpy(beta, bt, sizeof(double) * n);
                    memcpy(T, Tt, sizeof(double) * n * n);
                    memcpy(c, ct, sizeof(double) * n);
                }
            }
        }
        if (!accepted) {
            alpha_of_beta(H, n, beta, alpha);
            beta_of_alpha(H, n, alpha, beta);
            double sh = beta[m];
            for (int j = 0; j < n; ++j) beta[j] -= sh;
            eval_T(H, n, beta, T, c);
        }
        ++it;
    }
    for (int j = 0; j < n; ++j) beta_out[j] = beta[j];
    return conv ? it : -1;
}

/* ------------------------------------------------------------------ */
/* Implicit-differentiation backward ([P] section 4.1, eq (13))         */
/* ------------------------------------------------------------------ */

/* dH = d<G, T*>/dH for T* = proj(exp(H)).  eq (13) with eta = 1, a = b = 1:
 *   Gamma = G o T*, mu_r = Gamma 1, mu_c = (Gamma^T)_{-n} 1,
 *   Delta = I - T*_{-n}^T T*_{-n},
 *   w_{-n} = Delta^{-1} (mu_c - T*_{-n}^T mu_r),  w_n = 0,
 *   D = diag(mu_r - T*_{-n} w_{-n}) T* + T* diag(w) - Gamma   (= dl/dM),
 * and dH = -D because H = -M ([P] end of section 4.2).  Returns -1 when Delta
 * is singular (dH is then NaN). */
static int bwd_one(const double *T, const double *G, int n, double *dH)
{
    const int m = n - 1;
    double gam[ORACLE_NMAX * ORACLE_NMAX], mur[ORACLE_NMAX], rhs[ORACLE_NMAX];
    double delta[ORACLE_NMAX * ORACLE_NMAX], w[ORACLE_NMAX], v[ORACLE_NMAX];
    for (int k = 0; k < n * n; ++k) gam[k] = G[k] * T[k];
    for (int i = 0; i < n; ++i) {
        double s = 0.0;
        for (int j = 0; j < n; ++j) s += gam[i * n + j];
        mur[i] = s;
    }
    for (int j = 0; j < m; ++j) {
        double muc = 0.0, tmu = 0.0;
        for (int i = 0; i < n; ++i) {
            muc += gam[i * n + j];
            tmu += T[i * n + j] * mur[i];
        }
        rhs[j] = muc - tmu;
        for (int k = 0; k < m; ++k) {
            double p = 0.0;
            for (int i = 0; i < n; ++i) p += T[i * n + j] * T[i * n + k];
            delta[j * m + k] = (j == k ? 1.0 : 0.0) - p;
        }
    }
    int rc = solve_gepp(delta, rhs, m);
    for (int j = 0; j < m; ++j) w[j] = rc == 0 ? rhs[j] : NAN;
    w[m] = 0.0;
    for (int i = 0; i < n; ++i) {
        double s = mur[i];
        for (int j = 0; j < m; ++j) s -= T[i * n + j] * w[j];
        v[i] = s;
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) {
            double Dij = v[i] * T[i * n + j] + T[i * n + j] * w[j] - gam[i * n + j];
            dH[i * n + j] = -Dij;
        }
    return rc;
}

/* ------------------------------------------------------------------ */
/* General small entropic OT ([P] section 2.3, eqs (3)-(9); eq (13))    */
/* ------------------------------------------------------------------ */
/* Cost M is n x m (row-major), marginals a (n) > 0 and b (m) > 0 with equal
 * sums, regularisation eta > 0.  The plan is T_ij = exp((alpha_i + beta_j -
 * M_ij) / eta) (eq 4), the dual reported with beta_m = 0. */

/* eq (5): alpha_i = eta log a_i - eta log sum_j exp((beta_j - M_ij) / eta) */
static void eot_alpha(const double *M, const double *a, int n, int m, double eta, const double *beta,
                      double *alpha)
{
    double u[ORACLE_NMAX];
    for (int i = 0; i < n; ++i) {
        for (int j = 0; j < m; ++j) u[j] = (beta[j] - M[i * m + j]) / eta;
        alpha[i] = eta * log(a[i]) - eta * lse(u, m, 1);
    }
}

/* eq (6): beta_j = eta log b_j - eta log sum_i exp((alpha_i - M_ij) / eta) */
static void eot_beta(const double *M, const double *b, int n, int m, double eta, const double *alpha,
                     double *beta)
{
    double u[ORACLE_NMAX];
    for (int j = 0; j < m; ++j) {
        for (int i = 0; i < n; ++i) u[i] = (alpha[i] - M[i * m + j]) / eta;
        beta[j] = eta * log(b[j]) - eta * lse(u, n, 1);
    }
}

/* primal recovery after eq (4) */
static void eot_primal(const double *M, int n, int m, double eta, const double *alpha, const double *beta,
                       double *T)
{
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < m; ++j) T[i * m + j] = exp((alpha[i] + beta[j] - M[i * m + j]) / eta);
}

/* max(|T 1 - a|, |T^T 1 - b|) */
static double eot_marginal_residual(const double *T, const double *a, const double *b, int n, int m)
{
    double r = 0.0;
    for (int i = 0; i < n; ++i) {
        double s = 0.0;
        for (int j = 0; j < m; ++j) s += T[i * m + j];
        double e = fabs(s - a[i]);
        if (!(e <= r)) r = e;
    }
    for (int j = 0; j < m; ++j) {
        double s = 0.0;
        for (int i = 0; i < n; ++i) s += T[i * m + j];
        double e = fabs(s - b[j]);
        if (!(e <= r)) r = e;
    }
    return r;
}

/* Block coordinate ascent eq (7) (= Sinkhorn-Knopp) from beta = 0 until the
 * marginal residual is <= tol, at most cap sweeps. */
static int eot_sk_one(const double *M, const double *a, const double *b, int n, int m, double eta, double tol,
                      int cap, double *T, double *beta_out, int *conv)
{
    double alpha[ORACLE_NMAX], beta[ORACLE_NMAX];
    for (int j = 0; j < m; ++j) beta[j] = 0.0;
    *conv = 0;
    int k = 0;
    while (k < cap) {
        ++k;
        eot_alpha(M, a, n, m, eta, beta, alpha);
        eot_beta(M, b, n, m, eta, alpha, beta);
        eot_primal(M, n, m, eta, alpha, beta, T);
        if (eot_marginal_residual(T, a, b, n, m) <= tol) { *conv = 1; break; }
    }
    if (k == 0) {
        eot_alpha(M, a, n, m, eta, beta, alpha);
        eot_primal(M, n, m, eta, alpha, beta, T);
    }
    for (int j = 0; j < m; ++j) beta_out[j] = beta[j] - beta[m - 1];
    return k;
}

/* T(beta): T_i. = a_i Softmax((beta - M_i.) / eta) ([P] section 3.1); c = T^T 1. */
static void eot_eval_T(const double *M, const double *a, int n, int m, double eta, const double *beta, double *T,
                       double *c)
{
    for (int i = 0; i < n; ++i) {
        double mu = -INFINITY;
        for (int j = 0; j < m; ++j) {
            double u = (beta[j] - M[i * m + j]) / eta;
            if (u > mu) mu = u;
        }
        double s = 0.0;
        for (int j = 0; j < m; ++j) {
            double e = exp((beta[j] - M[i * m + j]) / eta - mu);
            T[i * m + j] = e;
            s += e;
        }
        for (int j = 0; j < m; ++j) T[i * m + j] *= a[i] / s;
    }
    for (int j = 0; j < m; ++j) {
        double s = 0.0;
        for (int i = 0; i < n; ++i) s += T[i * m + j];
        c[j] = s;
    }
}

/* Newton's method on the reduced dual (eq 8), from the dual after START_SWEEPS
 * Sinkhorn-Knopp sweeps (eqs 5-7) from beta = eta log(b / b_m) (the pages leave
 * x^(0) open; this reduces to newton_one's start when a = b = 1 and eta = 1, and
 * is already the optimum when the cost is constant, whose plan is
 * a b^T / sum(b)): each sweep, with c the column sums of T at beta,
 *   beta_j <- beta_j + eta (log(b_j / c_j) - log(b_m / c_m)),
 * not counted as updates (they stop when a column sum underflows):
 *   gradient  g = c_{-m} - b_{-m}                                   (eq 9)
 *   Hessian   eta^-1 [diag(c_{-m}) - T_{-m}^T diag(a)^-1 T_{-m}]    (eq 9)
 * with the step-size rule and Sinkhorn fallback of [B] section 2.2, as in
 * newton_one.  With S_i. = T_i. / a_i (row softmaxes) the objective change is
 *   f(x + s) - f(x) = eta sum_i a_i log(sum_j S_ij e^{s_j / eta}) - sum_j s_j b_j
 * (eq 8 with eq 5), written with log1p / expm1.  Stops when every column sum
 * is within tol of b (rows are exact by construction).  Returns the number of
 * updates, or -1 when tol was not reached. */
static int eot_newton_one(const double *M, const double *a, const double *b, int n, int m, double eta, double tol,
                          int max_iter, double *T, double *beta_out)
{
    static const double steps[5] = {1.0, 0.5, 0.1, 0.05, 0.01};
    const int k1 = m - 1;
    double beta[ORACLE_NMAX] = {0}, c[ORACLE_NMAX] = {0}, g[ORACLE_NMAX], d[ORACLE_NMAX];
    double hess[ORACLE_NMAX * ORACLE_NMAX];
    double bt[ORACLE_NMAX], Tt[ORACLE_NMAX * ORACLE_NMAX], ct[ORACLE_NMAX];
    double alpha[ORACLE_NMAX];
    for (int j = 0; j < m; ++j) beta[j] = eta * (log(b[j]) - log(b[m - 1]));
    eot_eval_T(M, a, n, m, eta, beta, T, c);
    int ok = 1;
    for (int j = 0; j < m; ++j) ok = ok && c[j] > 0.0 && isfinite(c[j]);
    for (int sw = 0; sw < START_SWEEPS && ok; ++sw) {
        const double cm = log(b[m - 1] / c[m - 1]);
        for (int j = 0; j < m; ++j) beta[j] += eta * (log(b[j] / c[j]) - cm);
        eot_eval_T(M, a, n, m, eta, beta, T, c);
        for (int j = 0; j < m; ++j) ok = ok && c[j] > 0.0 && isfinite(c[j]);
    }
    int it = 0, conv = 0;
    for (;;) {
        double res = 0.0;
        for (int j = 0; j < m; ++j) {
            double e = fabs(c[j] - b[j]);
            if (!(e <= res)) res = e;
        }
        if (res != res) break;
        if (res <= tol) { conv = 1; break; }
        if (it >= max_iter) break;

        double gn2 = 0.0;
        for (int j = 0; j < k1; ++j) { g[j] = c[j] - b[j]; gn2 += g[j] * g[j]; }
        /* eta h_jk = [j == k] c_j - sum_i T_ij T_ik / a_i (eq 9); the diagonal as
         * sum_i (T_ij / a_i) (sum_{l != j} T_il), the same number since row i of
         * T sums to a_i, without the cancellation (see newton_one). */
        for (int j = 0; j < k1; ++j)
            for (int k = 0; k < k1; ++k) {
                double p = 0.0;
                if (j == k) {
                    for (int i = 0; i < n; ++i) {
                        double o = 0.0;
                        for (int l = 0; l < m; ++l)
                            if (l != j) o += T[i * m + l];
                        p += T[i * m + j] / a[i] * o;
                    }
                    hess[j * k1 + k] = p / eta;
                } else {
                    for (int i = 0; i < n; ++i) p += T[i * m + j] * T[i * m + k] / a[i];
                    hess[j * k1 + k] = -p / eta;
                }
            }
        for (int j = 0; j < k1; ++j) d[j] = -g[j];
        int accepted = 0;
        if (solve_gepp(hess, d, k1) == 0) {
            for (int st = 0; st < 5 && !accepted; ++st) {
                double gam = steps[st];
                double df = 0.0;
                for (int i = 0; i < n; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < k1; ++j) acc += T[i * m + j] / a[i] * expm1(gam * d[j] / eta);
                    df += eta * a[i] * log1p(acc);
                }
                for (int j = 0; j < k1; ++j) df -= gam * d[j] * b[j];
                for (int j = 0; j < k1; ++j) bt[j] = beta[j] + gam * d[j];
                bt[k1] = 0.0;
                eot_eval_T(M, a, n, m, eta, bt, Tt, ct);
                double gt2 = 0.0;
                for (int j = 0; j < k1; ++j) gt2 += (ct[j] - b[j]) * (ct[j] - b[j]);
                if (df < 0.0 && gt2 < gn2) {
                    accepted = 1;
                    memcpy(beta, bt, sizeof(double) * m);
                    memcpy(T, Tt, sizeof(double) * n * m);
                    memcpy(c, ct, sizeof(double) * m);
                }
            }
        }
        if (!accepted) {
            eot_alpha(M, a, n, m, eta, beta, alpha);
            eot_beta(M, b, n, m, eta, alpha, beta);
            double sh = beta[k1];
            for (int j = 0; j < m; ++j) beta[j] -= sh;
            eot_eval_T(M, a, n, m, eta, beta, T, c);
        }
        ++it;
    }
    for (int j = 0; j < m; ++j) beta_out[j] = beta[j];
    return conv ? it : -1;
}

/* eq (13): D = d<G, T*>/dM =
 *   eta^-1 [diag((mu_r - T*_{-m} w_{-m}) / a) T* + T* diag(w) - G o T*],
 *   w_{-m} = Delta^-1 [mu_c - (T*_{-m})^T (mu_r / a)],  w_m = 0,
 *   mu_r = (G o T*) 1_m,  mu_c = (G o T*)^T_{-m} 1_n,
 *   Delta = diag(b_{-m}) - (T*)^T_{-m} diag(a)^-1 T*_{-m}.
 * Returns -1 when Delta is singular (D is then NaN). */
static int eot_bwd_one(const double *T, const double *G, const double *a, const double *b, int n, int m,
                       double eta, double *D)
{
    const int k1 = m - 1;
    double gam[ORACLE_NMAX * ORACLE_NMAX], mur[ORACLE_NMAX], rhs[ORACLE_NMAX];
    double delta[ORACLE_NMAX * ORACLE_NMAX], w[ORACLE_NMAX], v[ORACLE_NMAX];
    for (int k = 0; k < n * m; ++k) gam[k] = G[k] * T[k];
    for (int i = 0; i < n; ++i) {
        double s = 0.0;
        for (int j = 0; j < m; ++j) s += gam[i * m + j];
        mur[i] = s;
    }
    for (int j = 0; j < k1; ++j) {
        double mc = 0.0, tm = 0.0;
        for (int i = 0; i < n; ++i) {
            mc += gam[i * m + j];
            tm += T[i * m + j] * mur[i] / a[i];
        }
        rhs[j] = mc - tm;
        for (int k = 0; k < k1; ++k) {
            double p = 0.0;
            for (int i = 0; i < n; ++i) p += T[i * m + j] / a[i] * T[i * m + k];
            delta[j * k1 + k] = (j == k ? b[j] : 0.0) - p;
        }
    }
    int rc = solve_gepp(delta, rhs, k1);
    for (int j = 0; j < k1; ++j) w[j] = rc == 0 ? rhs[j] : NAN;
    w[k1] = 0.0;
    for (int i = 0; i < n; ++i) {
        double s = mur[i];
        for (int j = 0; j < k1; ++j) s -= T[i * m + j] * w[j];
        v[i] = s;
    }
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < m; ++j)
            D[i * m + j] = (v[i] / a[i] * T[i * m + j] + T[i * m + j] * w[j] - gam[i * m + j]) / eta;
    return rc;
}

/* ------------------------------------------------------------------ */
/* exported entry points                                                */
/* ------------------------------------------------------------------ */

static int bad_args(int64_t B, int n, const void *p)
{
    return B < 0 || n < 2 || n > ORACLE_NMAX || (B > 0 && p == NULL);
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int oracle_nmax(void) { return ORACLE_NMAX; }

/* Sinkhorn-Knopp to a marginal residual <= tol (cap sweeps). */
int oracle_sinkhorn_tol(const double *H, int64_t B, int n, double tol, int cap,
                        double *T, double *beta, int32_t *sweeps, int32_t *converged)
{
    if (bad_args(B, n, H) || (B > 0 && (!T || !beta || !sweeps || !converged)) || cap < 0)
        return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t b = 0; b < B; ++b) {
        int conv = 0;
        sweeps[b] = sk_to_tol_one(H + b * n * n, n, tol, cap, T + b * n * n, beta + b * n, &conv);
        converged[b] = conv;
    }
    return 0;
}

/* Exactly K Sinkhorn-Knopp sweeps (the fixed-iteration baseline). */
int oracle_sinkhorn_k(const double *H, int64_t B, int n, int K, double *T)
{
    if (bad_args(B, n, H) || (B > 0 && !T) || K < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) sk_fixed_one(H + b * n * n, n, K, T + b * n * n);
    return 0;
}

/* Newton's method on the reduced dual; iters[b] = updates, or -1 if tol not met. */
int oracle_newton(const double *H, int64_t B, int n, double tol, int max_iter,
                  double *T, double *beta, int32_t *iters)
{
    if (bad_args(B, n, H) || (B > 0 && (!T || !beta || !iters)) || max_iter < 0) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t b = 0; b < B; ++b)
        iters[b] = newton_one(H + b * n * n, n, tol, max_iter, T + b * n * n, beta + b * n);
    return 0;
}

/* Reference projection (float64):
 *   1. Sinkhorn-Knopp to residual 1e-13 (at most sk_cap sweeps);
 *   2. Newton to residual 1e-13 (at most 500 updates) as an independent check;
 *   3. status 0: Sinkhorn converged and both agree within 1e-12 -> Sinkhorn's T;
 *      status 1: Sinkhorn hit the cap, Newton converged and one further
 *                Sinkhorn sweep from Newton's dual moves T by <= 1e-12
 *                (a fixed-point check) -> Newton's T;
 *      status < 0: no reference could be certified (T holds the best effort).
 * beta is reported with beta_n = 0. */
int oracle_project(const double *H, int64_t B, int n, int sk_cap,
                   double *T, double *beta, int32_t *status)
{
    if (bad_args(B, n, H) || (B > 0 && (!T || !beta || !status)) || sk_cap < 0) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t b = 0; b < B; ++b) {
        const double *h = H + b * n * n;
        double tsk[ORACLE_NMAX * ORACLE_NMAX], tnw[ORACLE_NMAX * ORACLE_NMAX];
        double bsk[ORACLE_NMAX], bnw[ORACLE_NMAX];
        int conv = 0;
        sk_to_tol_one(h, n, 1e-13, sk_cap, tsk, bsk, &conv);
        int it = newton_one(h, n, 1e-13, 500, tnw, bnw);
        int st;
        if (conv) {
            st = (it >= 0 && max_abs_diff(tsk, tnw, n * n) <= 1e-12) ? 0 : -1;
            memcpy(T + b * n * n, tsk, sizeof(double) * n * n);
            memcpy(beta + b * n, bsk, sizeof(double) * n);
        } else {
            st = -2;
            if (it >= 0) {
                double alpha[ORACLE_NMAX], b1[ORACLE_NMAX], t1[ORACLE_NMAX * ORACLE_NMAX];
                alpha_of_beta(h, n, bnw, alpha);
                beta_of_alpha(h, n, alpha, b1);
                primal(h, n, alpha, b1, t1);
                if (max_abs_diff(t1, tnw, n * n) <= 1e-12) st = 1;
            }
            memcpy(T + b * n * n, tnw, sizeof(double) * n * n);
            memcpy(beta + b * n, bnw, sizeof(double) * n);
        }
        status[b] = st;
    }
    return 0;
}

/* Backward pass by eq (13) at the given projected matrices T (the caller
 * passes the reference T of oracle_project).  Returns the number of matrices
 * whose Delta was singular (their dH is NaN), or -1 on bad arguments. */
int oracle_bwd(const double *T, const double *G, int64_t B, int n, double *dH)
{
    if (bad_args(B, n, T) || (B > 0 && (!G || !dH))) return -1;
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t b = 0; b < B; ++b)
        if (bwd_one(T + b * n * n, G + b * n * n, n, dH + b * n * n) != 0) ++bad;
    return (int)(bad > 0x7fffffff ? 0x7fffffff : bad);
}

/* ---- general entropic OT: a [B, n], b [B, m], M / T / G / D [B, n, m] ---- */

static int eot_bad_args(int64_t B, int n, int m, double eta, const void *p)
{
    return B < 0 || n < 1 || m < 2 || n > ORACLE_NMAX || m > ORACLE_NMAX || !(eta > 0.0) || (B > 0 && p == NULL);
}

int oracle_eot_sinkhorn_tol(const double *M, const double *a, const double *b, int64_t B, int n, int m, double eta,
                            double tol, int cap, double *T, double *beta, int32_t *sweeps, int32_t *converged)
{
    if (eot_bad_args(B, n, m, eta, M) || (B > 0 && (!a || !b || !T || !beta || !sweeps || !converged)) || cap < 0)
        return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t q = 0; q < B; ++q) {
        int conv = 0;
        sweeps[q] = eot_sk_one(M + q * n * m, a + q * n, b + q * m, n, m, eta, tol, cap, T + q * n * m,
                               beta + q * m, &conv);
        converged[q] = conv;
    }
    return 0;
}

int oracle_eot_newton(const double *M, const double *a, const double *b, int64_t B, int n, int m, double eta,
                      double tol, int max_iter, double *T, double *beta, int32_t *iters)
{
    if (eot_bad_args(B, n, m, eta, M) || (B > 0 && (!a || !b || !T || !beta || !iters)) || max_iter < 0) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t q = 0; q < B; ++q)
        iters[q] = eot_newton_one(M + q * n * m, a + q * n, b + q * m, n, m, eta, tol, max_iter, T + q * n * m,
                                  beta + q * m);
    return 0;
}

/* Reference plan, certified as in oracle_project (Sinkhorn to 1e-13 and an
 * independent Newton, or Newton plus a Sinkhorn fixed-point check). */
int oracle_eot_project(const double *M, const double *a, const double *b, int64_t B, int n, int m, double eta,
                       int sk_cap, double *T, double *beta, int32_t *status)
{
    if (eot_bad_args(B, n, m, eta, M) || (B > 0 && (!a || !b || !T || !beta || !status)) || sk_cap < 0) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t q = 0; q < B; ++q) {
        const double *Mq = M + q * n * m, *aq = a + q * n, *bq = b + q * m;
        double tsk[ORACLE_NMAX * ORACLE_NMAX], tnw[ORACLE_NMAX * ORACLE_NMAX];
        double bsk[ORACLE_NMAX], bnw[ORACLE_NMAX];
        int conv = 0;
        eot_sk_one(Mq, aq, bq, n, m, eta, 1e-13, sk_cap, tsk, bsk, &conv);
        int it = eot_newton_one(Mq, aq, bq, n, m, eta, 1e-13, 500, tnw, bnw);
        int st;
        if (conv) {
            st = (it >= 0 && max_abs_diff(tsk, tnw, n * m) <= 1e-12) ? 0 : -1;
            memcpy(T + q * n * m, tsk, sizeof(double) * n * m);
            memcpy(beta + q * m, bsk, sizeof(double) * m);
        } else {
            st = -2;
            if (it >= 0) {
                double alpha[ORACLE_NMAX], b1[ORACLE_NMAX], t1[ORACLE_NMAX * ORACLE_NMAX];
                eot_alpha(Mq, aq, n, m, eta, bnw, alpha);
                eot_beta(Mq, bq, n, m, eta, alpha, b1);
                eot_primal(Mq, n, m, eta, alpha, b1, t1);
                if (max_abs_diff(t1, tnw, n * m) <= 1e-12) st = 1;
            }
            memcpy(T + q * n * m, tnw, sizeof(double) * n * m);
            memcpy(beta + q * m, bnw, sizeof(double) * m);
        }
        status[q] = st;
    }
    return 0;
}

/* eq (13) at the given plans; returns the number of singular Delta, or -1. */
int oracle_eot_bwd(const double *T, const double *G, const double *a, const double *b, int64_t B, int n, int m,
                   double eta, double *D)
{
    if (eot_bad_args(B, n, m, eta, T) || (B > 0 && (!G || !a || !b || !D))) return -1;
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t q = 0; q < B; ++q)
        if (eot_bwd_one(T + q * n * m, G + q * n * m, a + q * n, b + q * m, n, m, eta, D + q * n * m) != 0) ++bad;
    return (int)(bad > 0x7fffffff ? 0x7fffffff : bad);
}

/* ------------------------------------------------------------------ */
/* mHC consumer: the residual-stream mixing H_res x ([P] section 2.1)   */
/* ------------------------------------------------------------------ */
/* The projected matrix is the residual mapping H_res of the layer update
 * x_{l+1} = H_res x_l + H_post^T F(H_pre x_l) ([P] section 2.1), applied to the
 * n x C hidden matrix x of each token:  y = T x  (y_ic = sum_j T_ij x_jc).
 * Its backward, for upstream dy = dL/dy:  dx = T^T dy  and  dT = dy x^T
 * (dT_ij = sum_c dy_ic x_jc), which the eq (13) backward (oracle_bwd) turns into
 * dL/dH.  Arrays: T [B, n, n], x, y, dy, dx [B, n, C], dT [B, n, n]. */

int oracle_mix(const double *T, const double *x, int64_t B, int n, int64_t C, double *y)
{
    if (B < 0 || n < 1 || n > ORACLE_NMAX || C < 0 || (B > 0 && C > 0 && (!T || !x || !y))) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < B; ++q) {
        const double *Tq = T + q * n * n, *xq = x + q * n * C;
        double *yq = y + q * n * C;
        for (int i = 0; i < n; ++i)
            for (int64_t c = 0; c < C; ++c) {
                double s = 0.0;
                for (int j = 0; j < n; ++j) s += Tq[i * n + j] * xq[j * C + c];
                yq[i * C + c] = s;
            }
    }
    return 0;
}

int oracle_mix_bwd(const double *T, const double *x, const double *dy, int64_t B, int n, int64_t C, double *dx,
                   double *dT)
{
    if (B < 0 || n < 1 || n > ORACLE_NMAX || C < 0 || (B > 0 && (!T || !x || !dy || !dx || !dT))) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < B; ++q) {
        const double *Tq = T + q * n * n, *xq = x + q * n * C, *dyq = dy + q * n * C;
        double *dxq = dx + q * n * C, *dTq = dT + q * n * n;
        for (int j = 0; j < n; ++j)
            for (int64_t c = 0; c < C; ++c) {
                double s = 0.0;
                for (int i = 0; i < n; ++i) s += Tq[i * n + j] * dyq[i * C + c];
                dxq[j * C + c] = s;
            }
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < n; ++j) {
                double s = 0.0;
                for (int64_t c = 0; c < C; ++c) s += dyq[i * C + c] * xq[j * C + c];
                dTq[i * n + j] = s;
            }
    }
    return 0;
}
