/* Host driver for a sanitizer build of oracle/oracle.c (address and
 * undefined-behaviour sanitizers, OpenMP off): runs every exported entry point
 * on small seeded inputs -- sizes 2 to 8 (1 to 8 for entropic OT), empty batches, logit spans from 1 to
 * 120, permutation-like matrices whose eq (13) system is singular -- and on
 * the argument errors each entry point rejects.  Exits non-zero when a result
 * is not finite where it must be, or a return code is wrong; the sanitizers
 * abort on any invalid access or undefined operation. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_nmax(void);
int oracle_sinkhorn_tol(const double *H, int64_t B, int n, double tol, int cap, double *T, double *beta,
                        int32_t *sweeps, int32_t *converged);
int oracle_sinkhorn_k(const double *H, int64_t B, int n, int K, double *T);
int oracle_newton(const double *H, int64_t B, int n, double tol, int max_iter, double *T, double *beta,
                  int32_t *iters);
int oracle_project(const double *H, int64_t B, int n, int sk_cap, double *T, double *beta, int32_t *status);
int oracle_bwd(const double *T, const double *G, int64_t B, int n, double *dH);
int oracle_eot_sinkhorn_tol(const double *M, const double *a, const double *b, int64_t B, int n, int m, double eta,
                            double tol, int cap, double *T, double *beta, int32_t *sweeps, int32_t *converged);
int oracle_eot_newton(const double *M, const double *a, const double *b, int64_t B, int n, int m, double eta,
                      double tol, int max_iter, double *T, double *beta, int32_t *iters);
int oracle_eot_project(const double *M, const double *a, const double *b, int64_t B, int n, int m, double eta,
                       int sk_cap, double *T, double *beta, int32_t *status);
int oracle_eot_bwd(const double *T, const double *G, const double *a, const double *b, int64_t B, int n, int m,
                   double eta, double *D);
int oracle_mix(const double *T, const double *x, int64_t B, int n, int64_t C, double *y);
int oracle_mix_bwd(const double *T, const double *x, const double *dy, int64_t B, int n, int64_t C, double *dx,
                   double *dT);

static uint64_t state = 0x9e3779b97f4a7c15ull;

static double uniform(void) /* (0, 1), splitmix64 */
{
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return ((double)(z >> 11) + 0.5) / 9007199254740992.0;
}

static double normal(void) { return sqrt(-2.0 * log(uniform())) * cos(6.283185307179586 * uniform()); }

static int failures = 0;

static void expect(int ok, const char *what, int n, double s)
{
    if (!ok) {
        fprintf(stderr, "FAIL %s (n=%d scale=%g)\n", what, n, s);
        ++failures;
    }
}

static int all_finite(const double *x, size_t k)
{
    for (size_t i = 0; i < k; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

static void projection_case(int n, double scale, int perm)
{
    enum { B = 5 };
    const size_t nn = (size_t)n * n;
    double *H = malloc(sizeof(double) * B * nn), *T = malloc(sizeof(double) * B * nn);
    double *G = malloc(sizeof(double) * B * nn), *dH = malloc(sizeof(double) * B * nn);
    double *beta = malloc(sizeof(double) * B * n);
    int32_t st[B], cnt[B], conv[B];
    for (size_t i = 0; i < B * nn; ++i) {
        H[i] = scale * normal();
        G[i] = normal();
    }
    if (perm) /* scale on a cyclic permutation, 0 elsewhere */
        for (int b = 0; b < B; ++b)
            for (int i = 0; i < n; ++i)
                for (int j = 0; j < n; ++j) H[b * nn + i * n + j] = (j == (i + b) % n) ? scale : 0.0;
    expect(oracle_sinkhorn_k(H, B, n, 20, T) == 0 && all_finite(T, B * nn), "sinkhorn_k", n, scale);
    expect(oracle_sinkhorn_tol(H, B, n, 1e-10, 300, T, beta, cnt, conv) == 0 && all_finite(T, B * nn),
           "sinkhorn_tol", n, scale);
    expect(oracle_newton(H, B, n, 1e-10, 200, T, beta, cnt) == 0, "newton", n, scale);
    expect(oracle_project(H, B, n, 2000, T, beta, st) == 0 && all_finite(T, B * nn), "project", n, scale);
    const int bad = oracle_bwd(T, G, B, n, dH);
    expect(bad >= 0 && bad <= B, "bwd", n, scale);
    if (bad == 0) expect(all_finite(dH, B * nn), "bwd finite", n, scale);
    free(H); free(T); free(G); free(dH); free(beta);
}

static void eot_case(int n, int m, double eta)
{
    enum { B = 4 };
    const size_t nm = (size_t)n * m;
    double *M = malloc(sizeof(double) * B * nm), *T = malloc(sizeof(double) * B * nm);
    double *G = malloc(sizeof(double) * B * nm), *D = malloc(sizeof(double) * B * nm);
    double *a = malloc(sizeof(double) * B * n), *b = malloc(sizeof(double) * B * m);
    double *beta = malloc(sizeof(double) * B * m);
    int32_t st[B], cnt[B], conv[B];
    for (size_t i = 0; i < B * nm; ++i) {
        M[i] = normal();
        G[i] = normal();
    }
    for (int q = 0; q < B; ++q) { /* positive marginals of equal mass */
        double sa = 0, sb = 0;
        for (int i = 0; i < n; ++i) sa += (a[q * n + i] = 0.2 + uniform());
        for (int j = 0; j < m; ++j) sb += (b[q * m + j] = 0.2 + uniform());
        for (int j = 0; j < m; ++j) b[q * m + j] *= sa / sb;
    }
    expect(oracle_eot_sinkhorn_tol(M, a, b, B, n, m, eta, 1e-10, 500, T, beta, cnt, conv) == 0, "eot sk", n, eta);
    expect(oracle_eot_newton(M, a, b, B, n, m, eta, 1e-10, 300, T, beta, cnt) == 0, "eot newton", n, eta);
    expect(oracle_eot_project(M, a, b, B, n, m, eta, 5000, T, beta, st) == 0 && all_finite(T, B * nm), "eot project",
           n, eta);
    const int bad = oracle_eot_bwd(T, G, a, b, B, n, m, eta, D);
    expect(bad >= 0 && bad <= B, "eot bwd", n, eta);
    free(M); free(T); free(G); free(D); free(a); free(b); free(beta);
}

static void mix_case(int n, int64_t C)
{
    enum { B = 3 };
    double T[B * 64], dT[B * 64];
    double *x = malloc(sizeof(double) * (B * n * C + 1)), *y = malloc(sizeof(double) * (B * n * C + 1));
    double *dy = malloc(sizeof(double) * (B * n * C + 1)), *dx = malloc(sizeof(double) * (B * n * C + 1));
    for (int i = 0; i < B * n * n; ++i) T[i] = uniform();
    for (int64_t i = 0; i < B * n * C; ++i) {
        x[i] = normal();
        dy[i] = normal();
    }
    expect(oracle_mix(T, x, B, n, C, y) == 0 && all_finite(y, (size_t)(B * n * C)), "mix", n, (double)C);
    expect(oracle_mix_bwd(T, x, dy, B, n, C, dx, dT) == 0 && all_finite(dT, (size_t)(B * n * n)), "mix bwd", n,
           (double)C);
    free(x); free(y); free(dy); free(dx);
}

static void argument_errors(void)
{
    double h[16] = {0}, t[16], beta[4];
    int32_t st[1], cnt[1], conv[1];
    const int big = oracle_nmax() + 1;
    expect(oracle_project(h, -1, 4, 10, t, beta, st) == -1, "negative B", 4, 0);
    expect(oracle_project(h, 1, 1, 10, t, beta, st) == -1, "n = 1", 1, 0);
    expect(oracle_project(h, 1, big, 10, t, beta, st) == -1, "n too large", big, 0);
    expect(oracle_project(NULL, 1, 4, 10, t, beta, st) == -1, "NULL H", 4, 0);
    expect(oracle_project(h, 1, 4, 10, NULL, beta, st) == -1, "NULL T", 4, 0);
    expect(oracle_project(h, 1, 4, -1, t, beta, st) == -1, "negative cap", 4, 0);
    expect(oracle_sinkhorn_tol(h, 1, 4, 1e-9, 10, t, beta, NULL, conv) == -1, "NULL sweeps", 4, 0);
    expect(oracle_newton(h, 1, 4, 1e-9, -1, t, beta, cnt) == -1, "negative max_iter", 4, 0);
    expect(oracle_bwd(h, NULL, 1, 4, t) == -1, "NULL G", 4, 0);
    expect(oracle_eot_project(h, h, h, 1, 2, 2, 0.0, 10, t, beta, st) == -1, "eta = 0", 2, 0);
    expect(oracle_eot_project(h, h, h, 1, 2, 1, 1.0, 10, t, beta, st) == -1, "m = 1", 2, 0);
    expect(oracle_mix(h, h, 1, 4, -1, t) == -1, "negative C", 4, 0);
    /* empty batches take NULL pointers */
    expect(oracle_project(NULL, 0, 4, 10, NULL, NULL, NULL) == 0, "empty project", 4, 0);
    expect(oracle_bwd(NULL, NULL, 0, 4, NULL) == 0, "empty bwd", 4, 0);
    expect(oracle_eot_bwd(NULL, NULL, NULL, NULL, 0, 3, 3, 1.0, NULL) == 0, "empty eot bwd", 3, 0);
    expect(oracle_mix(NULL, NULL, 0, 4, 8, NULL) == 0, "empty mix", 4, 0);
}

int main(void)
{
    const int sizes[] = {2, 3, 4, 5, 8};
    const double scales[] = {1.0, 10.0, 30.0, 120.0};
    for (size_t i = 0; i < sizeof sizes / sizeof *sizes; ++i)
        for (size_t k = 0; k < sizeof scales / sizeof *scales; ++k) {
            projection_case(sizes[i], scales[k], 0);
            projection_case(sizes[i], scales[k], 1);
        }
    eot_case(1, 2, 1.0);
    eot_case(3, 5, 0.5);
    eot_case(8, 8, 0.1);
    eot_case(4, 4, 1.0 / 32);
    mix_case(4, 0);
    mix_case(4, 7);
    mix_case(8, 3);
    argument_errors();
    if (failures) return 1;
    puts("oracle driver: ok");
    return 0;
}
