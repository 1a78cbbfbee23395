// projection.hpp -- per-lane device routines for the batched KL projection
// onto the Birkhoff polytope and its implicit backward pass (gfx950).
//
// Layout.  One matrix per lane: a wave of 64 lanes owns 64 consecutive
// matrices, each held entirely in VGPRs (n = 4: 16 logits, 16 entries of T,
// the 6-entry Hessian triangle).  There is no cross-lane traffic, no LDS and
// no MFMA: the work is tiny and independent per matrix, and the per-matrix
// scalar logic (the 3x3 solve, the step-size search) runs once per matrix
// rather than being replicated across a group of lanes.  Control flow is
// per lane; the wave keeps stepping while any of its lanes is unconverged.
//
// Units.  Logits are scaled by log2(e) on load and the dual is kept in the
// same base-2 units (y = beta * log2 e), so that every exponential is one
// v_exp_f32.  Gradients, Hessians and Newton directions are in natural units
// as in the pages; a step x (natural) moves y by x * log2 e.
//
// Sources: "Accelerating Birkhoff Projection for Manifold-Constrained
// Hyper-Connections", sections 2.2-4.2, eqs (2), (5)-(13); the blog post
// "小矩阵遇上牛顿法", section 2.2, for the step sizes and the fallback.
#pragma once

#include "device_math.hpp"

namespace birk {

constexpr int kBlock = 256;  // threads per workgroup (4 waves of 64)

// packed lower triangle of an (N-1) x (N-1) symmetric matrix
template <int N>
struct Tri {
    static constexpr int M = N - 1;
    static constexpr int S = M * (M + 1) / 2;
    __host__ __device__ static constexpr int at(int j, int k) { return j * (j + 1) / 2 + k; }  // k <= j
};

// Rows of T are Softmax(H_i. + beta) ([P] section 3.1), evaluated with the row
// maximum subtracted as in eq (10):  T_ij = 2^{L_ij + y_j - mu_i} / sum_k 2^{L_ik + y_k - mu_i},
// with y_{N-1} = 0.  Each row then sums to one up to rounding.
template <int N>
__device__ __forceinline__ void softmax_rows(const float (&L)[N * N], const float (&y)[N - 1], float (&T)[N * N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float u[N];
#pragma unroll
        for (int j = 0; j < N - 1; ++j) u[j] = L[i * N + j] + y[j];
        u[N - 1] = L[i * N + N - 1];
        float mu = u[0];
#pragma unroll
        for (int j = 1; j < N; ++j) mu = fmaxf(mu, u[j]);
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            u[j] = ex2(u[j] - mu);
            s += u[j];
        }
        const float r = rcp(s);
#pragma unroll
        for (int j = 0; j < N; ++j) T[i * N + j] = u[j] * r;
    }
}

// column sums c_j = sum_i T_ij (eq 11); the gradient of the reduced dual is c_{-n} - 1 (eq 9)
template <int N>
__device__ __forceinline__ void col_sums(const float (&T)[N * N], float (&c)[N]) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float s = T[j];
#pragma unroll
        for (int i = 1; i < N; ++i) s += T[i * N + j];
        c[j] = s;
    }
}

// max_j |c_j - 1| over all N columns; NaN propagates
template <int N>
__device__ __forceinline__ float col_residual(const float (&c)[N]) {
    float r = fabsf(c[0] - 1.0f);
#pragma unroll
    for (int j = 1; j < N; ++j) {
        const float e = fabsf(c[j] - 1.0f);
        r = (e > r || e != e) ? e : r;
    }
    return r;
}

// Hessian of the reduced dual objective, eq (9) with eta = 1, a = b = 1:
//   h_jk = [j == k] c_j - sum_i T_ij T_ik,   j, k < N-1.
// The diagonal is evaluated as sum_i T_ij * (sum_{k != j} T_ik), which equals
// c_j - sum_i T_ij^2 when every row of T sums to one but has no cancellation
// when a column is dominated by one entry close to 1.  At the optimum this is
// also the Delta of eq (13) ([P] section 4.2).
template <int N>
__device__ __forceinline__ void hessian(const float (&T)[N * N], float (&h)[Tri<N>::S]) {
    constexpr int M = N - 1;
#pragma unroll
    for (int j = 0; j < M; ++j)
#pragma unroll
        for (int k = 0; k < j; ++k) {
            float p = T[j] * T[k];
#pragma unroll
            for (int i = 1; i < N; ++i) p = fmaf(T[i * N + j], T[i * N + k], p);
            h[Tri<N>::at(j, k)] = -p;
        }
    float dg[M];
#pragma unroll
    for (int j = 0; j < M; ++j) dg[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        // o_j = sum of row i without entry j, from prefix and suffix sums
        float pre[N], suf[N];
        pre[0] = 0.0f;
#pragma unroll
        for (int k = 1; k < N; ++k) pre[k] = (k == 1) ? T[i * N] : pre[k - 1] + T[i * N + k - 1];
        suf[N - 1] = 0.0f;
#pragma unroll
        for (int k = N - 2; k >= 0; --k) suf[k] = (k == N - 2) ? T[i * N + N - 1] : suf[k + 1] + T[i * N + k + 1];
#pragma unroll
        for (int j = 0; j < M; ++j) dg[j] = fmaf(T[i * N + j], pre[j] + suf[j], dg[j]);
    }
#pragma unroll
    for (int j = 0; j < M; ++j) h[Tri<N>::at(j, j)] = dg[j];
}

// x = H^{-1} r for the symmetric positive definite (N-1) x (N-1) matrix H.
// N = 4: the closed-form adjugate of eq (12).  Other N: Cholesky H = L L^T in
// registers.  Returns false when H is not numerically positive definite (a
// non-positive or non-finite determinant / pivot); x is then meaningless.
template <int N>
struct SpdSolve {
    __device__ __forceinline__ static bool run(const float (&h)[Tri<N>::S], const float (&r)[N - 1], float (&x)[N - 1]) {
        constexpr int M = N - 1;
        float l[Tri<N>::S];   // Cholesky factor, packed lower triangle
        float dinv[M];        // 1 / l_jj
        bool ok = true;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            float s = h[Tri<N>::at(j, j)];
#pragma unroll
            for (int k = 0; k < j; ++k) s = fmaf(-l[Tri<N>::at(j, k)], l[Tri<N>::at(j, k)], s);
            ok = ok && (s > 1.17549435e-38f) && (s < 3.0e38f);
            const float ri = rsq(s);
            dinv[j] = ri;
            l[Tri<N>::at(j, j)] = s * ri;
#pragma unroll
            for (int i = j + 1; i < M; ++i) {
                float t = h[Tri<N>::at(i, j)];
#pragma unroll
                for (int k = 0; k < j; ++k) t = fmaf(-l[Tri<N>::at(i, k)], l[Tri<N>::at(j, k)], t);
                l[Tri<N>::at(i, j)] = t * ri;
            }
        }
        float z[M];
#pragma unroll
        for (int j = 0; j < M; ++j) {
            float t = r[j];
#pragma unroll
            for (int k = 0; k < j; ++k) t = fmaf(-l[Tri<N>::at(j, k)], z[k], t);
            z[j] = t * dinv[j];
        }
#pragma unroll
        for (int j = M - 1; j >= 0; --j) {
            float t = z[j];
#pragma unroll
            for (int k = j + 1; k < M; ++k) t = fmaf(-l[Tri<N>::at(k, j)], x[k], t);
            x[j] = t * dinv[j];
        }
        return ok;
    }
};

template <>
struct SpdSolve<4> {
    // eq (12): cofactors of the symmetric 3x3 H, det(H) by the first column,
    // x = adj(H) r / det(H).
    __device__ __forceinline__ static bool run(const float (&h)[6], const float (&r)[3], float (&x)[3]) {
        const float h11 = h[0], h21 = h[1], h22 = h[2], h31 = h[3], h32 = h[4], h33 = h[5];
        const float a11 = fmaf(h22, h33, -h32 * h32);
        const float a12 = fmaf(h31, h32, -h21 * h33);
        const float a13 = fmaf(h21, h32, -h22 * h31);
        const float a22 = fmaf(h11, h33, -h31 * h31);
        const float a23 = fmaf(h21, h31, -h11 * h32);
        const float a33 = fmaf(h11, h22, -h21 * h21);
        const float det = fmaf(h11, a11, fmaf(h21, a12, h31 * a13));
        const float q = rcp(det);
        x[0] = fmaf(a11, r[0], fmaf(a12, r[1], a13 * r[2])) * q;
        x[1] = fmaf(a12, r[0], fmaf(a22, r[1], a23 * r[2])) * q;
        x[2] = fmaf(a13, r[0], fmaf(a23, r[1], a33 * r[2])) * q;
        return (det > 1.17549435e-38f) && (det < 3.0e38f);
    }
};

// f(x + s) - f(x) for the step s (natural units, s_{N-1} = 0), by the exact identity
//   sum_i log(sum_j T_ij e^{s_j}) - sum_j s_j
// that follows from f = n + sum_i LSE_i(H_i. + beta) - sum_j beta_j (eq 8 with eq 5),
// written as sum_i log1p(sum_j T_ij expm1(s_j)) - sum_j s_j so that it keeps its
// relative accuracy when the step is small (rows of T sum to one).
template <int N>
__device__ __forceinline__ float objective_change(const float (&T)[N * N], const float (&s)[N - 1]) {
    float em[N - 1];
    float df = 0.0f;
#pragma unroll
    for (int j = 0; j < N - 1; ++j) {
        em[j] = expm1_from(s[j], ex2(s[j] * kLog2e));
        df -= s[j];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float a = T[i * N] * em[0];
#pragma unroll
        for (int j = 1; j < N - 1; ++j) a = fmaf(T[i * N + j], em[j], a);
        df += log1p_acc(a);
    }
    return df;
}

// One Sinkhorn-Knopp sweep in the log domain (eq 7 = eq 2), used as the fallback
// when no step size is accepted: alpha = alpha*(beta) (eq 5, row log-sum-exp),
// then beta = beta*(alpha) (eq 6, column log-sum-exp), re-gauged to beta_{N-1} = 0.
// Base-2 units throughout; no column sum is ever formed, so an underflowed
// column cannot produce log(0).
template <int N>
__device__ __forceinline__ void sinkhorn_sweep(const float (&L)[N * N], float (&y)[N - 1]) {
    float a[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float u[N];
#pragma unroll
        for (int j = 0; j < N - 1; ++j) u[j] = L[i * N + j] + y[j];
        u[N - 1] = L[i * N + N - 1];
        float mu = u[0];
#pragma unroll
        for (int j = 1; j < N; ++j) mu = fmaxf(mu, u[j]);
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < N; ++j) s += ex2(u[j] - mu);
        a[i] = -(mu + lg2(s));
    }
    float z[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float v[N];
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = L[i * N + j] + a[i];
        float m = v[0];
#pragma unroll
        for (int i = 1; i < N; ++i) m = fmaxf(m, v[i]);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) s += ex2(v[i] - m);
        z[j] = -(m + lg2(s));
    }
#pragma unroll
    for (int j = 0; j < N - 1; ++j) y[j] = z[j] - z[N - 1];
}

__device__ __forceinline__ float step_size(int k) {
    // the blog's step sizes, tried in this order
    return k == 0 ? 1.0f : k == 1 ? 0.5f : k == 2 ? 0.1f : k == 3 ? 0.05f : 0.01f;
}

// ---------------------------------------------------------------------------
// Forward: Newton on the reduced dual (eq 8), one matrix per lane.
// ---------------------------------------------------------------------------
template <int N, typename IO, bool kStats>
__global__ void __launch_bounds__(kBlock)
newton_fwd_kernel(const IO* __restrict__ logits, IO* __restrict__ Tout, float* __restrict__ dual,
                  int32_t* __restrict__ iters, int64_t B, float tol, int max_iter) {
    constexpr int M = N - 1;
    const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (b >= B) return;

    float L[N * N];
    Storage<IO>::template load<N * N>(logits + b * (N * N), L);
#pragma unroll
    for (int k = 0; k < N * N; ++k) L[k] *= kLog2e;

    float y[M];
#pragma unroll
    for (int j = 0; j < M; ++j) y[j] = 0.0f;   // x^(0) = 0
    float T[N * N], c[N];
    softmax_rows<N>(L, y, T);
    col_sums<N>(T, c);
    float res = col_residual<N>(c);
    int it = 0;

    while (res > tol && it < max_iter) {
        float g[M], r[M], d[M];
        float gn2 = 0.0f;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            g[j] = c[j] - 1.0f;
            r[j] = -g[j];
            gn2 = fmaf(g[j], g[j], gn2);
        }
        float h[Tri<N>::S];
        hessian<N>(T, h);
        const bool ok = SpdSolve<N>::run(h, r, d);   // d = -H^{-1} g

        bool accepted = false;
        if (ok) {
            for (int k = 0; k < 5; ++k) {
                const float gam = step_size(k);
                float s[M], yt[M];
#pragma unroll
                for (int j = 0; j < M; ++j) {
                    s[j] = gam * d[j];
                    yt[j] = fmaf(s[j], kLog2e, y[j]);
                }
                const float df = objective_change<N>(T, s);
                float Tt[N * N], ct[N];
                softmax_rows<N>(L, yt, Tt);
                col_sums<N>(Tt, ct);
                float gt2 = 0.0f;
#pragma unroll
                for (int j = 0; j < M; ++j) gt2 = fmaf(ct[j] - 1.0f, ct[j] - 1.0f, gt2);
                if (df < 0.0f && gt2 < gn2) {
#pragma unroll
                    for (int j = 0; j < M; ++j) y[j] = yt[j];
#pragma unroll
                    for (int q = 0; q < N * N; ++q) T[q] = Tt[q];
#pragma unroll
                    for (int j = 0; j < N; ++j) c[j] = ct[j];
                    accepted = true;
                    break;
                }
            }
        }
        if (!accepted) {
            sinkhorn_sweep<N>(L, y);
            softmax_rows<N>(L, y, T);
            col_sums<N>(T, c);
        }
        ++it;
        res = col_residual<N>(c);
    }

    Storage<IO>::template store<N * N>(Tout + b * (N * N), T);
    float beta[N];
#pragma unroll
    for (int j = 0; j < M; ++j) beta[j] = y[j] * kLn2;
    beta[M] = 0.0f;
    Storage<float>::template store<N>(dual + b * N, beta);
    if (kStats) iters[b] = (res <= tol) ? it : -1;
}

// ---------------------------------------------------------------------------
// Backward: eq (13) at T recomputed from (logits, dual), one matrix per lane.
// ---------------------------------------------------------------------------
template <int N, typename IO>
__global__ void __launch_bounds__(kBlock)
implicit_bwd_kernel(const IO* __restrict__ logits, const float* __restrict__ dual, const IO* __restrict__ dT,
                    IO* __restrict__ dH, int64_t B) {
    constexpr int M = N - 1;
    const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (b >= B) return;

    float L[N * N], G[N * N], beta[N];
    Storage<IO>::template load<N * N>(logits + b * (N * N), L);
    Storage<float>::template load<N>(dual + b * N, beta);
    Storage<IO>::template load<N * N>(dT + b * (N * N), G);
#pragma unroll
    for (int k = 0; k < N * N; ++k) L[k] *= kLog2e;
    float y[M];
#pragma unroll
    for (int j = 0; j < M; ++j) y[j] = (beta[j] - beta[M]) * kLog2e;   // T is invariant to the gauge
    float T[N * N];
    softmax_rows<N>(L, y, T);   // recompute T* ([P] section 4.2)

    // mu_r = (G o T) 1;  rhs = mu_c - T_{-n}^T mu_r = sum_i T_ij (G_ij - mu_r_i)
    float mur[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float s = G[i * N] * T[i * N];
#pragma unroll
        for (int j = 1; j < N; ++j) s = fmaf(G[i * N + j], T[i * N + j], s);
        mur[i] = s;
    }
    float rhs[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        float s = T[j] * (G[j] - mur[0]);
#pragma unroll
        for (int i = 1; i < N; ++i) s = fmaf(T[i * N + j], G[i * N + j] - mur[i], s);
        rhs[j] = s;
    }
    // Delta = I - T_{-n}^T T_{-n} (= the Hessian at the optimum), w_{-n} = Delta^{-1} rhs, w_n = 0
    float h[Tri<N>::S], w[M];
    hessian<N>(T, h);
    SpdSolve<N>::run(h, rhs, w);
    // v = mu_r - T_{-n} w_{-n};  dH = -D = (G - v 1^T - 1 w^T) o T
    float out[N * N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float v = mur[i];
#pragma unroll
        for (int j = 0; j < M; ++j) v = fmaf(-T[i * N + j], w[j], v);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const float wj = (j < M) ? w[j] : 0.0f;
            out[i * N + j] = (G[i * N + j] - v - wj) * T[i * N + j];
        }
    }
    Storage<IO>::template store<N * N>(dH + b * (N * N), out);
}

// ---------------------------------------------------------------------------
// Baseline: a fixed number of Sinkhorn-Knopp sweeps in the log domain.
// ---------------------------------------------------------------------------
template <int N, typename IO>
__global__ void __launch_bounds__(kBlock)
sinkhorn_kernel(const IO* __restrict__ logits, IO* __restrict__ Tout, int64_t B, int sweeps) {
    const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (b >= B) return;
    float L[N * N];
    Storage<IO>::template load<N * N>(logits + b * (N * N), L);
#pragma unroll
    for (int k = 0; k < N * N; ++k) L[k] *= kLog2e;
    float a[N], z[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
        a[j] = 0.0f;
        z[j] = 0.0f;   // v^(0) = 1
    }
    for (int t = 0; t < sweeps; ++t) {
#pragma unroll
        for (int i = 0; i < N; ++i) {   // u = 1 / (A v): alpha_i = -LSE_j(H_ij + beta_j)
            float u[N];
#pragma unroll
            for (int j = 0; j < N; ++j) u[j] = L[i * N + j] + z[j];
            float mu = u[0];
#pragma unroll
            for (int j = 1; j < N; ++j) mu = fmaxf(mu, u[j]);
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < N; ++j) s += ex2(u[j] - mu);
            a[i] = -(mu + lg2(s));
        }
#pragma unroll
        for (int j = 0; j < N; ++j) {   // v = 1 / (A^T u): beta_j = -LSE_i(H_ij + alpha_i)
            float v[N];
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = L[i * N + j] + a[i];
            float m = v[0];
#pragma unroll
            for (int i = 1; i < N; ++i) m = fmaxf(m, v[i]);
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < N; ++i) s += ex2(v[i] - m);
            z[j] = -(m + lg2(s));
        }
    }
    float T[N * N];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int j = 0; j < N; ++j) T[i * N + j] = ex2(L[i * N + j] + a[i] + z[j]);
    Storage<IO>::template store<N * N>(Tout + b * (N * N), T);
}

}  // namespace birk
