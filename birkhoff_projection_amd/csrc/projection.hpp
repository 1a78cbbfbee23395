// projection.hpp -- device routines for the batched KL projection onto the
// Birkhoff polytope and its implicit backward pass (gfx950).
//
// Layout.  Each n x n matrix is held entirely in VGPRs by R adjacent lanes,
// each lane owning K = n / R of its rows: R = 1 for n = 4 (one matrix per
// lane, 64 per wave; 16 entries of T and the 6-entry Hessian triangle per
// lane) and R = 2 for n = 8 (a lane pair per matrix, 32 per wave, so that a
// lane's share of T, the 28-entry Hessian and its Cholesky factor fit three
// waves per SIMD without spilling).  Row-local work (softmaxes, row sums,
// trial-point updates) stays in the owning lane; column sums and the Hessian's
// dot products are completed with one DPP exchange inside the pair.  Both
// lanes of a pair then hold bit-identical copies of every per-matrix quantity
// (the exchange adds the two halves in either order, which is the same sum),
// so the Newton solve and the step-size search run redundantly in both and
// take identical decisions.  There is no MFMA: the work is tiny and
// independent per matrix.  LDS is used to make matrix loads and stores
// coalesced wave-wide accesses (WaveTile), in the fused kernel to land dL/dT
// while the iteration runs, and in the n = 4 forward to hand slow lanes to
// other waves of the workgroup.  Control flow is per lane (per pair); a wave
// keeps stepping while any of its matrices is unconverged.
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
// Sinkhorn-Knopp sweeps that give Newton's starting point (not counted as
// updates): kStartSweeps always, then up to kMoreSweeps more while the lane's
// column-sum residual is above kSweepOn.  A sweep costs a fifth of an update,
// and a wave runs until its slowest lane is done: on logits of large magnitude
// the far lanes hold their waves for several updates, on moderate ones
// (residuals of a few 1e-2 after three sweeps) no lane takes the extra sweeps.
// The decision is the lane's own, so a matrix's result does not depend on the
// other matrices of the batch.
// Measured: the hard-conditioning forward (B = 2^20, sigma in {1, 3, 5, 8})
// takes 84.6 us with no extra sweeps, 64.1 with these; the N(0, 10^2) forward at
// B = 512 / 8192 / 131072 (latency-bound: its slowest lanes set the time) 56 /
// 57 / 55 us before, 22 / 22 / 29 us with these; thresholds of 0.1 and 0.18 cost
// the hard workload 5-15 %; moderate workloads are unchanged within 1 %.
constexpr int kStartSweeps = 3;
constexpr int kMoreSweeps = 16;
constexpr float kSweepOn = 0.4f;

// lanes per matrix
template <int N>
struct Split {
    static constexpr int R = N == 8 ? 2 : 1;
    static constexpr int K = N / R;   // rows per lane
};

// Completing a per-matrix sum / maximum / product over the R lanes of a matrix.
template <int R>
struct Pair;

template <>
struct Pair<1> {
    __device__ __forceinline__ static float sum(float v) { return v; }
    __device__ __forceinline__ static float max(float v) { return v; }
    __device__ __forceinline__ static float min(float v) { return v; }
    __device__ __forceinline__ static float prod_m1(float q) { return q; }
};

template <>
struct Pair<2> {
    // the partner lane's value: DPP quad_perm [1,0,3,2] swaps lanes 2k and 2k+1.  Both
    // lanes of a pair are always active together (they hold the same per-matrix
    // state), so bound_ctrl changes no value; it lets the compiler fold the move
    // into the consuming add or max (one v_add_f32_dpp instead of two instructions).
    __device__ __forceinline__ static float other(float v) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
    }
    __device__ __forceinline__ static float sum(float v) { return v + other(v); }
    __device__ __forceinline__ static float max(float v) { return fmaxf(v, other(v)); }
    __device__ __forceinline__ static float min(float v) { return fminf(v, other(v)); }
    // (1 + q)(1 + q') - 1 for the two halves' partial products
    __device__ __forceinline__ static float prod_m1(float q) {
        const float o = other(q);
        return fmaf(q, o, q + o);
    }
};

// packed lower triangle of an (N-1) x (N-1) symmetric matrix
template <int N>
struct Tri {
    static constexpr int M = N - 1;
    static constexpr int S = M * (M + 1) / 2;
    __host__ __device__ static constexpr int at(int j, int k) { return j * (j + 1) / 2 + k; }  // k <= j
};

// Rows of T are Softmax(H_i. + beta) ([P] section 3.1), evaluated with the row
// maximum subtracted as in eq (10):  T_ij = 2^{L_ij + y_j - mu_i} / sum_k 2^{L_ik + y_k - mu_i},
// with y_{N-1} = 0.  Each row then sums to one up to rounding.  K rows.
template <int N, int K>
__device__ __forceinline__ void softmax_rows(const float (&L)[K * N], const float (&y)[N - 1], float (&T)[K * N]) {
#pragma unroll
    for (int i = 0; i < K; ++i) {
        float u[N];
#pragma unroll
        for (int j = 0; j < N - 1; ++j) u[j] = L[i * N + j] + y[j];
        u[N - 1] = L[i * N + N - 1];
        float mu = u[0];
#pragma unroll
        for (int j = 1; j < N; ++j) mu = fmaxf(mu, u[j]);
#pragma unroll
        for (int j = 0; j < N; ++j) u[j] = ex2(u[j] - mu);
        float s = u[0];
#pragma unroll
        for (int j = 1; j < N; ++j) s += u[j];
        const float r = rcp(s);
#pragma unroll
        for (int j = 0; j < N; ++j) T[i * N + j] = u[j] * r;
    }
}

// softmax_rows at beta = 0 (the starting point x^(0) = 0), from logits H in
// natural units.  The row maximum is taken before the scaling by log2 e: a
// positive scale keeps the order and rounding is monotone, so it is the
// maximum of the scaled row; each exponent is then one fma, H log2 e - mu.
// The maximum is IEEE 754-2019 `maximum` (gfx950's v_maximum3_f32, NaN
// propagating), which needs no quieting of the freshly loaded values first.
template <int N, int K>
__device__ __forceinline__ void softmax_rows0(const float (&H)[K * N], float (&T)[K * N]) {
#pragma unroll
    for (int i = 0; i < K; ++i) {
        float mu = H[i * N];
#pragma unroll
        for (int j = 1; j < N; ++j) mu = __builtin_elementwise_maximum(mu, H[i * N + j]);
        mu *= kLog2e;
        float u[N];
#pragma unroll
        for (int j = 0; j < N; ++j) u[j] = ex2(fmaf(H[i * N + j], kLog2e, -mu));
        float s = u[0];
#pragma unroll
        for (int j = 1; j < N; ++j) s += u[j];
        const float r = rcp(s);
#pragma unroll
        for (int j = 0; j < N; ++j) T[i * N + j] = u[j] * r;
    }
}

// column sums c_j = sum_i T_ij (eq 11); the gradient of the reduced dual is c_{-n} - 1 (eq 9)
template <int N>
__device__ __forceinline__ void col_sums(const float (&T)[Split<N>::K * N], float (&c)[N]) {
    // plain adds: T is held anyway, and fusing the products that formed it into
    // these sums would compute every product twice
#pragma clang fp contract(off)
    constexpr int K = Split<N>::K;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float s = T[j];
#pragma unroll
        for (int i = 1; i < K; ++i) s += T[i * N + j];
        c[j] = Pair<Split<N>::R>::sum(s);
    }
}

// max_j |c_j - 1| over all N columns; NaN propagates (IEEE 754-2019
// `maximum`, gfx950's v_maximum3_f32)
template <int N>
__device__ __forceinline__ float col_residual(const float (&c)[N]) {
    float r = fabsf(c[0] - 1.0f);
#pragma unroll
    for (int j = 1; j < N; ++j) r = __builtin_elementwise_maximum(r, fabsf(c[j] - 1.0f));
    return r;
}

// Entries of T below this are taken as possibly inexact.  The iteration moves T
// multiplicatively (trial points scale the columns of the current T), so an
// entry that has underflowed to zero, or lost bits as a subnormal, stays so; a
// T with an entry this small is therefore checked against its dual before it
// is accepted (newton_iterate).  2^-100 leaves 26 binades above the smallest
// normal number, and no entry this small can move a column sum by 1e-30.
constexpr float kTiny = 0x1.0p-100f;

// smallest entry of the matrix (over the R lanes that hold it); ordinary
// minimum: the callers only use it for matrices whose residual is finite
template <int N>
__device__ __forceinline__ float min_entry(const float (&T)[Split<N>::K * N]) {
    float m = T[0];
#pragma unroll
    for (int k = 1; k < Split<N>::K * N; ++k) m = fminf(m, T[k]);
    return Pair<Split<N>::R>::min(m);
}

// Hessian of the reduced dual objective, eq (9) with eta = 1, a = b = 1:
//   h_jk = [j == k] c_j - sum_i T_ij T_ik,   j, k < N-1.
// With the column Gram sums G_jk = sum_i T_ij T_ik (all N columns), the
// diagonal is evaluated as sum_{k != j} G_jk.  When every row of T sums to one
// this equals c_j - sum_i T_ij^2 (it is sum_i T_ij * (sum_{k != j} T_ik) with
// the two sums swapped), but it adds only non-negative terms, so it has no
// cancellation when a column is dominated by one entry close to 1; and the
// off-diagonal sums are the ones h needs anyway.  At the optimum this is also
// the Delta of eq (13) ([P] section 4.2).
template <int N>
__device__ __forceinline__ void hessian(const float (&T)[Split<N>::K * N], float (&h)[Tri<N>::S]) {
    constexpr int M = N - 1, K = Split<N>::K;
    using P = Pair<Split<N>::R>;
    // this lane's share of G_jk (k < j < M) and of G_jM
    float g[Tri<N>::S], gm[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
#pragma unroll
        for (int k = 0; k < j; ++k) {
            float p = T[j] * T[k];
#pragma unroll
            for (int i = 1; i < K; ++i) p = fmaf(T[i * N + j], T[i * N + k], p);
            g[Tri<N>::at(j, k)] = p;
        }
        float q = T[j] * T[M];
#pragma unroll
        for (int i = 1; i < K; ++i) q = fmaf(T[i * N + j], T[i * N + M], q);
        gm[j] = q;
    }
#pragma unroll
    for (int j = 0; j < M; ++j) {
        float d = gm[j];
#pragma unroll
        for (int k = 0; k < M; ++k)
            if (k != j) d += g[k < j ? Tri<N>::at(j, k) : Tri<N>::at(k, j)];
        h[Tri<N>::at(j, j)] = P::sum(d);
#pragma unroll
        for (int k = 0; k < j; ++k) h[Tri<N>::at(j, k)] = -P::sum(g[Tri<N>::at(j, k)]);
    }
}

// Adds 2^-22 tr(H) to the diagonal of the Newton system.  When some column of
// T is carried by a single entry near 1 (large-magnitude logits), the Hessian
// has an eigenvalue far below fp32 resolution (1e-8 relative, against a
// rounding level of 6e-8 in the gradient); the exact inverse then turns that
// rounding noise into a step of order one along the unresolvable direction,
// and the line search crawls.  The shift is below the rounding level of every
// entry of H, so resolvable directions keep their Newton step to within
// 2^-22 tr(H) / lambda relative, and the fixed point (g = 0) is unchanged.
template <int N>
__device__ __forceinline__ void damp(float (&h)[Tri<N>::S]) {
    float tr = h[Tri<N>::at(0, 0)];
#pragma unroll
    for (int j = 1; j < N - 1; ++j) tr += h[Tri<N>::at(j, j)];
    const float delta = tr * 0x1.0p-22f;
#pragma unroll
    for (int j = 0; j < N - 1; ++j) h[Tri<N>::at(j, j)] += delta;
}

// x = H^{-1} r for the symmetric positive definite (N-1) x (N-1) matrix H by a
// Cholesky factorisation H = L L^T in registers (backward stable: the computed
// x solves a system within a few ulps of H, however ill-conditioned).  Returns
// false when H is not numerically positive definite (a non-positive or
// non-finite pivot); x is then meaningless.  The Hessians solved here have
// bounded entries (at most n for the Birkhoff kernels, whose T lies in [0, 1];
// at most the total of the marginals a in the general problem), so for finite
// inputs a pivot is finite or NaN, and one comparison with the smallest
// normal number (false for NaN) decides.
template <int N>
struct CholSolve {
    // min_pivot: pivots at or below it count as failure (default: the smallest
    // normal number)
    __device__ __forceinline__ static bool run(const float (&h)[Tri<N>::S], const float (&r)[N - 1], float (&x)[N - 1],
                                               float min_pivot = 1.17549435e-38f) {
        constexpr int M = N - 1;
        float l[Tri<N>::S];   // Cholesky factor, packed lower triangle
        float dinv[M];        // 1 / l_jj
        bool ok = true;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            float s = h[Tri<N>::at(j, j)];
#pragma unroll
            for (int k = 0; k < j; ++k) s = fmaf(-l[Tri<N>::at(j, k)], l[Tri<N>::at(j, k)], s);
            ok = ok && (s > min_pivot);
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

// The Newton system of the forward: N = 4 uses the closed-form adjugate of
// eq (12), other N the Cholesky solve.  Same contract as CholSolve (false when
// the determinant is not a positive normal number).
template <int N>
struct SpdSolve : CholSolve<N> {};

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
        return det > 1.17549435e-38f;
    }
};

// Solves Delta w = rhs for eq (13)'s w_{-n}, Delta being the Hessian at the
// projection (entries at most `unit` in magnitude: 1 here, the total mass of
// the marginals in the general problem), formed by `fill(h)` as a packed lower
// triangle.  Near a permutation Delta is numerically singular: its entries
// that involve rows and columns carried by one entry near 1 are tiny or zero.
// The system stays consistent there (rhs vanishes along the same directions,
// up to its rounding, a few ulps of |G o T|), and dH = (G - v 1^T - 1 w^T) o T
// does not depend on the component of w along them -- at an exact permutation
// Delta = 0, rhs = 0 and dH = 0 for every w -- but the plain solution puts
// rhs's rounding / lambda into that component, and a w that large leaves its
// own rounding in dH.  So:
//   - first Delta is factored as it is, and a Cholesky pivot at or below
//     2^-24 unit (one ulp of the entry bound) counts as failure.  The pivots
//     are at least lambda_min(Delta), so every Delta that fp32 resolves is
//     solved exactly as eq (13) says, and its w carries at most a few |G o T|
//     of rounding;
//   - otherwise the solve is repeated with 2^-20 (unit + tr Delta) added to
//     the diagonal (16 ulps of the entry bound and of the trace), which keeps
//     what rounding can put into w within |G o T| and covers the rounding of
//     Delta's diagonal (at most n - 2 ulps of the trace: Delta is a grounded
//     Laplacian of the column Gram sums, diagonally dominant up to that), so
//     that its pivots stay above 2^-25 unit.  fill is called again for it, so
//     that h need not stay live through the first factorisation;
//   - it fails then only when Delta is not finite (a non-finite T): w = 0, and
//     the NaN stays in dH.
// The solve is the Cholesky one for every n: eq (13) needs Delta^{-1} rhs, not
// eq (12)'s closed form, and Cramer's rule (the adjugate) is not backward
// stable -- on a nearly singular 3 x 3 Delta its solution misses the system by
// a fraction of rhs.
template <int N, typename Fill>
__device__ __forceinline__ void solve_delta(Fill fill, const float (&rhs)[N - 1], float (&w)[N - 1],
                                            float unit = 1.0f) {
    float shift = 0.0f, min_pivot = unit * 0x1.0p-24f;   // the first attempt: Delta as it is
#pragma unroll 1
    for (int attempt = 0; attempt < 2; ++attempt) {
        float h[Tri<N>::S];
        fill(h);
        float tr = h[Tri<N>::at(0, 0)];
#pragma unroll
        for (int j = 1; j < N - 1; ++j) tr += h[Tri<N>::at(j, j)];
        const float delta = (unit + tr) * shift;
#pragma unroll
        for (int j = 0; j < N - 1; ++j) h[Tri<N>::at(j, j)] += delta;
        if (CholSolve<N>::run(h, rhs, w, min_pivot)) return;
        shift = 0x1.0p-20f;
        min_pivot = unit * 0x1.0p-25f;
    }
#pragma unroll
    for (int j = 0; j < N - 1; ++j) w[j] = 0.0f;
}

// Trial point x + s of the line search (natural units, s_{N-1} = 0), evaluated
// from the current T instead of from the logits.  Rows of T are softmaxes of
// H_i. + beta, so moving beta by s multiplies column j by e^{s_j} before the
// rows are normalised again:
//     T'_ij = (T_ij e^{s_j}) r_i,   r_i = 1 / sum_k T_ik e^{s_k}     (N-1 exponentials, not N^2).
// The same row sums give the change of the objective by the exact identity
//     f(x + s) - f(x) = sum_i log(sum_j T_ij e^{s_j}) - sum_j s_j,
// which follows from f = n + sum_i LSE_i(H_i. + beta) - sum_j beta_j (eq 8 with
// eq 5).  For a small step the sum of logarithms nearly cancels the sum of
// steps, so it is taken as log1p(q), q = prod_i (1 + a_i) - 1 with
// a_i = sum_j T_ij expm1(s_j) (rows of T sum to one), accumulated as
// q <- q + a_i + q a_i, which keeps its relative accuracy as the step shrinks.
// Otherwise (|q| >= 1/16) the logarithms of the row sums themselves are added.
// T' itself is not formed: the column sums ct of T' (for the gradient
// test) are accumulated row by row, and e, r are returned so that an accepted
// trial is applied to T in place by accept_trial.  Returns f(x + s) - f(x);
// `noise` receives 2^-21 times the magnitude of the two terms it is the
// difference of, the level below which fp32 cannot resolve its sign.
template <int N>
__device__ __forceinline__ float trial_point(const float (&T)[Split<N>::K * N], const float (&s)[N - 1],
                                             float (&e)[N - 1], float (&r)[Split<N>::K], float (&ct)[N],
                                             float& noise) {
    constexpr int M = N - 1, K = Split<N>::K;
    using P = Pair<Split<N>::R>;
    float em[M];
    float ssum = s[0];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        e[j] = ex2(s[j] * kLog2e);
        em[j] = expm1_from(s[j], e[j]);
        if (j > 0) ssum += s[j];
    }
    float q;   // prod_i (1 + a_i) - 1
#pragma unroll
    for (int i = 0; i < K; ++i) {
        float t = T[i * N] * em[0];
#pragma unroll
        for (int j = 1; j < M; ++j) t = fmaf(T[i * N + j], em[j], t);
        q = (i == 0) ? t : fmaf(q, t, q + t);
    }
    q = P::prod_m1(q);
    float lsum = 0.0f;   // sum_i log2(rs_i), used when the step is not small
#pragma unroll
    for (int i = 0; i < K; ++i) {
        float u[M];
        float rs = T[i * N + M];
#pragma unroll
        for (int j = 0; j < M; ++j) {
            u[j] = T[i * N + j] * e[j];
            rs += u[j];
        }
        r[i] = rcp(rs);
        lsum = (i == 0) ? lg2(rs) : lsum + lg2(rs);
#pragma unroll
        for (int j = 0; j < M; ++j) ct[j] = (i == 0) ? u[j] * r[i] : ct[j] + u[j] * r[i];
        ct[M] = (i == 0) ? T[i * N + M] * r[i] : ct[M] + T[i * N + M] * r[i];
    }
#pragma unroll
    for (int j = 0; j < N; ++j) ct[j] = P::sum(ct[j]);
    const float l = fabsf(q) < 0.0625f ? log1p_series(q) : P::sum(lsum) * kLn2;
    noise = (fabsf(l) + fabsf(ssum)) * 0x1.0p-21f;
    return l - ssum;
}

template <int N>
__device__ __forceinline__ void accept_trial(float (&T)[Split<N>::K * N], const float (&e)[N - 1],
                                             const float (&r)[Split<N>::K]) {
    constexpr int M = N - 1, K = Split<N>::K;
#pragma unroll
    for (int i = 0; i < K; ++i) {
#pragma unroll
        for (int j = 0; j < M; ++j) T[i * N + j] = (T[i * N + j] * e[j]) * r[i];
        T[i * N + M] *= r[i];
    }
}

// One Sinkhorn-Knopp sweep in the log domain (eq 7 = eq 2), used as the fallback
// when no step size is accepted: alpha = alpha*(beta) (eq 5, row log-sum-exp),
// then beta = beta*(alpha) (eq 6, column log-sum-exp), re-gauged to beta_{N-1} = 0.
// Base-2 units throughout; no column sum is ever formed, so an underflowed
// column cannot produce log(0).
template <int N>
__device__ __forceinline__ void sinkhorn_sweep(const float (&L)[Split<N>::K * N], float (&y)[N - 1]) {
    constexpr int K = Split<N>::K;
    using P = Pair<Split<N>::R>;
    float a[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        float u[N];
#pragma unroll
        for (int j = 0; j < N - 1; ++j) u[j] = L[i * N + j] + y[j];
        u[N - 1] = L[i * N + N - 1];
        float mu = u[0];
#pragma unroll
        for (int j = 1; j < N; ++j) mu = fmaxf(mu, u[j]);
        float s = ex2(u[0] - mu);
#pragma unroll
        for (int j = 1; j < N; ++j) s += ex2(u[j] - mu);
        a[i] = -(mu + lg2(s));
    }
    float z[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float v[K];
#pragma unroll
        for (int i = 0; i < K; ++i) v[i] = L[i * N + j] + a[i];
        float m = v[0];
#pragma unroll
        for (int i = 1; i < K; ++i) m = fmaxf(m, v[i]);
        m = P::max(m);
        float s = ex2(v[0] - m);
#pragma unroll
        for (int i = 1; i < K; ++i) s += ex2(v[i] - m);
        z[j] = -(m + lg2(P::sum(s)));
    }
#pragma unroll
    for (int j = 0; j < N - 1; ++j) y[j] = z[j] - z[N - 1];
}

__device__ __forceinline__ float step_size(int k) {
    // the blog's step sizes, tried in this order
    return k == 0 ? 1.0f : k == 1 ? 0.5f : k == 2 ? 0.1f : k == 3 ? 0.05f : 0.01f;
}

// ---------------------------------------------------------------------------
// Kernel geometry.  A workgroup is kBlock lanes = kWaves waves.  Lane l of
// wave w of workgroup g owns "item" (g*kWaves + w)*64 + l: rows
// [h*K, (h+1)*K) of matrix item / R, h = item mod R.  Items are contiguous in
// memory (K*n elements each), so a wave's items form one span; matrix I/O goes
// through the wave's private LDS tile (WaveTile) so that every global access
// instruction is coalesced.  The dual (n floats per matrix) and the iteration
// counts are already contiguous across lanes and are accessed directly.
// Lanes past the end of the batch compute on zeros and store nothing; whole
// waves past the end return at once.
// ---------------------------------------------------------------------------
constexpr int kWaves = kBlock / 64;

template <int N, typename IO>
struct Geometry {
    static constexpr int R = Split<N>::R, K = Split<N>::K;
    static constexpr int C = K * N * (int)sizeof(IO) / 16;   // 16-byte chunks per item
    static_assert(C * 16 == K * N * (int)sizeof(IO), "an item must be a whole number of 16-byte chunks");
    using Tile = WaveTile<C>;
    int lane, wave, nvalid;   // nvalid: items of this wave inside the batch (wave-uniform)
    int64_t base;             // first item of this wave
    __device__ __forceinline__ Geometry(int64_t B) {
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: base and the tile offsets go to SGPRs
        base = ((int64_t)blockIdx.x * kWaves + wave) * 64;
        const int64_t left = B * R - base;
        nvalid = __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : left >= 64 ? 64 : (int)left);
    }
    // one wave whose first item is `first` (wave-uniform) and which takes at most
    // `span` <= 64 items, for kernels where a single wave of the workgroup projects
    __device__ __forceinline__ Geometry(int64_t B, int64_t first, int span) {
        lane = threadIdx.x & 63;
        wave = 0;
        base = first;
        const int64_t left = B * R - base;
        nvalid = __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : left >= span ? span : (int)left);
    }
    __device__ __forceinline__ bool valid() const { return lane < nvalid; }
    __device__ __forceinline__ int half() const { return lane & (R - 1); }            // which rows of the matrix
    __device__ __forceinline__ int64_t matrix() const { return (base + lane) / R; }
    __device__ __forceinline__ int64_t item() const { return base + lane; }
    __device__ __forceinline__ const uint4* chunks(const IO* p) const {
        return reinterpret_cast<const uint4*>(p) + base * C;
    }
    __device__ __forceinline__ uint4* chunks(IO* p) const { return reinterpret_cast<uint4*>(p) + base * C; }
};

// The dual entries [h*K, (h+1)*K) of matrix b, as K/4 16-byte stores.
template <int N>
__device__ __forceinline__ void store_dual(float* __restrict__ dual, int64_t b, int h, const float (&beta)[N]) {
    constexpr int K = Split<N>::K;
    uint4* q = reinterpret_cast<uint4*>(dual + b * N + h * K);
#pragma unroll
    for (int k = 0; k < K / 4; ++k) {
        uint4 v = make_uint4(__float_as_uint(beta[4 * k]), __float_as_uint(beta[4 * k + 1]),
                             __float_as_uint(beta[4 * k + 2]), __float_as_uint(beta[4 * k + 3]));
        if constexpr (Split<N>::R == 2) {
            // the second lane of the pair stores the upper half (selected, not indexed by h,
            // so that beta stays in registers)
            const uint4 u = make_uint4(__float_as_uint(beta[K + 4 * k]), __float_as_uint(beta[K + 4 * k + 1]),
                                       __float_as_uint(beta[K + 4 * k + 2]), __float_as_uint(beta[K + 4 * k + 3]));
            v.x = h ? u.x : v.x;
            v.y = h ? u.y : v.y;
            v.z = h ? u.z : v.z;
            v.w = h ? u.w : v.w;
        }
        stream_store(q + k, v);
    }
}

template <int N>
__device__ __forceinline__ void load_dual(const float* __restrict__ dual, int64_t b, float (&beta)[N]) {
    const uint4* q = reinterpret_cast<const uint4*>(dual + b * N);
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        const uint4 t = stream_load(q + k);
        beta[4 * k] = __uint_as_float(t.x);
        beta[4 * k + 1] = __uint_as_float(t.y);
        beta[4 * k + 2] = __uint_as_float(t.z);
        beta[4 * k + 3] = __uint_as_float(t.w);
    }
}

// Where a lane's item index comes from, for the rare paths that re-read its
// logits.  WaveItem: the wave's first item (wave-uniform, in scalar registers)
// plus the lane's id, recomputed where it is needed instead of held in vector
// registers through the iteration.  LaneItem: an arbitrary item per lane (the
// gathered stragglers).
struct WaveItem {
    int64_t base;
    __device__ __forceinline__ int64_t get() const { return base + (int64_t)__lane_id(); }
};
struct LaneItem {
    int64_t item;
    __device__ __forceinline__ int64_t get() const { return item; }
};

// One lane reads its own item directly (used off the main path, where the
// other lanes of the wave do not take part).
template <int N, typename IO>
__device__ __forceinline__ void load_own(const IO* __restrict__ p, int64_t item, float (&v)[Split<N>::K * N]) {
    constexpr int KN = Split<N>::K * N;
    constexpr int C = KN * (int)sizeof(IO) / 16;
    const uint4* q = reinterpret_cast<const uint4*>(p) + item * C;
    uint4 w[C];
#pragma unroll
    for (int k = 0; k < C; ++k) w[k] = q[k];
    Storage<IO>::template decode<KN>(w, v);
}

// ---------------------------------------------------------------------------
// Forward: Newton on the reduced dual (eq 8).
// ---------------------------------------------------------------------------

// Newton's method on the reduced dual (eq 8) from the lane's current iterate
// (T, y, its column sums c and residual res, it updates so far) until the
// column-sum residual is <= tol or it reaches max_iter.  `item` is the lane's
// item index, whose logits the rare fallback sweep re-reads; `sweeps` counts
// the fallback sweeps taken.
//
// Checked convergence.  Rows of T are Softmax(H_i. + beta) ([P] section 3.1),
// and the projection is the unique doubly stochastic matrix of that form ([P]
// section 2.2, eq 1).  The iteration forms T multiplicatively (a trial point
// scales the columns of the current T), which keeps every entry's relative
// accuracy except for entries that underflow: logit spans beyond about 100
// give row softmaxes with entries below 2^-149, which stay zero, and subnormal
// ones keep a few bits, so the iteration could converge to the projection of a
// different matrix.  A lane that converges with an entry below kTiny, or that
// started with one (`wide`, set by newton_start), therefore rebuilds T from
// the logits at its dual once (`checked`) and goes on iterating from it:
// entries lost on the way are back, and since the rebuilt T is exactly of the
// form above at the fp32 dual, one or two more updates bring its column sums
// (off by the dual's accumulated rounding) back within tol, or, with lost mass,
// the iteration continues until they are.  Updates are counted as before; a
// lane whose check falls on its last allowed update ends with count -1 if the
// rebuilt T misses tol.  Lanes whose entries all stay above kTiny -- every
// benchmark input -- take none of this.
// One update of newton_iterate: the Newton step with the line search, or the
// fallback sweep when no step size is accepted.
template <int N, typename IO, typename Item>
__device__ __forceinline__ void newton_update(const IO* __restrict__ logits, Item item, float (&T)[Split<N>::K * N],
                                              float (&y)[N - 1], float (&c)[N], float& res, int& it, int& sweeps) {
    constexpr int M = N - 1, K = Split<N>::K;
    float g[M], r[M], d[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        g[j] = c[j] - 1.0f;
        r[j] = -g[j];
    }
    float gn2 = g[0] * g[0];
#pragma unroll
    for (int j = 1; j < M; ++j) gn2 = fmaf(g[j], g[j], gn2);
    float h[Tri<N>::S];
    hessian<N>(T, h);
    damp<N>(h);
    const bool ok = SpdSolve<N>::run(h, r, d);   // d = -H^{-1} g

    bool accepted = false;
    if (ok) {
        for (int k = 0; k < 5; ++k) {
            const float gam = step_size(k);
            float s[M], e[M], rr[K], ct[N];
#pragma unroll
            for (int j = 0; j < M; ++j) s[j] = gam * d[j];
            float noise;
            const float df = trial_point<N>(T, s, e, rr, ct, noise);
            float gt2 = (ct[0] - 1.0f) * (ct[0] - 1.0f);
#pragma unroll
            for (int j = 1; j < M; ++j) gt2 = fmaf(ct[j] - 1.0f, ct[j] - 1.0f, gt2);
            // the objective must not increase beyond what fp32 can resolve, and
            // the gradient norm must decrease
            if (df < noise && gt2 < gn2) {
#pragma unroll
                for (int j = 0; j < M; ++j) y[j] = fmaf(s[j], kLog2e, y[j]);
                accept_trial<N>(T, e, rr);
#pragma unroll
                for (int j = 0; j < N; ++j) c[j] = ct[j];
                accepted = true;
                break;
            }
        }
    }
    if (!accepted) {
        float L[K * N];
        load_own<N, IO>(logits, item.get(), L);
#pragma unroll
        for (int k = 0; k < K * N; ++k) L[k] *= kLog2e;
        sinkhorn_sweep<N>(L, y);
        softmax_rows<N, K>(L, y, T);
        col_sums<N>(T, c);
        ++sweeps;
    }
    ++it;
    res = col_residual<N>(c);
}

// The check of a converged lane (see newton_iterate): true when the lane is done;
// otherwise T has been rebuilt from the logits at its dual, with its column sums
// and residual, and the iteration goes on from it.
template <int N, typename IO, typename Item>
__device__ __forceinline__ bool converged_or_rebuilt(const IO* __restrict__ logits, Item item, float tol,
                                                     float (&T)[Split<N>::K * N], const float (&y)[N - 1],
                                                     float (&c)[N], float& res, bool& wide, bool& checked) {
    constexpr int K = Split<N>::K;
    if (!(res <= tol) || checked || (!wide && min_entry<N>(T) >= kTiny)) return true;
    checked = true;
    wide = false;
    float L[K * N];
    load_own<N, IO>(logits, item.get(), L);
#pragma unroll
    for (int k = 0; k < K * N; ++k) L[k] *= kLog2e;
    softmax_rows<N, K>(L, y, T);
    col_sums<N>(T, c);
    res = col_residual<N>(c);
    return false;
}

template <int N, typename IO, bool kOneLoop = (Split<N>::R == 1), typename Item>
__device__ __forceinline__ void newton_iterate(const IO* __restrict__ logits, Item item, float tol, int max_iter,
                                               float (&T)[Split<N>::K * N], float (&y)[N - 1], float (&c)[N],
                                               float& res, int& it, bool& wide, bool& checked, int& sweeps) {
    // The same iteration in two loop shapes, chosen by measurement per kernel.
    // kOneLoop: a single loop with the check on its exit path, and the update
    // written out in it (the same steps as newton_update; called through a
    // function, inlined or not, the update costs one matrix per lane a wave of
    // occupancy); an inner loop around the check makes the compiler copy T at
    // every update.  Otherwise the updates run in an inner loop and the check
    // after it: lane pairs spill in the single loop, and the gather kernel,
    // which holds two copies of the iteration, runs faster this way.
    if constexpr (kOneLoop) {
        constexpr int K = Split<N>::K;
        for (;;) {
            if (!(res > tol && it < max_iter)) {
                if (!(res <= tol) || checked || (!wide && min_entry<N>(T) >= kTiny)) break;
                checked = true;
                wide = false;
                float L[K * N];
                load_own<N, IO>(logits, item.get(), L);
#pragma unroll
                for (int k = 0; k < K * N; ++k) L[k] *= kLog2e;
                softmax_rows<N, K>(L, y, T);
                col_sums<N>(T, c);
                res = col_residual<N>(c);
                continue;
            }
            constexpr int M = N - 1;
            float g[M], r[M], d[M];
#pragma unroll
            for (int j = 0; j < M; ++j) {
                g[j] = c[j] - 1.0f;
                r[j] = -g[j];
            }
            float gn2 = g[0] * g[0];
#pragma unroll
            for (int j = 1; j < M; ++j) gn2 = fmaf(g[j], g[j], gn2);
            float h[Tri<N>::S];
            hessian<N>(T, h);
            damp<N>(h);
            const bool ok = SpdSolve<N>::run(h, r, d);   // d = -H^{-1} g

            bool accepted = false;
            if (ok) {
                for (int k = 0; k < 5; ++k) {
                    const float gam = step_size(k);
                    float s[M], e[M], rr[K], ct[N];
#pragma unroll
                    for (int j = 0; j < M; ++j) s[j] = gam * d[j];
                    float noise;
                    const float df = trial_point<N>(T, s, e, rr, ct, noise);
                    float gt2 = (ct[0] - 1.0f) * (ct[0] - 1.0f);
#pragma unroll
                    for (int j = 1; j < M; ++j) gt2 = fmaf(ct[j] - 1.0f, ct[j] - 1.0f, gt2);
                    // the objective must not increase beyond what fp32 can resolve, and
                    // the gradient norm must decrease
                    if (df < noise && gt2 < gn2) {
#pragma unroll
                        for (int j = 0; j < M; ++j) y[j] = fmaf(s[j], kLog2e, y[j]);
                        accept_trial<N>(T, e, rr);
#pragma unroll
                        for (int j = 0; j < N; ++j) c[j] = ct[j];
                        accepted = true;
                        break;
                    }
                }
            }
            if (!accepted) {
                float L[K * N];
                load_own<N, IO>(logits, item.get(), L);
#pragma unroll
                for (int k = 0; k < K * N; ++k) L[k] *= kLog2e;
                sinkhorn_sweep<N>(L, y);
                softmax_rows<N, K>(L, y, T);
                col_sums<N>(T, c);
                ++sweeps;
            }
            ++it;
            res = col_residual<N>(c);
        }
    } else {
        for (;;) {
            while (res > tol && it < max_iter) newton_update<N, IO>(logits, item, T, y, c, res, it, sweeps);
            if (converged_or_rebuilt<N, IO>(logits, item, tol, T, y, c, res, wide, checked)) break;
        }
    }
}

// Loads the wave's logits and evaluates the start x^(0) (kStartSweeps
// Sinkhorn sweeps from beta = 0): T (the lane's rows), y (base-2 dual,
// y_{N-1} = 0 implied), c (column sums of T) and res (their residual; 0 for
// lanes past the end of the batch, which are thereby done).  `wide` is set
// when an entry of this T is below kTiny (logit spans of about 70 or more),
// so that newton_iterate checks the converged T against its dual.  The logits
// are needed again only by the rare fallback sweep and that check, which
// re-read this lane's rows; they do not stay in registers through the
// iteration.
template <int N, typename IO, bool kPrefetch = false>
__device__ __forceinline__ void newton_start(const Geometry<N, IO>& geo, uint4* lds, const IO* __restrict__ logits,
                                             float (&T)[Split<N>::K * N], float (&y)[N - 1], float (&c)[N],
                                             float& res, bool& wide, const IO* __restrict__ prefetch_src = nullptr) {
    constexpr int M = N - 1, K = Split<N>::K;
    using G = Geometry<N, IO>;
    {
        float H[K * N];
        uint4 w[G::C];
        G::Tile::load(geo.chunks(logits), geo.nvalid * G::C, lds, geo.lane, w);
        Storage<IO>::template decode<K * N>(w, H);
        softmax_rows0<N, K>(H, T);
    }
    // optionally start copying another tile of the wave (dL/dT) into the now
    // free LDS region, to be read after the iteration
    if constexpr (kPrefetch) G::Tile::prefetch(geo.chunks(prefetch_src), geo.nvalid * G::C, lds, geo.lane);
    // start: the dual after kStartSweeps Sinkhorn-Knopp sweeps from v = 1.  The
    // rows of exp(H) are normalised above (T at beta = 0); each sweep scales the
    // columns of T to sum to one and normalises the rows again, which moves the
    // dual by beta_j += log c_{n-1} - log c_j.  The sweeps are skipped when a
    // column sum of this T is 0 or not finite: rows sum to one, so a column sum
    // is at most n or NaN, and one comparison per column (false for NaN) decides.
    // After one sweep no later sweep can fail that test: every column of
    // T diag(1/c) sums to one and no row of it sums to more than n (each entry
    // T_ij / c_j is at most 1), so every column sum of the renormalised T is at
    // least 1/n.  The later sweeps' ratios c_{n-1} / c_j therefore lie within
    // [n^-2, n^2]; their product is formed and its logarithm taken once.
    static_assert(kStartSweeps >= 1, "the start has at least one sweep");
#pragma unroll
    for (int j = 0; j < M; ++j) y[j] = 0.0f;
    col_sums<N>(T, c);
    bool ok = true;
#pragma unroll
    for (int j = 0; j < N; ++j) ok = ok && c[j] > 1.17549435e-38f;
    if (ok) {
        float q[M];   // product of the later sweeps' ratios
        // one sweep with c the column sums of T: scale the columns to sum to one and
        // renormalise the rows; the first sweep sets y, later ones multiply into q
        auto sweep = [&](bool first_sweep, bool second_sweep) __attribute__((always_inline)) {
            float rc[N];
#pragma unroll
            for (int j = 0; j < N; ++j) rc[j] = rcp(c[j]);
#pragma unroll
            for (int j = 0; j < M; ++j) {
                const float ratio = c[N - 1] * rc[j];
                if (first_sweep) y[j] = lg2(ratio);
                else q[j] = second_sweep ? ratio : q[j] * ratio;
            }
#pragma unroll
            for (int i = 0; i < K; ++i) {
#pragma clang fp contract(off)
                // (plain adds of the scaled entries, which are kept)
#pragma unroll
                for (int j = 0; j < N; ++j) T[i * N + j] *= rc[j];
                float rs = T[i * N];
#pragma unroll
                for (int j = 1; j < N; ++j) rs += T[i * N + j];
                const float r = rcp(rs);
#pragma unroll
                for (int j = 0; j < N; ++j) T[i * N + j] *= r;
            }
        };
#pragma unroll
        for (int sw = 0; sw < kStartSweeps; ++sw) {
            if (sw > 0) col_sums<N>(T, c);
            sweep(sw == 0, sw == 1);
        }
        // the extra sweeps (q multiplies up to kStartSweeps + kMoreSweeps - 1 ratios
        // in [n^-2, n^2]: at most 2^108 for n = 8, inside fp32's range); both lanes
        // of a pair hold the same column sums and decide alike
        static_assert((kStartSweeps + kMoreSweeps - 1) * 2 * (N == 8 ? 3 : 2) < 127, "q stays finite");
        // (leaves c the column sums of the final T)
#pragma unroll 1
        for (int sw = 0;; ++sw) {
            col_sums<N>(T, c);
            if (sw == kMoreSweeps || !(col_residual<N>(c) > kSweepOn)) break;
            sweep(false, kStartSweeps == 1 && sw == 0);
        }
        if constexpr (kStartSweeps + kMoreSweeps > 1)
#pragma unroll
            for (int j = 0; j < M; ++j) y[j] += lg2(q[j]);
    }
    // c holds the column sums of T on either path (T is unchanged when the sweeps are skipped)
    res = geo.valid() ? col_residual<N>(c) : 0.0f;   // lanes past the end are done
    wide = geo.valid() && min_entry<N>(T) < kTiny;
}

// newton_start, then Newton's method to column-sum residual <= tol or max_iter
// updates.  On return T is the lane's rows of the last iterate, y the dual
// (base-2 units, y_{N-1} = 0 implied), res its residual, `sweeps` the number
// of fallback sweeps among the updates; returns the number of updates.
template <int N, typename IO, bool kPrefetch = false>
__device__ __forceinline__ int newton_solve(const Geometry<N, IO>& geo, uint4* lds, const IO* __restrict__ logits,
                                            float tol, int max_iter, float (&T_out)[Split<N>::K * N],
                                            float (&y_out)[N - 1], float& res_out, int& sweeps,
                                            const IO* __restrict__ prefetch_src = nullptr) {
    constexpr int M = N - 1, K = Split<N>::K;
    // the iteration works on locals, copied out at the end (keeps the loop in registers)
    float T[K * N], y[M], c[N], res;
    bool wide, checked = false;
    newton_start<N, IO, kPrefetch>(geo, lds, logits, T, y, c, res, wide, prefetch_src);
    int it = 0;
    sweeps = 0;
    newton_iterate<N, IO>(logits, WaveItem{geo.base}, tol, max_iter, T, y, c, res, it, wide, checked, sweeps);
#pragma unroll
    for (int k = 0; k < K * N; ++k) T_out[k] = T[k];
#pragma unroll
    for (int j = 0; j < M; ++j) y_out[j] = y[j];
    res_out = res;
    return it;
}

// Writes the wave's T through its LDS tile and, per valid lane, the lane's
// share of the dual (natural units, beta_{N-1} = 0).
template <int N, typename IO, bool kPin = true>
__device__ __forceinline__ void store_forward(const Geometry<N, IO>& geo, uint4* lds, IO* __restrict__ Tout,
                                              float* __restrict__ dual, const float (&T)[Split<N>::K * N],
                                              const float (&y)[N - 1]) {
    using G = Geometry<N, IO>;
    {
        uint4 w[G::C];
        Storage<IO>::template encode<G::K * N>(T, w);
        G::Tile::template store<kPin>(w, lds, geo.lane, geo.chunks(Tout), geo.nvalid * G::C);
    }
    if (geo.valid()) {
        float beta[N];
#pragma unroll
        for (int j = 0; j < N - 1; ++j) beta[j] = y[j] * kLn2;
        beta[N - 1] = 0.0f;
        store_dual<N>(dual, geo.matrix(), geo.half(), beta);
    }
}

template <int N, typename IO, bool kStats>
__global__ void __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(N == 4 ? 7 : 3)))
newton_fwd_kernel(const IO* __restrict__ logits, IO* __restrict__ Tout, float* __restrict__ dual,
                  int32_t* __restrict__ iters, int32_t* __restrict__ fallbacks, int64_t B, float tol,
                  int max_iter) {
    using G = Geometry<N, IO>;
    __shared__ uint4 lds[kWaves][G::Tile::kLdsChunks];
    const G geo(B);
    if (geo.nvalid == 0) return;
    float T[G::K * N], y[N - 1], res;
    int sweeps;
    const int it = newton_solve<N, IO>(geo, lds[geo.wave], logits, tol, max_iter, T, y, res, sweeps);
    store_forward<N, IO>(geo, lds[geo.wave], Tout, dual, T, y);
    if (kStats && geo.valid() && geo.half() == 0) {
        iters[geo.matrix()] = (res <= tol) ? it : -1;
        if (fallbacks) fallbacks[geo.matrix()] = sweeps;
    }
}

// ---------------------------------------------------------------------------
// Forward with the slow lanes gathered (n = 4, one matrix per lane).
//
// The number of Newton updates differs from matrix to matrix, and a wave runs
// until its slowest lane is done; on inputs with a long tail (logits of large
// magnitude) most lanes of a wave sit idle for most of its updates.  Here each
// wave first runs at most kFirstPass updates and stores the matrices that are
// done.  A wave with at most kHandOff lanes still running ("slow" lanes) hands
// their state (T, dual, column sums) to the workgroup through its LDS region;
// a wave with more keeps them.  After a workgroup barrier the waves that handed
// off (or had nothing left) take the handed-off states 64 to a wave and carry
// them on to tol or max_iter, while the rest exit, so that the updates of the
// tail are spent on fewer waves.  Every matrix goes through exactly the updates
// of the fused kernel's forward from the same state (the loop shapes differ, the
// arithmetic of each update does not), so T and the dual are bit-identical.
// ---------------------------------------------------------------------------
constexpr int kFirstPass = 4;   // updates before the slow lanes are gathered
constexpr int kHandOff = 32;    // most slow lanes a wave hands to the workgroup

template <typename IO>
struct Gather {
    static constexpr int N = 4, M = N - 1, KN = Split<N>::K * N;
    static_assert(Split<N>::R == 1, "one matrix per lane");
    using G = Geometry<N, IO>;
    // one handed-off state: T, y, c and a word holding the owner's lane in the
    // workgroup (bits 0-7), its `wide` and `checked` flags (bits 8 and 9) and, when
    // counted, its fallback sweeps so far (bits 10 and up); word j of record p sits
    // at float j * kHandOff + p of the wave's region
    static constexpr int kWords = KN + M + N + 1;
    static constexpr int kRecordChunks = (kWords * kHandOff * 4 + 15) / 16;
    static constexpr int kRegion = G::Tile::kLdsChunks > kRecordChunks ? G::Tile::kLdsChunks : kRecordChunks;
};

// The dual of every matrix of the workgroup is collected in LDS and written out
// as one contiguous block by the wave that finishes last (an LDS counter says
// which): a gathered lane's 16-byte dual alone would be a partial write to HBM,
// and so would the fast lanes' around it.
template <typename IO, bool kStats>
__global__ void __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kStats ? 6 : 7)))
newton_fwd_gather_kernel(const IO* __restrict__ logits, IO* __restrict__ Tout, float* __restrict__ dual,
                         int32_t* __restrict__ iters, int32_t* __restrict__ fallbacks, int64_t B, float tol,
                         int max_iter) {
    using Q = Gather<IO>;
    constexpr int N = Q::N, M = Q::M, KN = Q::KN;
    using G = typename Q::G;
    __shared__ uint4 lds[kWaves][Q::kRegion];
    __shared__ uint4 duals[kBlock];   // the workgroup's duals, by matrix
    __shared__ int handed[kWaves];    // states a wave handed off; -1: it keeps its slow lanes
    __shared__ int finished;          // waves done with their matrices
    const G geo(B);
    const int first = max_iter < kFirstPass ? max_iter : kFirstPass;
    float T[KN], y[M], c[N], res = 0.0f;
    int it = 0, sweeps = 0;
    bool slow = false, wide = false, checked = false;
    // the lane's dual, base-e with beta_{N-1} = 0, into the workgroup's block
    auto keep_dual = [&](int slot) __attribute__((always_inline)) {
        duals[slot] = make_uint4(__float_as_uint(y[0] * kLn2), __float_as_uint(y[1] * kLn2),
                                 __float_as_uint(y[2] * kLn2), 0u);
    };
    if (threadIdx.x == 0) finished = 0;
    if (geo.nvalid > 0) {   // wave-uniform; waves past the end still reach the barrier
        newton_start<N, IO>(geo, lds[geo.wave], logits, T, y, c, res, wide);
        newton_iterate<N, IO, false>(logits, WaveItem{geo.base}, tol, first, T, y, c, res, it, wide, checked, sweeps);
        slow = geo.valid() && res > tol && it < max_iter;
        const uint64_t mask = __ballot(slow);
        {
            uint4 w[G::C];
            Storage<IO>::template encode<KN>(T, w);
            // (the statistics variant, near its register limit, recomputes the tile addresses)
            G::Tile::template store_except<kStats>(w, lds[geo.wave], geo.lane, geo.chunks(Tout), geo.nvalid * G::C,
                                                   mask);
        }
        if (geo.valid() && !slow) {
            keep_dual(threadIdx.x);
            if (kStats) {
                iters[geo.matrix()] = (res <= tol) ? it : -1;
                if (fallbacks) fallbacks[geo.matrix()] = sweeps;
            }
        }
        const int nslow = __popcll(mask);
        if (nslow > 0 && nslow <= kHandOff) {
            // the tile's last reads completed inside store_except; the region is free
            float* rec = reinterpret_cast<float*>(lds[geo.wave]);
            const int p = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
            if (slow) {
#pragma unroll
                for (int k = 0; k < KN; ++k) rec[k * kHandOff + p] = T[k];
#pragma unroll
                for (int j = 0; j < M; ++j) rec[(KN + j) * kHandOff + p] = y[j];
#pragma unroll
                for (int j = 0; j < N; ++j) rec[(KN + M + j) * kHandOff + p] = c[j];
                rec[(KN + M + N) * kHandOff + p] = __int_as_float(
                    (int)threadIdx.x | (wide ? 0x100 : 0) | (checked ? 0x200 : 0) | (kStats ? sweeps << 10 : 0));
            }
            slow = false;   // carried on by the workgroup
        }
        if (geo.lane == 0) handed[geo.wave] = nslow > kHandOff ? -1 : nslow;
    } else if (geo.lane == 0) {
        handed[geo.wave] = 0;
    }
    __syncthreads();

    // states handed off in the workgroup, and the waves before this one that take them
    int total = 0, rank = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        const int h = handed[v];
        total += h > 0 ? h : 0;
        rank += (v < geo.wave && h >= 0) ? 1 : 0;
    }
    int slot = threadIdx.x;   // the lane's matrix in the workgroup
    // a taking wave: handed-off state number t = rank * 64 + lane, if it exists
    // (the takers are at least half as many as the waves that handed off, each of
    // which handed off at most kHandOff <= 32 states, so all are taken)
    if (handed[geo.wave] >= 0 && rank * 64 < total) {
        const int t = rank * 64 + geo.lane;
        slow = t < total;
        if (slow) {
            int src = 0, p = t;
#pragma unroll
            for (int v = 0; v < kWaves - 1; ++v) {
                const int h = handed[v] > 0 ? handed[v] : 0;
                const bool past = src == v && p >= h;
                p -= past ? h : 0;
                src += past ? 1 : 0;
            }
            const float* rec = reinterpret_cast<const float*>(lds[src]);
#pragma unroll
            for (int k = 0; k < KN; ++k) T[k] = rec[k * kHandOff + p];
#pragma unroll
            for (int j = 0; j < M; ++j) y[j] = rec[(KN + j) * kHandOff + p];
#pragma unroll
            for (int j = 0; j < N; ++j) c[j] = rec[(KN + M + j) * kHandOff + p];
            const int word = __float_as_int(rec[(KN + M + N) * kHandOff + p]);
            slot = word & 0xFF;
            wide = (word & 0x100) != 0;
            checked = (word & 0x200) != 0;
            sweeps = word >> 10;
            res = col_residual<N>(c);
            it = first;
        }
    }
    if (slow) {
        const int64_t item = (int64_t)blockIdx.x * kBlock + slot;
        newton_iterate<N, IO, false>(logits, LaneItem{item}, tol, max_iter, T, y, c, res, it, wide, checked, sweeps);
        uint4 w[G::C];
        Storage<IO>::template encode<KN>(T, w);
        // cached stores: the L2 merges these scattered 64-byte pieces with the
        // lines around them (streaming stores of them cost 4 % more HBM writes)
        uint4* q = reinterpret_cast<uint4*>(Tout) + item * G::C;
#pragma unroll
        for (int k = 0; k < G::C; ++k) q[k] = w[k];
        keep_dual(slot);
        if (kStats) {
            iters[item] = (res <= tol) ? it : -1;
            if (fallbacks) fallbacks[item] = sweeps;
        }
    }
    // the last wave to finish writes the workgroup's duals (its valid matrices)
    int before = 0;
    if (geo.lane == 0) before = __hip_atomic_fetch_add(&finished, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    before = __shfl(before, 0);
    if (before == kWaves - 1) {
        const int64_t left = B - (int64_t)blockIdx.x * kBlock;
        const int valid = left >= kBlock ? kBlock : (int)left;
        uint4* q = reinterpret_cast<uint4*>(dual) + (int64_t)blockIdx.x * kBlock;
#pragma unroll
        for (int k = 0; k < kBlock / 64; ++k) {
            const int m = k * 64 + geo.lane;
            if (m < valid) stream_store(q + m, duals[m]);
        }
    }
}

// ---------------------------------------------------------------------------
// Backward: eq (13).
// ---------------------------------------------------------------------------

// dH = d<G, T>/dH at the projection T, for upstream G = dL/dT (the lane's K
// rows of each).  eq (13) with eta = 1, a = b = 1 and the sign flipped for
// H = -M ([P] section 4.2):
//   mu_r = (G o T) 1,  rhs = mu_c - T_{-n}^T mu_r = sum_i T_ij (G_ij - mu_r_i),
//   Delta = I - T_{-n}^T T_{-n} (the Hessian at the optimum), w_{-n} = Delta^{-1} rhs, w_n = 0,
//   v = mu_r - T_{-n} w_{-n},  dH = -D = (G - v 1^T - 1 w^T) o T.
template <int N>
__device__ __forceinline__ void implicit_grad(const float (&T)[Split<N>::K * N], const float (&G)[Split<N>::K * N],
                                              float (&out)[Split<N>::K * N]) {
    constexpr int M = N - 1, K = Split<N>::K;
    using P = Pair<Split<N>::R>;
    float mur[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
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
        for (int i = 1; i < K; ++i) s = fmaf(T[i * N + j], G[i * N + j] - mur[i], s);
        rhs[j] = P::sum(s);
    }
    float w[M];
    solve_delta<N>([&](float (&h)[Tri<N>::S]) { hessian<N>(T, h); }, rhs, w);
#pragma unroll
    for (int i = 0; i < K; ++i) {
        float v = mur[i];
#pragma unroll
        for (int j = 0; j < M; ++j) v = fmaf(-T[i * N + j], w[j], v);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const float wj = (j < M) ? w[j] : 0.0f;
            out[i * N + j] = (G[i * N + j] - v - wj) * T[i * N + j];
        }
    }
}

// T is recomputed from (logits, dual) as a row softmax ([P] section 4.2: Delta
// may be recomputed from T* instead of saving the last Hessian).
template <int N, typename IO>
__global__ void __launch_bounds__(kBlock)
implicit_bwd_kernel(const IO* __restrict__ logits, const float* __restrict__ dual, const IO* __restrict__ dT,
                    IO* __restrict__ dH, int64_t B) {
    constexpr int M = N - 1;
    using Gm = Geometry<N, IO>;
    constexpr int C = Gm::C, K = Gm::K;
    __shared__ uint4 lds[kWaves][Gm::Tile::kLdsChunks];
    const Gm geo(B);
    if (geo.nvalid == 0) return;

    // issue every global load first, then route the chunks to their owners
    uint4 th[C], tg[C];
    Gm::Tile::fetch(geo.chunks(logits), geo.nvalid * C, geo.lane, th);
    Gm::Tile::fetch(geo.chunks(dT), geo.nvalid * C, geo.lane, tg);
    float beta[N];
    if (geo.valid())
        load_dual<N>(dual, geo.matrix(), beta);
    else
#pragma unroll
        for (int j = 0; j < N; ++j) beta[j] = 0.0f;
    float L[K * N], G[K * N];
    {
        uint4 w[C];
        Gm::Tile::route(th, lds[geo.wave], geo.lane, w);
        Storage<IO>::template decode<K * N>(w, L);
        Gm::Tile::route(tg, lds[geo.wave], geo.lane, w);
        Storage<IO>::template decode<K * N>(w, G);
    }
#pragma unroll
    for (int k = 0; k < K * N; ++k) L[k] *= kLog2e;
    float y[M];
#pragma unroll
    for (int j = 0; j < M; ++j) y[j] = (beta[j] - beta[M]) * kLog2e;   // T is invariant to the gauge
    float T[K * N];
    softmax_rows<N, K>(L, y, T);
    float out[K * N];
    implicit_grad<N>(T, G, out);
    {
        uint4 wo[C];
        Storage<IO>::template encode<K * N>(out, wo);
        Gm::Tile::template store<N != 4>(wo, lds[geo.wave], geo.lane, geo.chunks(dH), geo.nvalid * C);
    }
}

// The backward from the projection itself ([P] section 4.2: dH needs only T*
// and G): reads T and dT, writes dH; no exponentials.
template <int N>
__global__ void __launch_bounds__(kBlock)
implicit_bwd_from_T_kernel(const float* __restrict__ Tin, const float* __restrict__ dT, float* __restrict__ dH,
                           int64_t B) {
    using Gm = Geometry<N, float>;
    constexpr int C = Gm::C, K = Gm::K;
    __shared__ uint4 lds[kWaves][Gm::Tile::kLdsChunks];
    const Gm geo(B);
    if (geo.nvalid == 0) return;
    uint4 tt[C], tg[C];
    Gm::Tile::fetch(geo.chunks(Tin), geo.nvalid * C, geo.lane, tt);
    Gm::Tile::fetch(geo.chunks(dT), geo.nvalid * C, geo.lane, tg);
    float T[K * N], G[K * N], out[K * N];
    {
        uint4 w[C];
        Gm::Tile::route(tt, lds[geo.wave], geo.lane, w);
        Storage<float>::template decode<K * N>(w, T);
        Gm::Tile::route(tg, lds[geo.wave], geo.lane, w);
        Storage<float>::template decode<K * N>(w, G);
    }
    implicit_grad<N>(T, G, out);
    {
        uint4 wo[C];
        Storage<float>::template encode<K * N>(out, wo);
        Gm::Tile::template store<N != 4>(wo, lds[geo.wave], geo.lane, geo.chunks(dH), geo.nvalid * C);
    }
}

// ---------------------------------------------------------------------------
// Forward and backward in one launch, for callers that hold dL/dT when they
// project.  The forward is newton_solve, as in birkhoff_fwd; the backward is eq (13) at the
// final iterate T, still in registers, so neither the logits nor the dual are
// read back.  Reads logits and dT, writes T, dual and dH.
// ---------------------------------------------------------------------------
template <int N, typename IO>
__global__ void __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(N == 4 ? 6 : 4)))
fused_fwd_bwd_kernel(const IO* __restrict__ logits, const IO* __restrict__ dT, IO* __restrict__ Tout,
                     float* __restrict__ dual, IO* __restrict__ dH, int64_t B, float tol, int max_iter) {
    using Gm = Geometry<N, IO>;
    constexpr int C = Gm::C, K = Gm::K;
    // the lane-pair kernels need their tile addresses recomputed to stay clear of spills; the n = 4
    // kernel keeps them (measured 1.7 % faster on the training and bf16 workloads)
    constexpr bool kPin = N != 4;
    __shared__ uint4 lds[kWaves][Gm::Tile::kLdsChunks];
    const Gm geo(B);
    if (geo.nvalid == 0) return;
    float T[K * N], y[N - 1], res;
    float G[K * N], out[K * N];
    if constexpr (Gm::Tile::kStaged) {
        // dL/dT travels into LDS while the Newton iteration runs
        int sweeps;
        newton_solve<N, IO, true>(geo, lds[geo.wave], logits, tol, max_iter, T, y, res, sweeps, dT);
        uint4 w[C];
        Gm::Tile::template read_prefetched<kPin>(lds[geo.wave], geo.lane, w);
        Storage<IO>::template decode<K * N>(w, G);
        store_forward<N, IO, kPin>(geo, lds[geo.wave], Tout, dual, T, y);
    } else {
        int sweeps;
        newton_solve<N, IO>(geo, lds[geo.wave], logits, tol, max_iter, T, y, res, sweeps);
        uint4 tg[C];
        Gm::Tile::fetch(geo.chunks(dT), geo.nvalid * C, geo.lane, tg);   // in flight while T is stored
        store_forward<N, IO, kPin>(geo, lds[geo.wave], Tout, dual, T, y);
        uint4 w[C];
        Gm::Tile::route(tg, lds[geo.wave], geo.lane, w);
        Storage<IO>::template decode<K * N>(w, G);
    }
    implicit_grad<N>(T, G, out);
    {
        uint4 wo[C];
        Storage<IO>::template encode<K * N>(out, wo);
        Gm::Tile::template store<kPin>(wo, lds[geo.wave], geo.lane, geo.chunks(dH), geo.nvalid * C);
    }
}

// ---------------------------------------------------------------------------
// Baseline: a fixed number of Sinkhorn-Knopp sweeps in the log domain.
// ---------------------------------------------------------------------------
template <int N, typename IO>
__global__ void __launch_bounds__(kBlock)
sinkhorn_kernel(const IO* __restrict__ logits, IO* __restrict__ Tout, int64_t B, int sweeps) {
    using G = Geometry<N, IO>;
    constexpr int K = G::K;
    using P = Pair<G::R>;
    __shared__ uint4 lds[kWaves][G::Tile::kLdsChunks];
    const G geo(B);
    if (geo.nvalid == 0) return;
    float L[K * N];
    {
        uint4 w[G::C];
        G::Tile::load(geo.chunks(logits), geo.nvalid * G::C, lds[geo.wave], geo.lane, w);
        Storage<IO>::template decode<K * N>(w, L);
    }
#pragma unroll
    for (int k = 0; k < K * N; ++k) L[k] *= kLog2e;
    float a[K], z[N];
#pragma unroll
    for (int i = 0; i < K; ++i) a[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < N; ++j) z[j] = 0.0f;   // v^(0) = 1
    for (int t = 0; t < sweeps; ++t) {
#pragma unroll
        for (int i = 0; i < K; ++i) {   // u = 1 / (A v): alpha_i = -LSE_j(H_ij + beta_j)
            float u[N];
#pragma unroll
            for (int j = 0; j < N; ++j) u[j] = L[i * N + j] + z[j];
            float mu = u[0];
#pragma unroll
            for (int j = 1; j < N; ++j) mu = fmaxf(mu, u[j]);
            float s = ex2(u[0] - mu);
#pragma unroll
            for (int j = 1; j < N; ++j) s += ex2(u[j] - mu);
            a[i] = -(mu + lg2(s));
        }
#pragma unroll
        for (int j = 0; j < N; ++j) {   // v = 1 / (A^T u): beta_j = -LSE_i(H_ij + alpha_i)
            float v[K];
#pragma unroll
            for (int i = 0; i < K; ++i) v[i] = L[i * N + j] + a[i];
            float m = v[0];
#pragma unroll
            for (int i = 1; i < K; ++i) m = fmaxf(m, v[i]);
            m = P::max(m);
            float s = ex2(v[0] - m);
#pragma unroll
            for (int i = 1; i < K; ++i) s += ex2(v[i] - m);
            z[j] = -(m + lg2(P::sum(s)));
        }
    }
    float T[K * N];
#pragma unroll
    for (int i = 0; i < K; ++i)
#pragma unroll
        for (int j = 0; j < N; ++j) T[i * N + j] = ex2(L[i * N + j] + a[i] + z[j]);
    {
        uint4 w[G::C];
        Storage<IO>::template encode<K * N>(T, w);
        G::Tile::store(w, lds[geo.wave], geo.lane, geo.chunks(Tout), geo.nvalid * G::C);
    }
}

}  // namespace birk
