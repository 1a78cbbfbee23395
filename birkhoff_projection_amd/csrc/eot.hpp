// eot.hpp -- device routines for batched small entropic optimal transport
// with general cost, marginals and regularisation (gfx950).
//
// Problem ([P] section 2.3, eq 3): for a cost M (n x m), marginals a > 0 (n)
// and b > 0 (m) with equal sums and eta > 0, find the plan
//     T = argmin { <T, M> - eta h(T) : T 1 = a, T^T 1 = b },
// whose dual form (eq 4) gives T_ij = exp((alpha_i + beta_j - M_ij) / eta).
// The Birkhoff projection is the case a = b = 1, eta = 1, M = -H.
//
// Layout.  One problem per lane (64 per wave), all n*m entries of its plan in
// VGPRs; no lane pairs and no MFMA -- every problem is independent and tiny.
// Problems are stored back to back (cost, plan and gradients [B, n, m]
// row-major; per-problem marginals [B, n] and [B, m]; dual [B, m]), so a
// wave's 64 problems form one contiguous span of each array.  Spans move
// between HBM and the owning lanes through the wave's LDS region
// (Items<F>): coalesced 16-byte global accesses, an odd LDS stride per item so
// that per-lane reads and writes are free of bank conflicts.
//
// State.  The iteration keeps the row softmaxes S_ij = T_ij / a_i
// (eq 10: S_i. = Softmax((beta - M_i.) / eta)); then T = diag(a) S, the
// column sums are c = S^T a, and the Hessian of eq (9), scaled by eta, is
// diag(c) - S^T diag(a) S.  Newton runs on z = beta / eta, whose iterates are
// those of eq (8) in beta (the gradient c - b is the same and the Hessian
// and the objective only pick up the factor 1/eta); the dual is returned as
// beta = eta z.  Logits L = -M / eta and z are held in base-2 units
// (times log2 e) so that each exponential is one v_exp_f32.
//
// Sources: "Accelerating Birkhoff Projection for Manifold-Constrained
// Hyper-Connections", section 2.3 (eqs 3-7), section 3.1 (eqs 8-10),
// section 4.1 (eq 13) and section 4.2; the blog post "小矩阵遇上牛顿法",
// section 2.2, for the step sizes and the Sinkhorn fallback.
#pragma once

#include "projection.hpp"

namespace birk {
namespace eot {

// ---------------------------------------------------------------------------
// Wave-wide movement of F-float items.  The wave's span is 64*F floats =
// 16*F 16-byte chunks starting 256-byte aligned (when the array is 16-byte
// aligned).  A full span is read in ceil(F/4) coalesced 16-byte accesses per
// lane, whose floats are scattered to LDS at item * FP + offset with an odd
// stride FP; each lane then reads its own F floats (stride FP across lanes:
// 64 distinct banks).  Stores run the other way.  The last, partial span of a
// batch uses coalesced 4-byte accesses instead (no access crosses the end of
// the array).
// ---------------------------------------------------------------------------
template <int F>
struct Items {
    static constexpr int FP = F | 1;
    static constexpr int kLdsFloats = 64 * FP;
    static constexpr int kChunks = 16 * F;
    static constexpr int kSteps = (kChunks + 63) / 64;

    __device__ __forceinline__ static int pos(int f) { return (f / F) * FP + f % F; }
    // LDS position of float e (< 4) of 16-byte chunk c.  When an item is a whole
    // number of chunks the four floats of a chunk belong to one item and sit side
    // by side, so one division per chunk serves all four.
    __device__ __forceinline__ static int chunk_pos(int c, int e) {
        if constexpr (F % 4 == 0) {
            constexpr int CI = F / 4;   // chunks per item
            return (c / CI) * FP + 4 * (c % CI) + e;
        } else {
            return pos(4 * c + e);
        }
    }

    // `src` is the span's first float; `nf` (wave-uniform) floats of it exist.
    __device__ __forceinline__ static void load(const float* __restrict__ src, int nf, float* lds, int lane,
                                                float (&v)[F]) {
        if (nf == 64 * F) {
            const uint4* s4 = reinterpret_cast<const uint4*>(src);
            uint4 t[kSteps];
#pragma unroll
            for (int k = 0; k < kSteps; ++k) {
                const int c = k * 64 + lane;
                t[k] = stream_load(s4 + (c < kChunks ? c : kChunks - 1));
            }
#pragma unroll
            for (int k = 0; k < kSteps; ++k) {
                const int c = k * 64 + lane;
                if ((k + 1) * 64 <= kChunks || c < kChunks) {
                    lds[chunk_pos(c, 0)] = __uint_as_float(t[k].x);
                    lds[chunk_pos(c, 1)] = __uint_as_float(t[k].y);
                    lds[chunk_pos(c, 2)] = __uint_as_float(t[k].z);
                    lds[chunk_pos(c, 3)] = __uint_as_float(t[k].w);
                }
            }
        } else {
            float t[F];
#pragma unroll
            for (int k = 0; k < F; ++k) {
                const int f = k * 64 + lane;
                t[k] = __builtin_nontemporal_load(src + (f < nf ? f : nf - 1));
            }
#pragma unroll
            for (int k = 0; k < F; ++k) {
                const int f = k * 64 + lane;
                lds[pos(f)] = f < nf ? t[k] : 0.0f;
            }
        }
        wave_lds_sync();
#pragma unroll
        for (int q = 0; q < F; ++q) v[q] = lds[lane * FP + q];
        wave_lds_sync();
    }

    // `dst` is the span's first float; only its first `nf` floats are written.
    __device__ __forceinline__ static void store(const float (&v)[F], float* lds, int lane, float* __restrict__ dst,
                                                 int nf) {
#pragma unroll
        for (int q = 0; q < F; ++q) lds[lane * FP + q] = v[q];
        wave_lds_sync();
        if (nf == 64 * F) {
            uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
            for (int k = 0; k < kSteps; ++k) {
                const int c = k * 64 + lane;
                if ((k + 1) * 64 <= kChunks || c < kChunks) {
                    const uint4 w = make_uint4(__float_as_uint(lds[chunk_pos(c, 0)]), __float_as_uint(lds[chunk_pos(c, 1)]),
                                               __float_as_uint(lds[chunk_pos(c, 2)]), __float_as_uint(lds[chunk_pos(c, 3)]));
                    stream_store(d4 + c, w);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < F; ++k) {
                const int f = k * 64 + lane;
                if (f < nf) __builtin_nontemporal_store(lds[pos(f)], dst + f);
            }
        }
        wave_lds_sync();
    }
};

// Marginals of the lane's problem: per-problem arrays ([B, F], through the
// wave's LDS) or one vector shared by every problem.
template <int F>
__device__ __forceinline__ void load_marginal(const float* __restrict__ p, bool shared, int64_t base, int nvalid,
                                              float* lds, int lane, float (&v)[F]) {
    if (shared) {
#pragma unroll
        for (int q = 0; q < F; ++q) v[q] = p[q];
    } else {
        Items<F>::load(p + base * F, nvalid * F, lds, lane, v);
    }
}

// ---------------------------------------------------------------------------
// Newton pieces with weights a (S holds row softmaxes, rows sum to one).
// ---------------------------------------------------------------------------

// c_j = sum_i a_i S_ij (the column sums of T = diag(a) S; eq 9's gradient is c_{-m} - b_{-m})
template <int N, int M>
__device__ __forceinline__ void col_sums(const float (&S)[N * M], const float (&a)[N], float (&c)[M]) {
#pragma unroll
    for (int j = 0; j < M; ++j) {
        float s = a[0] * S[j];
#pragma unroll
        for (int i = 1; i < N; ++i) s = fmaf(a[i], S[i * M + j], s);
        c[j] = s;
    }
}

// max_j |c_j - b_j|; NaN propagates (IEEE 754-2019 `maximum`, gfx950's
// v_maximum3_f32)
template <int M>
__device__ __forceinline__ float col_residual(const float (&c)[M], const float (&b)[M]) {
    float r = fabsf(c[0] - b[0]);
#pragma unroll
    for (int j = 1; j < M; ++j) r = __builtin_elementwise_maximum(r, fabsf(c[j] - b[j]));
    return r;
}

// eta times the Hessian of eq (9): h_jk = [j == k] c_j - sum_i a_i S_ij S_ik,
// j, k < m - 1.  With the weighted column Gram sums G_jk = sum_i a_i S_ij S_ik
// (all m columns), the diagonal is formed as sum_{k != j} G_jk: the same
// non-negative terms as sum_i a_i S_ij (sum_{k != j} S_ik), which equals
// c_j - sum_i a_i S_ij^2 since rows of S sum to one, so it does not cancel when a
// column is carried by one entry; the off-diagonal sums are reused.  At the
// optimum this is also eq (13)'s Delta ([P] section 4.2).
template <int N, int M>
__device__ __forceinline__ void hessian(const float (&S)[N * M], const float (&a)[N], float (&h)[Tri<M>::S]) {
    constexpr int K1 = M - 1;
    float aS[N * K1];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int j = 0; j < K1; ++j) aS[i * K1 + j] = a[i] * S[i * M + j];
    float g[Tri<M>::S], gm[K1];   // G_jk (k < j < m-1) and G_j,m-1
#pragma unroll
    for (int j = 0; j < K1; ++j) {
#pragma unroll
        for (int k = 0; k < j; ++k) {
            float p = aS[j] * S[k];
#pragma unroll
            for (int i = 1; i < N; ++i) p = fmaf(aS[i * K1 + j], S[i * M + k], p);
            g[Tri<M>::at(j, k)] = p;
            h[Tri<M>::at(j, k)] = -p;
        }
        float q = aS[j] * S[K1];
#pragma unroll
        for (int i = 1; i < N; ++i) q = fmaf(aS[i * K1 + j], S[i * M + K1], q);
        gm[j] = q;
    }
#pragma unroll
    for (int j = 0; j < K1; ++j) {
        float d = gm[j];
#pragma unroll
        for (int k = 0; k < K1; ++k)
            if (k != j) d += g[k < j ? Tri<M>::at(j, k) : Tri<M>::at(k, j)];
        h[Tri<M>::at(j, j)] = d;
    }
}

// e^x - 1 and e^x - 1 - x (the latter of second order in x) from one Taylor
// polynomial below |x| = 1/16 (e^x - 1 - x = x^2 p(x), truncation below 1e-9
// relative), from `ex` = e^x elsewhere.
__device__ __forceinline__ void expm1_pair(float x, float ex, float& em, float& xm) {
    float p = fmaf(x, 1.0f / 5040.0f, 1.0f / 720.0f);
    p = fmaf(x, p, 1.0f / 120.0f);
    p = fmaf(x, p, 1.0f / 24.0f);
    p = fmaf(x, p, 1.0f / 6.0f);
    p = fmaf(x, p, 0.5f);
    const float x2p = x * x * p;
    const bool small = fabsf(x) < 0.0625f;
    em = small ? x + x2p : ex - 1.0f;
    xm = small ? x2p : (ex - 1.0f) - x;
}

// log(1 + q) - q, of second order in q: Taylor series below |q| = 1/16
// (truncation below 1e-9 relative), `l1p` = log(1 + q) elsewhere.

__device__ __forceinline__ float log1p_minus_x(float q, float l1p) {
    float p = fmaf(q, 1.0f / 9.0f, -1.0f / 8.0f);
    p = fmaf(q, p, 1.0f / 7.0f);
    p = fmaf(q, p, -1.0f / 6.0f);
    p = fmaf(q, p, 1.0f / 5.0f);
    p = fmaf(q, p, -1.0f / 4.0f);
    p = fmaf(q, p, 1.0f / 3.0f);
    p = fmaf(q, p, -0.5f);
    return fabsf(q) < 0.0625f ? q * q * p : l1p - q;
}

// Trial point z + s of the line search (natural units, s_{m-1} = 0) from the
// current S: moving z by s multiplies column j of S by e^{s_j} before the rows
// are normalised again, S'_ij = S_ij e^{s_j} r_i, r_i = 1 / sum_k S_ik e^{s_k}.
// The objective of eq (8) divided by eta, F(z) = sum_i a_i LSE_i(z - M_i. / eta) - z^T b
// (eq 8 with eq 5), changes by
//     F(z + s) - F(z) = sum_i a_i log(1 + q_i) - s^T b,   q_i = sum_j S_ij (e^{s_j} - 1),
// which is rearranged (using c = S^T a and g = c - b) into terms that are each
// of second order in s:
//     = sum_j [c_j (e^{s_j} - 1 - s_j) + g_j s_j] + sum_i a_i [log(1 + q_i) - q_i],
// so that its sign stays reliable in fp32 down to tiny steps.  Returns the
// change; e, r and the column sums ct of T' = diag(a) S' are returned for
// accept_trial and the gradient test, and `noise` is 2^-21 times the sum of the
// terms' magnitudes (below it fp32 cannot resolve the change's sign).
template <int N, int M>
__device__ __forceinline__ float trial_point(const float (&S)[N * M], const float (&a)[N], const float (&c)[M],
                                             const float (&g)[M - 1], const float (&s)[M - 1], float (&e)[M - 1],
                                             float (&r)[N], float (&ct)[M], float& noise) {
    constexpr int K1 = M - 1;
    float em[K1];
    float df = 0.0f, mag = 0.0f;
#pragma unroll
    for (int j = 0; j < K1; ++j) {
        e[j] = ex2(s[j] * kLog2e);
        float xm;
        expm1_pair(s[j], e[j], em[j], xm);
        df = fmaf(c[j], xm, fmaf(g[j], s[j], df));
        mag += fabsf(c[j] * xm) + fabsf(g[j] * s[j]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float q = S[i * M] * em[0];
#pragma unroll
        for (int j = 1; j < K1; ++j) q = fmaf(S[i * M + j], em[j], q);
        float u[K1];
        float rs = S[i * M + K1];
#pragma unroll
        for (int j = 0; j < K1; ++j) {
            u[j] = S[i * M + j] * e[j];
            rs += u[j];
        }
        r[i] = rcp(rs);
        const float lq = a[i] * log1p_minus_x(q, lg2(rs) * kLn2);
        df += lq;
        mag += fabsf(lq);
        const float ar = a[i] * r[i];
#pragma unroll
        for (int j = 0; j < K1; ++j) ct[j] = (i == 0) ? u[j] * ar : fmaf(u[j], ar, ct[j]);
        ct[K1] = (i == 0) ? S[i * M + K1] * ar : fmaf(S[i * M + K1], ar, ct[K1]);
    }
    noise = mag * 0x1.0p-21f;
    return df;
}

template <int N, int M>
__device__ __forceinline__ void accept_trial(float (&S)[N * M], const float (&e)[M - 1], const float (&r)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
        for (int j = 0; j < M - 1; ++j) S[i * M + j] = (S[i * M + j] * e[j]) * r[i];
        S[i * M + M - 1] *= r[i];
    }
}

// One Sinkhorn-Knopp sweep of eq (7) in the log domain (base-2 units, L the
// base-2 logits -M log2(e) / eta): alpha_i = log2 a_i - LSE2_j(L_ij + y_j)
// (eq 5), then beta_j = log2 b_j - LSE2_i(L_ij + alpha_i) (eq 6), re-gauged to
// beta_{m-1} = 0.  No column sum is formed, so an underflowed column cannot
// produce log(0).
template <int N, int M>
__device__ __forceinline__ void sinkhorn_sweep(const float (&L)[N * M], const float (&a)[N], const float (&b)[M],
                                               float (&y)[M - 1]) {
    float al[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float u[M];
#pragma unroll
        for (int j = 0; j < M - 1; ++j) u[j] = L[i * M + j] + y[j];
        u[M - 1] = L[i * M + M - 1];
        float mu = u[0];
#pragma unroll
        for (int j = 1; j < M; ++j) mu = fmaxf(mu, u[j]);
        float s = ex2(u[0] - mu);
#pragma unroll
        for (int j = 1; j < M; ++j) s += ex2(u[j] - mu);
        al[i] = lg2(a[i]) - (mu + lg2(s));
    }
    float z[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
        float v[N];
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = L[i * M + j] + al[i];
        float mx = v[0];
#pragma unroll
        for (int i = 1; i < N; ++i) mx = fmaxf(mx, v[i]);
        float s = ex2(v[0] - mx);
#pragma unroll
        for (int i = 1; i < N; ++i) s += ex2(v[i] - mx);
        z[j] = lg2(b[j]) - (mx + lg2(s));
    }
#pragma unroll
    for (int j = 0; j < M - 1; ++j) y[j] = z[j] - z[M - 1];
}

// ---------------------------------------------------------------------------
// Kernels.  Lane l of wave w of workgroup g owns problem (g*W + w)*64 + l,
// W = Waves<N*M>::value waves per workgroup: 4, or 2 where four waves' LDS
// regions would exceed 64 KiB (8 x 8).
// ---------------------------------------------------------------------------
template <int F>
struct Waves {
    static constexpr int value = 4 * Items<F>::kLdsFloats * 4 <= 65536 ? 4 : 2;
    static constexpr int threads = 64 * value;
};

template <int W>
struct Lanes {
    int lane, wave, nvalid;   // nvalid: problems of this wave inside the batch (wave-uniform)
    int64_t base;             // first problem of this wave
    __device__ __forceinline__ explicit Lanes(int64_t B) {
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: base goes to SGPRs
        base = ((int64_t)blockIdx.x * W + wave) * 64;
        const int64_t left = B - base;
        nvalid = __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : left >= 64 ? 64 : (int)left);
    }
    __device__ __forceinline__ bool valid() const { return lane < nvalid; }
    __device__ __forceinline__ int64_t problem() const { return base + lane; }
};

// Forward: Newton on the reduced dual (eq 8) from kStartSweeps Sinkhorn sweeps until the column
// marginals are met to `tol` (absolute) or `max_iter` updates; rows are met by
// construction.  Step sizes 1, 1/2, 1/10, 1/20, 1/100, the first that lowers
// both the objective and the gradient norm is taken; otherwise one Sinkhorn
// sweep (eqs 5-7) replaces the update.  Writes T = diag(a) S, the dual
// beta = eta z (cost units, beta_{m-1} = 0) and optionally the update count
// (-1 when tol was not reached).
template <int N, int M, bool kStats>
__global__ void __launch_bounds__(Waves<N * M>::threads)
eot_fwd_kernel(const float* __restrict__ cost, const float* __restrict__ a_in, const float* __restrict__ b_in,
               int shared_marginals, float* __restrict__ Tout, float* __restrict__ dual, int32_t* __restrict__ iters,
               int64_t B, float eta, float tol, int max_iter) {
    constexpr int K1 = M - 1;
    constexpr int W = Waves<N * M>::value;
    __shared__ float lds_all[W][Items<N * M>::kLdsFloats];
    const Lanes<W> ln(B);
    if (ln.nvalid == 0) return;
    float* lds = lds_all[ln.wave];
    const bool shared = shared_marginals != 0;
    const float lscale = -kLog2e / eta;   // cost -> base-2 logits

    float a[N], b[M];
    load_marginal<N>(a_in, shared, ln.base, ln.nvalid, lds, ln.lane, a);
    load_marginal<M>(b_in, shared, ln.base, ln.nvalid, lds, ln.lane, b);
    // start: kStartSweeps Sinkhorn-Knopp sweeps (eqs 5-6) from z = log(b / b_{m-1})
    // (base 2 here): the rows normalised at that z, then per sweep the columns
    // scaled to b and the rows normalised again, z_j += log(b_j / c_j) -
    // log(b_{m-1} / c_{m-1}).  It is the optimum when the cost is constant (plan
    // a b^T / sum(b)) and the Birkhoff kernels' start when a = b = 1.  A sweep is
    // skipped if a column sum is 0 or not finite; lanes past the end (b = 0)
    // start at 0.
    float S[N * M], y[K1], c[M];
    {
        const float lbm = ln.valid() ? lg2(b[K1]) : 0.0f;
#pragma unroll
        for (int j = 0; j < K1; ++j) y[j] = ln.valid() ? lg2(b[j]) - lbm : 0.0f;
        float L[N * M];
        Items<N * M>::load(cost + ln.base * (N * M), ln.nvalid * (N * M), lds, ln.lane, L);
#pragma unroll
        for (int k = 0; k < N * M; ++k) L[k] *= lscale;
        softmax_rows<M, N>(L, y, S);
    }
#pragma unroll
    for (int sw = 0; sw < kStartSweeps; ++sw) {
        // a sweep's column step: S_ij <- S_ij b_j / c_j, rows normalised again
        col_sums<N, M>(S, a, c);
        bool ok = ln.valid();
#pragma unroll
        for (int j = 0; j < M; ++j) ok = ok && c[j] > 1.17549435e-38f && c[j] < 3.0e38f;
        float f[M];
#pragma unroll
        for (int j = 0; j < M; ++j) f[j] = ok ? b[j] * rcp(c[j]) : 1.0f;
        const float rf = rcp(f[K1]);
#pragma unroll
        for (int j = 0; j < K1; ++j) y[j] = ok ? y[j] + lg2(f[j] * rf) : y[j];
#pragma unroll
        for (int i = 0; i < N; ++i) {
#pragma clang fp contract(off)
            // (plain adds of the scaled entries, which are kept)
#pragma unroll
            for (int j = 0; j < M; ++j) S[i * M + j] *= f[j];
            float rs = S[i * M];
#pragma unroll
            for (int j = 1; j < M; ++j) rs += S[i * M + j];
            const float r = rcp(rs);
#pragma unroll
            for (int j = 0; j < M; ++j) S[i * M + j] *= r;
        }
    }
    col_sums<N, M>(S, a, c);
    float res = ln.valid() ? col_residual<M>(c, b) : 0.0f;
    int it = 0;
    // Lanes with lost entries, as in the Birkhoff iteration (birk::newton_iterate):
    // S is formed multiplicatively, so an entry that underflowed stays zero.  A
    // lane is `wide` when S has an entry below kTiny at the start (cost spans of
    // about 70 eta), or when it converges with one and S rebuilt from the costs at
    // its dual misses tol; a wide lane re-evaluates S from the costs after every
    // accepted step.
    float smin = S[0];
#pragma unroll
    for (int k = 1; k < N * M; ++k) smin = fminf(smin, S[k]);
    bool wide = ln.valid() && smin < kTiny;

    for (;;) {
        while (res > tol && it < max_iter) {
            float g[K1], rhs[K1], d[K1];
#pragma unroll
            for (int j = 0; j < K1; ++j) {
                g[j] = c[j] - b[j];
                rhs[j] = -g[j];
            }
            float gn2 = g[0] * g[0];
#pragma unroll
            for (int j = 1; j < K1; ++j) gn2 = fmaf(g[j], g[j], gn2);
            float h[Tri<M>::S];
            hessian<N, M>(S, a, h);
            damp<M>(h);
            const bool ok = SpdSolve<M>::run(h, rhs, d);

            bool accepted = false;
            if (ok) {
                for (int k = 0; k < 5; ++k) {
                    const float gam = step_size(k);
                    float s[K1], e[K1], rr[N], ct[M];
#pragma unroll
                    for (int j = 0; j < K1; ++j) s[j] = gam * d[j];
                    float noise;
                    const float df = trial_point<N, M>(S, a, c, g, s, e, rr, ct, noise);
                    float gt2 = (ct[0] - b[0]) * (ct[0] - b[0]);
#pragma unroll
                    for (int j = 1; j < K1; ++j) gt2 = fmaf(ct[j] - b[j], ct[j] - b[j], gt2);
                    if (df < noise && gt2 < gn2) {
#pragma unroll
                        for (int j = 0; j < K1; ++j) y[j] = fmaf(s[j], kLog2e, y[j]);
                        accept_trial<N, M>(S, e, rr);
#pragma unroll
                        for (int j = 0; j < M; ++j) c[j] = ct[j];
                        accepted = true;
                        break;
                    }
                }
            }
            if (!accepted || wide) {
                // the fallback sweep, or a wide lane's step: S from the costs (re-read
                // by this lane alone, only on these rare paths)
                float L[N * M];
                const float* p = cost + ln.problem() * (N * M);
#pragma unroll
                for (int k = 0; k < N * M; ++k) L[k] = p[k] * lscale;
                if (!accepted) sinkhorn_sweep<N, M>(L, a, b, y);
                softmax_rows<M, N>(L, y, S);
                col_sums<N, M>(S, a, c);
            }
            ++it;
            res = col_residual<M>(c, b);
        }
        if (!(res <= tol) || wide) break;
        float mn = S[0];
#pragma unroll
        for (int k = 1; k < N * M; ++k) mn = fminf(mn, S[k]);
        if (mn >= kTiny) break;
        // converged with an entry below kTiny: checked against its dual once
        wide = true;
        float L[N * M];
        const float* p = cost + ln.problem() * (N * M);
#pragma unroll
        for (int k = 0; k < N * M; ++k) L[k] = p[k] * lscale;
        softmax_rows<M, N>(L, y, S);
        col_sums<N, M>(S, a, c);
        res = col_residual<M>(c, b);
        if (res <= tol) break;
    }

    {
        float T[N * M];
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int j = 0; j < M; ++j) T[i * M + j] = a[i] * S[i * M + j];
        Items<N * M>::store(T, lds, ln.lane, Tout + ln.base * (N * M), ln.nvalid * (N * M));
    }
    {
        float beta[M];
        const float bscale = eta * kLn2;   // base-2 z -> beta in cost units
#pragma unroll
        for (int j = 0; j < K1; ++j) beta[j] = y[j] * bscale;
        beta[K1] = 0.0f;
        Items<M>::store(beta, lds, ln.lane, dual + ln.base * M, ln.nvalid * M);
    }
    if (kStats && ln.valid()) __builtin_nontemporal_store((res <= tol) ? it : -1, iters + ln.problem());
}

// Backward, eq (13): D = dl/dM from the plan T* and upstream G = dl/dT,
//   D = eta^-1 [diag((mu_r - T_{-m} w_{-m}) / a) T + T diag(w) - G o T],
//   mu_r = (G o T) 1,  w_{-m} = Delta^-1 [mu_c - T_{-m}^T (mu_r / a)],  w_m = 0.
// With S = diag(a)^-1 T and nu = mu_r / a = (G o S) 1 this is
//   rhs_j = sum_i T_ij (G_ij - nu_i),   D_ij = T_ij (nu_i - (S w)_i + w_j - G_ij) / eta.
// Delta is recomputed from T* as the Hessian at T* ([P] section 4.2), which
// equals diag(b_{-m}) - T_{-m}^T diag(a)^-1 T_{-m} at the optimum.
template <int N, int M>
__global__ void __launch_bounds__(Waves<N * M>::threads)
eot_bwd_kernel(const float* __restrict__ Tin, const float* __restrict__ Gin, const float* __restrict__ a_in,
               int shared_marginals, float* __restrict__ Dout, int64_t B, float eta) {
    constexpr int K1 = M - 1;
    constexpr int W = Waves<N * M>::value;
    __shared__ float lds_all[W][Items<N * M>::kLdsFloats];
    const Lanes<W> ln(B);
    if (ln.nvalid == 0) return;
    float* lds = lds_all[ln.wave];
    const int nf = ln.nvalid * (N * M);

    float a[N];
    load_marginal<N>(a_in, shared_marginals != 0, ln.base, ln.nvalid, lds, ln.lane, a);
    float T[N * M], G[N * M];
    Items<N * M>::load(Tin + ln.base * (N * M), nf, lds, ln.lane, T);
    Items<N * M>::load(Gin + ln.base * (N * M), nf, lds, ln.lane, G);
    if (!ln.valid()) {
#pragma unroll
        for (int i = 0; i < N; ++i) a[i] = 1.0f;   // keeps the unused lanes finite
    }
    float S[N * M], nu[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float ra = rcp(a[i]);
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < M; ++j) {
            S[i * M + j] = T[i * M + j] * ra;
            v = fmaf(G[i * M + j], S[i * M + j], v);
        }
        nu[i] = v;
    }
    float rhs[K1];
#pragma unroll
    for (int j = 0; j < K1; ++j) {
        float s = T[j] * (G[j] - nu[0]);
#pragma unroll
        for (int i = 1; i < N; ++i) s = fmaf(T[i * M + j], G[i * M + j] - nu[i], s);
        rhs[j] = s;
    }
    float w[K1];
    float mass = a[0];   // bounds the entries of the Hessian
#pragma unroll
    for (int i = 1; i < N; ++i) mass += a[i];
    solve_delta<M>([&](float (&h)[Tri<M>::S]) { hessian<N, M>(S, a, h); }, rhs, w, mass);
    const float ieta = 1.0f / eta;
    float D[N * M];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float v = nu[i];
#pragma unroll
        for (int j = 0; j < K1; ++j) v = fmaf(-S[i * M + j], w[j], v);
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const float wj = (j < K1) ? w[j] : 0.0f;
            D[i * M + j] = (v + wj - G[i * M + j]) * T[i * M + j] * ieta;
        }
    }
    Items<N * M>::store(D, lds, ln.lane, Dout + ln.base * (N * M), nf);
}

}  // namespace eot
}  // namespace birk
