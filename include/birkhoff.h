/*
 * birkhoff.h -- C ABI of libbirkhoff, batched KL projection onto the Birkhoff
 * polytope for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every one of B independent n x n logit matrices H
 * (n = 4 or n = 8) the forward pass returns
 *
 *     T = argmin_{P in B_n} KL(P || exp(H)),      B_n = doubly stochastic n x n,
 *
 * i.e. the unique T = D1 exp(H) D2 with unit row and column sums
 * ("Accelerating Birkhoff Projection for Manifold-Constrained Hyper-Connections",
 * section 2.2, eq (1); Sinkhorn's theorem).  It is found by Newton's method on
 * the reduced (n-1)-dimensional entropic-OT dual (section 3.1, eqs (8)-(9);
 * section 3.2, eqs (10)-(12) for n = 4) with the step-size rule and Sinkhorn
 * fallback of the author's blog post "小矩阵遇上牛顿法" (section 2.2).  The
 * backward pass returns dL/dH from dL/dT by implicit differentiation at the
 * optimal dual (section 4.1, eq (13); section 4.2), without unrolling.
 *
 * Conventions shared by every entry point.
 *   - All array pointers are DEVICE pointers owned by the caller (for example
 *     torch tensors on the GPU).  The library never allocates, frees or keeps
 *     them, and holds no global mutable state; calls are thread-safe.
 *   - Matrices are contiguous, row-major and stored back to back: element
 *     (b, i, j) of an [B, n, n] array is at offset (b*n + i)*n + j.
 *     The dual is [B, n] fp32: dual[b*n + j] = beta_j of matrix b, with the
 *     gauge beta_{n-1} = 0 (zero-based last column) stored explicitly.
 *   - Every pointer must be 16-byte aligned (iters and fallbacks of
 *     birkhoff_fwd_ex: 4-byte aligned); arrays must not overlap.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *     Work is enqueued asynchronously on it; nothing synchronizes.
 *   - B == 0 is a no-op that returns BIRKHOFF_OK (pointers may then be NULL).
 *   - Arguments are validated on the host before any HIP call; a rejected
 *     call enqueues nothing.
 *   - A matrix that does not reach `tol` within `max_iter` updates is not an
 *     error: its last iterate is written (see birkhoff_fwd_ex to detect it).
 *     Non-finite logits yield NaN in that matrix's outputs only.
 *   - The backward passes solve eq (13)'s system with Delta, the Hessian at
 *     the projection, by Cholesky.  Where Delta is numerically singular (a
 *     projection within rounding of a permutation on some rows and columns), dH
 *     does not depend on the undetermined part of the solution: a pivot below
 *     2^-24 (times the plan's mass for entropic OT) makes the solve fail, and it
 *     is repeated once with 2^-20 (mass + trace) added to the diagonal, which
 *     fails only for a non-finite Delta (the solution is then taken as 0 and the
 *     NaN stays in dH).  At an exact permutation (Delta = 0) the right-hand side
 *     is exactly 0 as well, and the result is the exact dH = 0.
 *
 * Return codes: BIRKHOFF_OK or one of the negative BIRKHOFF_E* codes below;
 * birkhoff_strerror() describes them.
 */
#ifndef BIRKHOFF_H
#define BIRKHOFF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BIRKHOFF_OK 0
#define BIRKHOFF_EINVAL (-1)  /* NULL pointer with B > 0, B < 0, unsupported n, tol <= 0 or NaN,
                                 max_iter < 1, iters < 1, or B too large for one launch */
#define BIRKHOFF_EALIGN (-2)  /* a pointer is not 16-byte aligned (iters, fallbacks: not 4-byte aligned) */
#define BIRKHOFF_ELAUNCH (-3) /* the HIP runtime rejected this call's kernel launch (the status that
                                 hipLaunchKernel returned for it; an error left by an earlier HIP call
                                 on the thread is neither reported here nor cleared) */

/* Forward pass, fp32 storage.
 *   logits   [B, n, n] fp32, input H
 *   T        [B, n, n] fp32, output: the projection of exp(H) onto B_n
 *   dual     [B, n]    fp32, output: beta with beta_{n-1} = 0, such that
 *            T_ij = exp(H_ij + beta_j) / sum_k exp(H_ik + beta_k)
 *            (section 3.1: rows of T are Softmax(H_i. + beta)); it is the only
 *            state the backward pass needs
 *   n        4 or 8
 *   tol      stop when every column sum of T is within tol of 1 (rows sum to one
 *            by construction); typical 1e-6
 *   max_iter cap on Newton updates (an accepted step or a fallback sweep), >= 1
 */
int birkhoff_fwd(const float* logits, float* T, float* dual, int64_t B, int n,
                 float tol, int max_iter, void* stream);

/* As birkhoff_fwd, and additionally writes per-matrix statistics (int32, [B]):
 *   iters[b]     the number of updates matrix b took to reach tol, or -1 when it
 *                did not reach tol within max_iter updates (or its input was
 *                not finite).  Must be non-NULL.
 *   fallbacks[b] how many of those updates were the Sinkhorn-Knopp fallback
 *                sweep, taken when no step size of the line search is accepted
 *                (blog post, section 2.2).  May be NULL.
 * A matrix counts as converged only if its T, rebuilt from the logits at the
 * returned dual (rows Softmax(H_i. + beta), section 3.1), also meets tol
 * whenever the iterate had entries below 2^-100 (logit spans of about 70 and
 * more, where multiplicatively formed entries may have underflowed); the
 * rebuilt T is then the one returned, and the iteration continues from it when
 * it misses tol.  birkhoff_fwd computes the same T and dual. */
int birkhoff_fwd_ex(const float* logits, float* T, float* dual, int32_t* iters, int32_t* fallbacks,
                    int64_t B, int n, float tol, int max_iter, void* stream);

/* Backward pass, fp32 storage (section 4.1 eq (13), section 4.2).
 *   logits [B, n, n] fp32, the forward input H
 *   dual   [B, n]    fp32, the forward's dual output
 *   dT     [B, n, n] fp32, upstream gradient dL/dT
 *   dH     [B, n, n] fp32, output dL/dH (sign already flipped from dL/dM, H = -M)
 * T is recomputed from (logits, dual); the Newton iterates are not needed. */
int birkhoff_bwd(const float* logits, const float* dual, const float* dT, float* dH,
                 int64_t B, int n, void* stream);

/* Backward pass from the projection itself, fp32 storage (section 4.2: the
 * gradient needs only T* and the upstream G; no dual, no exponentials).
 *   T  [B, n, n] fp32, a doubly stochastic projection (e.g. birkhoff_fwd's T)
 *   dT [B, n, n] fp32, upstream gradient dL/dT
 *   dH [B, n, n] fp32, output dL/dH
 * Moves 3n^2 * 4 bytes per matrix instead of birkhoff_bwd's 3n^2 * 4 + 4n.
 * dH agrees with birkhoff_bwd up to rounding (birkhoff_bwd recomputes T from
 * the logits and the dual; this entry point takes T as given). */
int birkhoff_bwd_from_T(const float* T, const float* dT, float* dH, int64_t B, int n, void* stream);

/* Comparison baseline: exactly `iters` Sinkhorn-Knopp sweeps (section 2.2 eq (2),
 * evaluated in the log domain as the block coordinate ascent of eq (7)) from
 * v = 1, then T = diag(u) exp(H) diag(v).  One sweep = row then column
 * normalisation, so after it the columns sum to one and the rows carry the error.
 *   logits [B, n, n] fp32 input, T [B, n, n] fp32 output, iters >= 1. */
int sinkhorn_fwd(const float* logits, float* T, int64_t B, int n, int iters, void* stream);

/* bf16-storage variants: logits, T, dT and dH hold bfloat16 bit patterns
 * (uint16_t), the dual stays fp32; all arithmetic is fp32 and T / dH are
 * rounded to bf16 (nearest, ties to even) when stored.  Otherwise identical to
 * the fp32 entry points. */
int birkhoff_fwd_bf16(const uint16_t* logits, uint16_t* T, float* dual, int64_t B, int n,
                      float tol, int max_iter, void* stream);
int birkhoff_bwd_bf16(const uint16_t* logits, const float* dual, const uint16_t* dT,
                      uint16_t* dH, int64_t B, int n, void* stream);

/* Forward and backward in one launch, for callers that already hold dL/dT when
 * they project (a training step that has the loss gradient at hand, or a fused
 * benchmark pass).  Computes exactly what birkhoff_fwd computes (T and dual
 * are bit-identical to it) and then dH by eq (13) at the final iterate T, still
 * in registers, instead of recomputing T from (logits, dual) as birkhoff_bwd
 * does; dH therefore agrees with birkhoff_fwd + birkhoff_bwd up to rounding.
 * Moves 4n^2 s + 4n bytes per matrix (s = storage bytes per element) instead of
 * the 5n^2 s + 8n of the two separate calls, in one launch.
 *   logits [B, n, n] input H;  dT [B, n, n] input dL/dT
 *   T      [B, n, n] output;   dual [B, n] fp32 output;  dH [B, n, n] output dL/dH
 *   n, tol, max_iter as for birkhoff_fwd.  No argument may alias another. */
int birkhoff_fwd_bwd(const float* logits, const float* dT, float* T, float* dual, float* dH, int64_t B, int n,
                     float tol, int max_iter, void* stream);
int birkhoff_fwd_bwd_bf16(const uint16_t* logits, const uint16_t* dT, uint16_t* T, float* dual, uint16_t* dH,
                          int64_t B, int n, float tol, int max_iter, void* stream);

/* ---- General small entropic optimal transport ------------------------------
 * For every one of B independent problems with cost M (n x m), marginals
 * a > 0 (n) and b > 0 (m) with sum(a) = sum(b), and regularisation eta > 0,
 * the forward pass returns the plan
 *
 *     T = argmin { <T, M> - eta h(T) : T 1 = a, T^T 1 = b }      (section 2.3, eq (3)),
 *
 * T_ij = exp((alpha_i + beta_j - M_ij) / eta) at the optimal dual (eq (4)).  It is
 * found by Newton's method on the reduced dual of eq (8) with the gradient and
 * Hessian of eq (9), with the same step-size rule and Sinkhorn fallback (eqs
 * (5)-(7)) as the Birkhoff forward; the backward pass is eq (13) (section 4.1).
 * The Birkhoff projection is the case a = b = 1, eta = 1, M = -H.
 *
 * Shapes: 1 <= n <= 8 rows, 2 <= m <= 8 columns.  Layouts as above: cost, T, dT
 * and dcost are [B, n, m] row-major back to back; the dual is [B, m].  With
 * shared_marginals == 0, a is [B, n] and b is [B, m] (one pair per problem);
 * with shared_marginals != 0, a is [n] and b is [m], used by every problem
 * (these two need only 4-byte alignment).  Marginals are not checked for
 * positivity or equal sums: a problem whose marginals violate this has no
 * plan, and its outputs are whatever the iteration reached (its iters entry
 * is -1 unless the column residual happens to fall below tol).
 * Return codes as above; BIRKHOFF_EINVAL also covers n or m out of range and
 * eta <= 0 or not finite. */

/* Forward pass (fp32).
 *   cost     [B, n, m] input M;  a, b marginals (see shared_marginals)
 *   T        [B, n, m] output plan (rows sum to a up to rounding)
 *   dual     [B, m] output beta in cost units with beta_{m-1} = 0, such that
 *            T_ij = a_i exp((beta_j - M_ij) / eta) / sum_k exp((beta_k - M_ik) / eta)
 *            (section 3.1)
 *   iters    [B] int32 output or NULL: updates taken, -1 when tol was not reached
 *   tol      stop when every column sum of T is within tol of b_j (absolute)
 *   max_iter cap on updates (accepted steps or fallback sweeps), >= 1 */
int birkhoff_eot_fwd(const float* cost, const float* a, const float* b, int shared_marginals, float* T, float* dual,
                     int32_t* iters, int64_t B, int n, int m, float eta, float tol, int max_iter, void* stream);

/* Backward pass (fp32), eq (13): dcost = dL/dM from the plan and dL/dT.
 *   T      [B, n, m] a plan (e.g. birkhoff_eot_fwd's output)
 *   dT     [B, n, m] upstream gradient dL/dT
 *   a      row marginals (see shared_marginals); b is not needed: eq (13)'s Delta
 *          is recomputed from T as the Hessian of eq (9) at T (section 4.2),
 *          which equals diag(b_{-m}) - T_{-m}^T diag(a)^-1 T_{-m} at the optimum
 *   dcost  [B, n, m] output dL/dM
 * No argument may alias another. */
int birkhoff_eot_bwd(const float* T, const float* dT, const float* a, int shared_marginals, float* dcost, int64_t B,
                     int n, int m, float eta, void* stream);

/* ---- The projection's consumer in an mHC layer --------------------------------
 * The projected matrix is the residual mapping H_res of the layer update
 * x_{l+1} = H_res x_l + H_post^T F(H_pre x_l) (section 2.1), applied to each
 * token's n x C hidden matrix x (n streams of C features).  These entry points
 * fuse that mixing into the projection (forward) and run its backward together
 * with eq (13) (backward).  n must be 4.  Per token b: logits [B, 4, 4] fp32,
 * T [B, 4, 4] fp32, dual [B, 4] fp32, dH [B, 4, 4] fp32; x, y, dy, dx
 * [B, 4, C] row-major (fp32, or bf16 bit patterns for the _bf16 variants), so
 * element (b, i, c) is at (b*4 + i)*C + c.  C >= 0 must be a multiple of 4
 * (fp32) or 8 (bf16) so that every row is a whole number of 16-byte chunks;
 * x, y, dy, dx may be NULL when C == 0.  Arithmetic is fp32; bf16 results are
 * rounded to nearest, ties to even.  Return codes as above; BIRKHOFF_EINVAL
 * also covers n != 4, C out of range or not such a multiple. */

/* Forward: T and dual exactly as birkhoff_fwd computes them (bit-identical), and
 *   y[b] = T[b] x[b]     (y_ic = sum_j T_ij x_jc)
 * in the same launch; T is not read back from memory for the product. */
int birkhoff_fwd_mix(const float* logits, const float* x, float* T, float* dual, float* y, int64_t B, int n,
                     int64_t C, float tol, int max_iter, void* stream);
int birkhoff_fwd_mix_bf16(const float* logits, const uint16_t* x, float* T, float* dual, uint16_t* y, int64_t B,
                          int n, int64_t C, float tol, int max_iter, void* stream);

/* Backward of y = T x followed by the projection's backward, for upstream dy:
 *   dx[b] = T[b]^T dy[b],   dT[b] = dy[b] x[b]^T   (sum over the C columns),
 *   dH[b] = dL/dlogits from (T[b], dT[b]) by eq (13), as birkhoff_bwd_from_T.
 * T is the forward's output; dT itself is not stored. */
int birkhoff_mix_bwd(const float* T, const float* x, const float* dy, float* dx, float* dH, int64_t B, int n,
                     int64_t C, void* stream);
int birkhoff_mix_bwd_bf16(const float* T, const uint16_t* x, const uint16_t* dy, uint16_t* dx, float* dH, int64_t B,
                          int n, int64_t C, void* stream);

/* ---- measurement aid (not part of the method) ------------------------------
 *
 * birkhoff_clock_probe: the engine clock that kernels run at, for benchmark
 * reports (the driver's sampled clock can lag the load).  Enqueues on `stream`
 * `blocks` workgroups of one wave each; workgroup k writes
 * counts[2k] = shader-clock cycles and counts[2k+1] = ticks of the
 * constant-rate counter over the same interval of about `ticks` ticks.  The
 * clock in kHz is sum(counts[even]) / sum(counts[odd]) * *wall_khz, where
 * *wall_khz (written before return, on the host) is the constant counter's
 * rate on the current device.  counts: device memory of 2*blocks uint64,
 * 16-byte aligned, owned by the caller, valid once the stream has reached the
 * probe.  1 <= blocks <= 65536, 1 <= ticks <= 2^20.  Returns BIRKHOFF_EINVAL
 * for a NULL pointer or a size out of range, BIRKHOFF_EALIGN for a misaligned
 * counts, BIRKHOFF_ELAUNCH when the device query or the launch fails. */
int birkhoff_clock_probe(uint64_t* counts, int blocks, int ticks, int* wall_khz, void* stream);

/* Static description of a return code (never NULL). */
const char* birkhoff_strerror(int code);

/* ABI version, currently 2 (version 1's birkhoff_fwd_ex had no fallbacks argument). */
int birkhoff_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BIRKHOFF_H */
