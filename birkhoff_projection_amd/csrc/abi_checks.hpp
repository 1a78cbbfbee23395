// abi_checks.hpp -- argument validation of every C ABI entry point in
// include/birkhoff.h, in plain C++ (no HIP): the entry points call these
// before any HIP call, and a host-side test compiles this header on its own
// with address and undefined-behaviour sanitizers.
//
// Each validator returns BIRKHOFF_OK, BIRKHOFF_EINVAL or BIRKHOFF_EALIGN.  The
// scalar arguments are checked first and an empty batch (B == 0) is accepted
// before any pointer is looked at, so that an empty call may pass NULL
// pointers; the caller returns at once when the result is not BIRKHOFF_OK or
// when B == 0, and launches otherwise.  Pointers are only compared and their
// addresses tested for alignment; nothing is dereferenced.
#pragma once

#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "birkhoff.h"

namespace birk {
namespace abi {

// Largest batches one launch covers: grid.x is at most 2^31 - 1 workgroups.
// Projections: 256 lanes per workgroup, an 8 x 8 matrix takes two lanes.
constexpr int64_t kProjLanesPerGroup = 256;
constexpr int64_t kMaxBatch = (int64_t)0x7fffffff * kProjLanesPerGroup / 2;
// General entropic OT: at least 128 lanes per workgroup, one problem per lane.
constexpr int64_t kMaxEotBatch = (int64_t)0x7fffffff * 128;
constexpr int kMaxEotSide = 8;
// The fused mixing: kMixTokens tokens per workgroup; C and the element count
// bounded so that every offset stays far inside int64.
constexpr int64_t kMixTokens = 4;
constexpr int64_t kMaxMixTokens = (int64_t)0x7fffffff * kMixTokens;
constexpr int64_t kMaxMixC = (int64_t)1 << 28;
constexpr int64_t kMaxMixElements = (int64_t)1 << 60;

inline bool misaligned(const void* p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) != 0; }

// every pointer non-NULL (else EINVAL) and 16-byte aligned (else EALIGN)
inline int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (p == nullptr) return BIRKHOFF_EINVAL;
    for (const void* p : ps)
        if (misaligned(p, 16)) return BIRKHOFF_EALIGN;
    return BIRKHOFF_OK;
}

// an int32 per-matrix output: NULL allowed unless required; 4-byte aligned
inline int check_counts(const int32_t* p, bool required) {
    if (p == nullptr) return required ? BIRKHOFF_EINVAL : BIRKHOFF_OK;
    return misaligned(p, 4) ? BIRKHOFF_EALIGN : BIRKHOFF_OK;
}

inline bool bad_tol(float tol, int max_iter) { return !(tol > 0.0f) || !std::isfinite(tol) || max_iter < 1; }

inline bool bad_eta(float eta) { return !(eta > 0.0f) || !std::isfinite(eta); }

inline int check_batch(int64_t B, int n) {
    if (B < 0 || B > kMaxBatch) return BIRKHOFF_EINVAL;
    if (n != 4 && n != 8) return BIRKHOFF_EINVAL;
    return BIRKHOFF_OK;
}

// birkhoff_fwd / _bf16 / _ex: iters is required by birkhoff_fwd_ex (need_iters),
// fallbacks is optional there; both are NULL for the plain forward.
inline int validate_fwd(const void* logits, const void* T, const float* dual, const int32_t* iters,
                        const int32_t* fallbacks, bool need_iters, int64_t B, int n, float tol, int max_iter) {
    int rc = check_batch(B, n);
    if (rc == BIRKHOFF_OK && bad_tol(tol, max_iter)) rc = BIRKHOFF_EINVAL;
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({logits, T, dual});
    if (rc == BIRKHOFF_OK && need_iters) rc = check_counts(iters, true);
    if (rc == BIRKHOFF_OK && need_iters) rc = check_counts(fallbacks, false);
    return rc;
}

inline int validate_bwd(const void* logits, const float* dual, const void* dT, const void* dH, int64_t B, int n) {
    const int rc = check_batch(B, n);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    return check_ptrs({logits, dual, dT, dH});
}

inline int validate_bwd_from_T(const float* T, const float* dT, const float* dH, int64_t B, int n) {
    const int rc = check_batch(B, n);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    return check_ptrs({T, dT, dH});
}

inline int validate_sinkhorn(const float* logits, const float* T, int64_t B, int n, int iters) {
    int rc = check_batch(B, n);
    if (rc == BIRKHOFF_OK && iters < 1) rc = BIRKHOFF_EINVAL;
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    return check_ptrs({logits, T});
}

inline int validate_fused(const void* logits, const void* dT, const void* T, const float* dual, const void* dH,
                          int64_t B, int n, float tol, int max_iter) {
    int rc = check_batch(B, n);
    if (rc == BIRKHOFF_OK && bad_tol(tol, max_iter)) rc = BIRKHOFF_EINVAL;
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    return check_ptrs({logits, dT, T, dual, dH});
}

// ---- general entropic OT

inline int check_eot_shape(int64_t B, int n, int m) {
    if (B < 0 || B > kMaxEotBatch) return BIRKHOFF_EINVAL;
    if (n < 1 || n > kMaxEotSide || m < 2 || m > kMaxEotSide) return BIRKHOFF_EINVAL;
    return BIRKHOFF_OK;
}

// marginals: per problem 16-byte aligned, shared by the batch 4-byte aligned
inline int check_marginal(const float* p, int shared) {
    if (p == nullptr) return BIRKHOFF_EINVAL;
    return misaligned(p, shared ? 4 : 16) ? BIRKHOFF_EALIGN : BIRKHOFF_OK;
}

inline int validate_eot_fwd(const float* cost, const float* a, const float* b, int shared, const float* T,
                            const float* dual, const int32_t* iters, int64_t B, int n, int m, float eta, float tol,
                            int max_iter) {
    int rc = check_eot_shape(B, n, m);
    if (rc == BIRKHOFF_OK && (bad_eta(eta) || bad_tol(tol, max_iter))) rc = BIRKHOFF_EINVAL;
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({cost, T, dual});
    if (rc == BIRKHOFF_OK) rc = check_marginal(a, shared);
    if (rc == BIRKHOFF_OK) rc = check_marginal(b, shared);
    if (rc == BIRKHOFF_OK) rc = check_counts(iters, false);
    return rc;
}

inline int validate_eot_bwd(const float* T, const float* dT, const float* a, int shared, const float* dcost,
                            int64_t B, int n, int m, float eta) {
    int rc = check_eot_shape(B, n, m);
    if (rc == BIRKHOFF_OK && bad_eta(eta)) rc = BIRKHOFF_EINVAL;
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({T, dT, dcost});
    if (rc == BIRKHOFF_OK) rc = check_marginal(a, shared);
    return rc;
}

// ---- the projection fused with the residual mixing: B tokens of n = 4 streams
// with C features, C a multiple of per_chunk (the elements of a 16-byte chunk)

inline int check_mix_shape(int64_t B, int n, int64_t C, int per_chunk) {
    if (B < 0 || B > kMaxMixTokens || n != 4) return BIRKHOFF_EINVAL;
    if (C < 0 || C > kMaxMixC || C % per_chunk != 0) return BIRKHOFF_EINVAL;
    if (C > 0 && B > kMaxMixElements / (4 * C)) return BIRKHOFF_EINVAL;
    return BIRKHOFF_OK;
}

inline int validate_mix_fwd(const float* logits, const void* x, const float* T, const float* dual, const void* y,
                            int64_t B, int n, int64_t C, int per_chunk, float tol, int max_iter) {
    int rc = check_mix_shape(B, n, C, per_chunk);
    if (rc == BIRKHOFF_OK && bad_tol(tol, max_iter)) rc = BIRKHOFF_EINVAL;
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({logits, T, dual});
    if (rc == BIRKHOFF_OK && C > 0) rc = check_ptrs({x, y});
    return rc;
}

inline int validate_mix_bwd(const float* T, const void* x, const void* dy, const void* dx, const float* dH,
                            int64_t B, int n, int64_t C, int per_chunk) {
    int rc = check_mix_shape(B, n, C, per_chunk);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({T, dH});
    if (rc == BIRKHOFF_OK && C > 0) rc = check_ptrs({x, dy, dx});
    return rc;
}

}  // namespace abi
}  // namespace birk
