// eot.hip -- the C ABI entry points for batched small entropic OT with
// general cost, marginals and regularisation (declared in include/birkhoff.h):
// argument validation, dispatch on the shape (n, m) and launch.
//
// As for the Birkhoff entry points, every argument is checked before any HIP
// call, launches are asynchronous on the caller's stream, and nothing is
// allocated.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "birkhoff.h"
#include "eot_launch.hpp"

namespace {

using birk::eot::BwdArgs;
using birk::eot::by_m;
using birk::eot::FwdArgs;

constexpr int kMaxSide = 8;
// grid.x <= 2^31 - 1 workgroups of at least 128 lanes, one problem per lane
constexpr int64_t kMaxBatch = (int64_t)0x7fffffff * 128;

int check_shape(int64_t B, int n, int m) {
    if (B < 0 || B > kMaxBatch) return BIRKHOFF_EINVAL;
    if (n < 1 || n > kMaxSide || m < 2 || m > kMaxSide) return BIRKHOFF_EINVAL;
    return BIRKHOFF_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (p == nullptr) return BIRKHOFF_EINVAL;
    for (const void* p : ps)
        if (reinterpret_cast<uintptr_t>(p) & 15u) return BIRKHOFF_EALIGN;
    return BIRKHOFF_OK;
}

// marginals shared by the batch only need float alignment
int check_marginal(const float* p, int shared) {
    if (p == nullptr) return BIRKHOFF_EINVAL;
    const uintptr_t mask = shared ? 3u : 15u;
    return (reinterpret_cast<uintptr_t>(p) & mask) ? BIRKHOFF_EALIGN : BIRKHOFF_OK;
}

int launched() { return hipGetLastError() == hipSuccess ? BIRKHOFF_OK : BIRKHOFF_ELAUNCH; }

// shape dispatch: n in [1, 8]
template <typename Args>
void by_shape(int n, int m, const Args& x) {
    switch (n) {
        case 1: by_m<1>(m, x); break;
        case 2: by_m<2>(m, x); break;
        case 3: by_m<3>(m, x); break;
        case 4: by_m<4>(m, x); break;
        case 5: by_m<5>(m, x); break;
        case 6: by_m<6>(m, x); break;
        case 7: by_m<7>(m, x); break;
        default: by_m<8>(m, x); break;
    }
}

bool bad_eta(float eta) { return !(eta > 0.0f) || !std::isfinite(eta); }

}  // namespace

extern "C" {

int birkhoff_eot_fwd(const float* cost, const float* a, const float* b, int shared_marginals, float* T, float* dual,
                     int32_t* iters, int64_t B, int n, int m, float eta, float tol, int max_iter, void* stream) {
    int rc = check_shape(B, n, m);
    if (rc == BIRKHOFF_OK && (bad_eta(eta) || !(tol > 0.0f) || !std::isfinite(tol) || max_iter < 1))
        rc = BIRKHOFF_EINVAL;
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({cost, T, dual});
    if (rc == BIRKHOFF_OK) rc = check_marginal(a, shared_marginals);
    if (rc == BIRKHOFF_OK) rc = check_marginal(b, shared_marginals);
    if (rc == BIRKHOFF_OK && iters != nullptr && (reinterpret_cast<uintptr_t>(iters) & 3u)) rc = BIRKHOFF_EALIGN;
    if (rc != BIRKHOFF_OK) return rc;
    const FwdArgs x{cost, a, b, shared_marginals != 0, T, dual, iters, B, eta, tol, max_iter,
                    static_cast<hipStream_t>(stream)};
    by_shape(n, m, x);
    return launched();
}

int birkhoff_eot_bwd(const float* T, const float* dT, const float* a, int shared_marginals, float* dcost, int64_t B,
                     int n, int m, float eta, void* stream) {
    int rc = check_shape(B, n, m);
    if (rc == BIRKHOFF_OK && bad_eta(eta)) rc = BIRKHOFF_EINVAL;
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({T, dT, dcost});
    if (rc == BIRKHOFF_OK) rc = check_marginal(a, shared_marginals);
    if (rc != BIRKHOFF_OK) return rc;
    const BwdArgs x{T, dT, a, shared_marginals != 0, dcost, B, eta, static_cast<hipStream_t>(stream)};
    by_shape(n, m, x);
    return launched();
}

}  // extern "C"
