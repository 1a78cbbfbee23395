// eot.hip -- the C ABI entry points for batched small entropic OT with
// general cost, marginals and regularisation (declared in include/birkhoff.h):
// argument validation, dispatch on the shape (n, m) and launch.
//
// As for the Birkhoff entry points, every argument is checked (abi_checks.hpp)
// before any HIP call, launches are asynchronous on the caller's stream and
// report their own status, and nothing is allocated.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "abi_checks.hpp"
#include "birkhoff.h"
#include "eot_launch.hpp"

namespace {

using birk::eot::BwdArgs;
using birk::eot::by_m;
using birk::eot::FwdArgs;

static_assert(birk::abi::kMaxEotSide == 8, "shapes up to 8 x 8 are instantiated");
static_assert(birk::eot::Waves<64>::threads >= 128, "the batch limit assumes at least 128 lanes per workgroup");

// shape dispatch: n in [1, 8]
template <typename Args>
int by_shape(int n, int m, const Args& x) {
    switch (n) {
        case 1: return by_m<1>(m, x);
        case 2: return by_m<2>(m, x);
        case 3: return by_m<3>(m, x);
        case 4: return by_m<4>(m, x);
        case 5: return by_m<5>(m, x);
        case 6: return by_m<6>(m, x);
        case 7: return by_m<7>(m, x);
        default: return by_m<8>(m, x);
    }
}

}  // namespace

extern "C" {

int birkhoff_eot_fwd(const float* cost, const float* a, const float* b, int shared_marginals, float* T, float* dual,
                     int32_t* iters, int64_t B, int n, int m, float eta, float tol, int max_iter, void* stream) {
    const int rc = birk::abi::validate_eot_fwd(cost, a, b, shared_marginals, T, dual, iters, B, n, m, eta, tol,
                                               max_iter);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    const FwdArgs x{cost, a, b, shared_marginals != 0, T, dual, iters, B, eta, tol, max_iter,
                    static_cast<hipStream_t>(stream)};
    return by_shape(n, m, x);
}

int birkhoff_eot_bwd(const float* T, const float* dT, const float* a, int shared_marginals, float* dcost, int64_t B,
                     int n, int m, float eta, void* stream) {
    const int rc = birk::abi::validate_eot_bwd(T, dT, a, shared_marginals, dcost, B, n, m, eta);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    const BwdArgs x{T, dT, a, shared_marginals != 0, dcost, B, eta, static_cast<hipStream_t>(stream)};
    return by_shape(n, m, x);
}

}  // extern "C"
