// mix.hip -- C ABI entry points for the projection fused with its mHC consumer,
// the residual-stream mixing y = H_res x (declared in include/birkhoff.h):
// argument validation and launch.  As everywhere in the library, arguments are
// checked (abi_checks.hpp) before any HIP call, launches are asynchronous on
// the caller's stream and report their own status, and nothing is allocated.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "abi_checks.hpp"
#include "birkhoff.h"
#include "launch.hpp"
#include "mix.hpp"

namespace {

using birk::kBlock;
using birk::mix::kTokens;

static_assert(birk::abi::kMixTokens == kTokens, "the token limit assumes the kernels' geometry");

dim3 grid_for(int64_t B) { return dim3((unsigned)((B + kTokens - 1) / kTokens)); }

template <typename XT>
int fwd_mix(const float* logits, const XT* x, float* T, float* dual, XT* y, int64_t B, int n, int64_t C, float tol,
            int max_iter, void* stream) {
    constexpr int V = birk::mix::Vec<XT>::V;
    const int rc = birk::abi::validate_mix_fwd(logits, x, T, dual, y, B, n, C, V, tol, max_iter);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    return birk::launch(birk::mix::project_mix_kernel<XT>, grid_for(B), dim3(kBlock), static_cast<hipStream_t>(stream),
                        logits, x, T, dual, y, B, C / V, tol, max_iter);
}

template <typename XT>
int mix_bwd(const float* T, const XT* x, const XT* dy, XT* dx, float* dH, int64_t B, int n, int64_t C,
            void* stream) {
    constexpr int V = birk::mix::Vec<XT>::V;
    const int rc = birk::abi::validate_mix_bwd(T, x, dy, dx, dH, B, n, C, V);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    return birk::launch(birk::mix::mix_bwd_kernel<XT>, grid_for(B), dim3(kBlock), static_cast<hipStream_t>(stream), T,
                        x, dy, dx, dH, B, C / V);
}

}  // namespace

extern "C" {

int birkhoff_fwd_mix(const float* logits, const float* x, float* T, float* dual, float* y, int64_t B, int n,
                     int64_t C, float tol, int max_iter, void* stream) {
    return fwd_mix<float>(logits, x, T, dual, y, B, n, C, tol, max_iter, stream);
}

int birkhoff_fwd_mix_bf16(const float* logits, const uint16_t* x, float* T, float* dual, uint16_t* y, int64_t B,
                          int n, int64_t C, float tol, int max_iter, void* stream) {
    return fwd_mix<uint16_t>(logits, x, T, dual, y, B, n, C, tol, max_iter, stream);
}

int birkhoff_mix_bwd(const float* T, const float* x, const float* dy, float* dx, float* dH, int64_t B, int n,
                     int64_t C, void* stream) {
    return mix_bwd<float>(T, x, dy, dx, dH, B, n, C, stream);
}

int birkhoff_mix_bwd_bf16(const float* T, const uint16_t* x, const uint16_t* dy, uint16_t* dx, float* dH, int64_t B,
                          int n, int64_t C, void* stream) {
    return mix_bwd<uint16_t>(T, x, dy, dx, dH, B, n, C, stream);
}

}  // extern "C"
