// mix.hip -- C ABI entry points for the projection fused with its mHC consumer,
// the residual-stream mixing y = H_res x (declared in include/birkhoff.h):
// argument validation and launch.  As everywhere in the library, arguments are
// checked before any HIP call, launches are asynchronous on the caller's
// stream, and nothing is allocated.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "birkhoff.h"
#include "mix.hpp"

namespace {

using birk::kBlock;
using birk::mix::kTokens;

// grid.x <= 2^31 - 1 workgroups of kTokens tokens
constexpr int64_t kMaxTokens = (int64_t)0x7fffffff * kTokens;
// keep every element offset (tokens * 4 * C) far inside int64
constexpr int64_t kMaxC = (int64_t)1 << 28;
constexpr int64_t kMaxElements = (int64_t)1 << 60;

int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (p == nullptr) return BIRKHOFF_EINVAL;
    for (const void* p : ps)
        if (reinterpret_cast<uintptr_t>(p) & 15u) return BIRKHOFF_EALIGN;
    return BIRKHOFF_OK;
}

// B tokens of n = 4 streams with C features; C * element size a multiple of 16
int check_shape(int64_t B, int n, int64_t C, int per_chunk) {
    if (B < 0 || B > kMaxTokens || n != 4) return BIRKHOFF_EINVAL;
    if (C < 0 || C > kMaxC || C % per_chunk != 0) return BIRKHOFF_EINVAL;
    if (C > 0 && B > kMaxElements / (4 * C)) return BIRKHOFF_EINVAL;
    return BIRKHOFF_OK;
}

int launched() { return hipGetLastError() == hipSuccess ? BIRKHOFF_OK : BIRKHOFF_ELAUNCH; }

dim3 grid_for(int64_t B) { return dim3((unsigned)((B + kTokens - 1) / kTokens)); }

template <typename XT>
int fwd_mix(const float* logits, const XT* x, float* T, float* dual, XT* y, int64_t B, int n, int64_t C, float tol,
            int max_iter, void* stream) {
    constexpr int V = birk::mix::Vec<XT>::V;
    int rc = check_shape(B, n, C, V);
    if (rc == BIRKHOFF_OK && (!(tol > 0.0f) || !std::isfinite(tol) || max_iter < 1)) rc = BIRKHOFF_EINVAL;
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({logits, T, dual});
    if (rc == BIRKHOFF_OK && C > 0) rc = check_ptrs({x, y});
    if (rc != BIRKHOFF_OK) return rc;
    hipLaunchKernelGGL((birk::mix::project_mix_kernel<XT>), grid_for(B), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), logits, x, T, dual, y, B, C / V, tol, max_iter);
    return launched();
}

template <typename XT>
int mix_bwd(const float* T, const XT* x, const XT* dy, XT* dx, float* dH, int64_t B, int n, int64_t C,
            void* stream) {
    constexpr int V = birk::mix::Vec<XT>::V;
    int rc = check_shape(B, n, C, V);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({T, dH});
    if (rc == BIRKHOFF_OK && C > 0) rc = check_ptrs({x, dy, dx});
    if (rc != BIRKHOFF_OK) return rc;
    hipLaunchKernelGGL((birk::mix::mix_bwd_kernel<XT>), grid_for(B), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), T, x, dy, dx, dH, B, C / V);
    return launched();
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
