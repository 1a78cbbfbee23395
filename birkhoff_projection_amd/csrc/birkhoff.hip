// birkhoff.hip -- the C ABI of libbirkhoff (declared in include/birkhoff.h):
// host-side argument validation, dispatch on n and storage type, and launch.
//
// Every argument is checked before any HIP call, so a rejected call enqueues
// nothing and never touches the device.  Launches are asynchronous on the
// caller's stream; the library allocates nothing and keeps no state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "birkhoff.h"
#include "projection.hpp"

namespace {

using birk::kBlock;

// Largest batch one launch covers: grid.x <= 2^31 - 1 workgroups of kBlock lanes,
// and an 8 x 8 matrix takes two lanes.
constexpr int64_t kMaxBatch = (int64_t)0x7fffffff * kBlock / 2;

// lanes per matrix, as in the kernels
int lanes_per_matrix(int n) { return n == 8 ? birk::Split<8>::R : birk::Split<4>::R; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int check_batch(int64_t B, int n) {
    if (B < 0 || B > kMaxBatch) return BIRKHOFF_EINVAL;
    if (n != 4 && n != 8) return BIRKHOFF_EINVAL;
    return BIRKHOFF_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (p == nullptr) return BIRKHOFF_EINVAL;
    for (const void* p : ps)
        if (misaligned(p)) return BIRKHOFF_EALIGN;
    return BIRKHOFF_OK;
}

int check_tol(float tol, int max_iter) {
    if (!(tol > 0.0f) || !std::isfinite(tol) || max_iter < 1) return BIRKHOFF_EINVAL;
    return BIRKHOFF_OK;
}

int launched() { return hipGetLastError() == hipSuccess ? BIRKHOFF_OK : BIRKHOFF_ELAUNCH; }

dim3 grid_for(int64_t B, int n) {
    const int64_t lanes = B * lanes_per_matrix(n);
    return dim3((unsigned)((lanes + kBlock - 1) / kBlock));
}

template <int N, typename IO>
int fwd_launch(const IO* logits, IO* T, float* dual, int32_t* iters, int64_t B, float tol, int max_iter,
               hipStream_t s) {
    if constexpr (N == 4) {
        if (iters)
            hipLaunchKernelGGL((birk::newton_fwd_gather_kernel<IO, true>), grid_for(B, N), dim3(kBlock), 0, s,
                               logits, T, dual, iters, B, tol, max_iter);
        else
            hipLaunchKernelGGL((birk::newton_fwd_gather_kernel<IO, false>), grid_for(B, N), dim3(kBlock), 0, s,
                               logits, T, dual, iters, B, tol, max_iter);
    } else {
        if (iters)
            hipLaunchKernelGGL((birk::newton_fwd_kernel<N, IO, true>), grid_for(B, N), dim3(kBlock), 0, s, logits,
                               T, dual, iters, B, tol, max_iter);
        else
            hipLaunchKernelGGL((birk::newton_fwd_kernel<N, IO, false>), grid_for(B, N), dim3(kBlock), 0, s, logits,
                               T, dual, iters, B, tol, max_iter);
    }
    return launched();
}

template <typename IO>
int fwd_entry(const IO* logits, IO* T, float* dual, int32_t* iters, bool need_iters, int64_t B, int n, float tol,
              int max_iter, void* stream) {
    int rc = check_batch(B, n);
    if (rc == BIRKHOFF_OK) rc = check_tol(tol, max_iter);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({logits, T, dual});
    if (rc == BIRKHOFF_OK && need_iters)
        rc = iters == nullptr ? BIRKHOFF_EINVAL : (reinterpret_cast<uintptr_t>(iters) & 3u) ? BIRKHOFF_EALIGN : rc;
    if (rc != BIRKHOFF_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return n == 4 ? fwd_launch<4, IO>(logits, T, dual, iters, B, tol, max_iter, s)
                  : fwd_launch<8, IO>(logits, T, dual, iters, B, tol, max_iter, s);
}

template <typename IO>
int bwd_entry(const IO* logits, const float* dual, const IO* dT, IO* dH, int64_t B, int n, void* stream) {
    int rc = check_batch(B, n);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({logits, dual, dT, dH});
    if (rc != BIRKHOFF_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 4)
        hipLaunchKernelGGL((birk::implicit_bwd_kernel<4, IO>), grid_for(B, 4), dim3(kBlock), 0, s, logits, dual, dT, dH,
                           B);
    else
        hipLaunchKernelGGL((birk::implicit_bwd_kernel<8, IO>), grid_for(B, 8), dim3(kBlock), 0, s, logits, dual, dT, dH,
                           B);
    return launched();
}

template <typename IO>
int fused_entry(const IO* logits, const IO* dT, IO* T, float* dual, IO* dH, int64_t B, int n, float tol,
                int max_iter, void* stream) {
    int rc = check_batch(B, n);
    if (rc == BIRKHOFF_OK) rc = check_tol(tol, max_iter);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({logits, dT, T, dual, dH});
    if (rc != BIRKHOFF_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 4)
        hipLaunchKernelGGL((birk::fused_fwd_bwd_kernel<4, IO>), grid_for(B, 4), dim3(kBlock), 0, s, logits, dT, T, dual,
                           dH, B, tol, max_iter);
    else
        hipLaunchKernelGGL((birk::fused_fwd_bwd_kernel<8, IO>), grid_for(B, 8), dim3(kBlock), 0, s, logits, dT, T, dual,
                           dH, B, tol, max_iter);
    return launched();
}

}  // namespace

extern "C" {

int birkhoff_fwd(const float* logits, float* T, float* dual, int64_t B, int n, float tol, int max_iter,
                 void* stream) {
    return fwd_entry<float>(logits, T, dual, nullptr, false, B, n, tol, max_iter, stream);
}

int birkhoff_fwd_ex(const float* logits, float* T, float* dual, int32_t* iters, int64_t B, int n, float tol,
                    int max_iter, void* stream) {
    return fwd_entry<float>(logits, T, dual, iters, true, B, n, tol, max_iter, stream);
}

int birkhoff_bwd(const float* logits, const float* dual, const float* dT, float* dH, int64_t B, int n,
                 void* stream) {
    return bwd_entry<float>(logits, dual, dT, dH, B, n, stream);
}

int sinkhorn_fwd(const float* logits, float* T, int64_t B, int n, int iters, void* stream) {
    int rc = check_batch(B, n);
    if (rc == BIRKHOFF_OK && iters < 1) rc = BIRKHOFF_EINVAL;
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({logits, T});
    if (rc != BIRKHOFF_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 4)
        hipLaunchKernelGGL((birk::sinkhorn_kernel<4, float>), grid_for(B, 4), dim3(kBlock), 0, s, logits, T, B, iters);
    else
        hipLaunchKernelGGL((birk::sinkhorn_kernel<8, float>), grid_for(B, 8), dim3(kBlock), 0, s, logits, T, B, iters);
    return launched();
}

int birkhoff_fwd_bf16(const uint16_t* logits, uint16_t* T, float* dual, int64_t B, int n, float tol, int max_iter,
                      void* stream) {
    return fwd_entry<uint16_t>(logits, T, dual, nullptr, false, B, n, tol, max_iter, stream);
}

int birkhoff_bwd_bf16(const uint16_t* logits, const float* dual, const uint16_t* dT, uint16_t* dH, int64_t B, int n,
                      void* stream) {
    return bwd_entry<uint16_t>(logits, dual, dT, dH, B, n, stream);
}

int birkhoff_bwd_from_T(const float* T, const float* dT, float* dH, int64_t B, int n, void* stream) {
    int rc = check_batch(B, n);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    rc = check_ptrs({T, dT, dH});
    if (rc != BIRKHOFF_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 4)
        hipLaunchKernelGGL((birk::implicit_bwd_from_T_kernel<4>), grid_for(B, 4), dim3(kBlock), 0, s, T, dT, dH, B);
    else
        hipLaunchKernelGGL((birk::implicit_bwd_from_T_kernel<8>), grid_for(B, 8), dim3(kBlock), 0, s, T, dT, dH, B);
    return launched();
}

int birkhoff_fwd_bwd(const float* logits, const float* dT, float* T, float* dual, float* dH, int64_t B, int n,
                     float tol, int max_iter, void* stream) {
    return fused_entry<float>(logits, dT, T, dual, dH, B, n, tol, max_iter, stream);
}

int birkhoff_fwd_bwd_bf16(const uint16_t* logits, const uint16_t* dT, uint16_t* T, float* dual, uint16_t* dH,
                          int64_t B, int n, float tol, int max_iter, void* stream) {
    return fused_entry<uint16_t>(logits, dT, T, dual, dH, B, n, tol, max_iter, stream);
}

const char* birkhoff_strerror(int code) {
    switch (code) {
        case BIRKHOFF_OK: return "success";
        case BIRKHOFF_EINVAL:
            return "invalid argument (NULL pointer with B > 0, B < 0 or too large, n not 4 or 8, tol <= 0 or "
                   "not finite, max_iter < 1 or iters < 1)";
        case BIRKHOFF_EALIGN: return "a pointer is not 16-byte aligned (iters: 4-byte aligned)";
        case BIRKHOFF_ELAUNCH: return "the HIP runtime reported an error when launching the kernel";
        default: return "unknown birkhoff error code";
    }
}

int birkhoff_abi_version(void) { return 1; }

}  // extern "C"
