// birkhoff.hip -- the C ABI of libbirkhoff (declared in include/birkhoff.h):
// dispatch on n and storage type, and launch.
//
// Every argument is checked (abi_checks.hpp) before any HIP call, so a
// rejected call enqueues nothing and never touches the device.  Launches are
// asynchronous on the caller's stream and report their own status
// (launch.hpp); the library allocates nothing and keeps no state.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "abi_checks.hpp"
#include "birkhoff.h"
#include "launch.hpp"
#include "projection.hpp"

namespace {

using birk::kBlock;
using birk::launch;

static_assert(birk::abi::kProjLanesPerGroup == kBlock && birk::Split<8>::R == 2 && birk::Split<4>::R == 1,
              "the batch limit assumes the kernels' geometry");

dim3 grid_for(int64_t B, int n) {
    const int64_t lanes = B * (n == 8 ? birk::Split<8>::R : birk::Split<4>::R);
    return dim3((unsigned)((lanes + kBlock - 1) / kBlock));
}

template <int N, typename IO>
int fwd_launch(const IO* logits, IO* T, float* dual, int32_t* iters, int32_t* fallbacks, int64_t B, float tol,
               int max_iter, hipStream_t s) {
    const dim3 g = grid_for(B, N), blk(kBlock);
    if constexpr (N == 4) {
        if (iters)
            return launch(birk::newton_fwd_gather_kernel<IO, true>, g, blk, s, logits, T, dual, iters, fallbacks, B,
                          tol, max_iter);
        return launch(birk::newton_fwd_gather_kernel<IO, false>, g, blk, s, logits, T, dual, iters, fallbacks, B, tol,
                      max_iter);
    } else {
        if (iters)
            return launch(birk::newton_fwd_kernel<N, IO, true>, g, blk, s, logits, T, dual, iters, fallbacks, B, tol,
                          max_iter);
        return launch(birk::newton_fwd_kernel<N, IO, false>, g, blk, s, logits, T, dual, iters, fallbacks, B, tol,
                      max_iter);
    }
}

template <typename IO>
int fwd_entry(const IO* logits, IO* T, float* dual, int32_t* iters, int32_t* fallbacks, bool need_iters, int64_t B,
              int n, float tol, int max_iter, void* stream) {
    const int rc = birk::abi::validate_fwd(logits, T, dual, iters, fallbacks, need_iters, B, n, tol, max_iter);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return n == 4 ? fwd_launch<4, IO>(logits, T, dual, iters, fallbacks, B, tol, max_iter, s)
                  : fwd_launch<8, IO>(logits, T, dual, iters, fallbacks, B, tol, max_iter, s);
}

template <typename IO>
int bwd_entry(const IO* logits, const float* dual, const IO* dT, IO* dH, int64_t B, int n, void* stream) {
    const int rc = birk::abi::validate_bwd(logits, dual, dT, dH, B, n);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 4) return launch(birk::implicit_bwd_kernel<4, IO>, grid_for(B, 4), dim3(kBlock), s, logits, dual, dT, dH, B);
    return launch(birk::implicit_bwd_kernel<8, IO>, grid_for(B, 8), dim3(kBlock), s, logits, dual, dT, dH, B);
}

template <typename IO>
int fused_entry(const IO* logits, const IO* dT, IO* T, float* dual, IO* dH, int64_t B, int n, float tol,
                int max_iter, void* stream) {
    const int rc = birk::abi::validate_fused(logits, dT, T, dual, dH, B, n, tol, max_iter);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 4)
        return launch(birk::fused_fwd_bwd_kernel<4, IO>, grid_for(B, 4), dim3(kBlock), s, logits, dT, T, dual, dH, B,
                      tol, max_iter);
    return launch(birk::fused_fwd_bwd_kernel<8, IO>, grid_for(B, 8), dim3(kBlock), s, logits, dT, T, dual, dH, B, tol,
                  max_iter);
}

}  // namespace

extern "C" {

int birkhoff_fwd(const float* logits, float* T, float* dual, int64_t B, int n, float tol, int max_iter,
                 void* stream) {
    return fwd_entry<float>(logits, T, dual, nullptr, nullptr, false, B, n, tol, max_iter, stream);
}

int birkhoff_fwd_ex(const float* logits, float* T, float* dual, int32_t* iters, int32_t* fallbacks, int64_t B, int n,
                    float tol, int max_iter, void* stream) {
    return fwd_entry<float>(logits, T, dual, iters, fallbacks, true, B, n, tol, max_iter, stream);
}

int birkhoff_bwd(const float* logits, const float* dual, const float* dT, float* dH, int64_t B, int n,
                 void* stream) {
    return bwd_entry<float>(logits, dual, dT, dH, B, n, stream);
}

int sinkhorn_fwd(const float* logits, float* T, int64_t B, int n, int iters, void* stream) {
    const int rc = birk::abi::validate_sinkhorn(logits, T, B, n, iters);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 4) return launch(birk::sinkhorn_kernel<4, float>, grid_for(B, 4), dim3(kBlock), s, logits, T, B, iters);
    return launch(birk::sinkhorn_kernel<8, float>, grid_for(B, 8), dim3(kBlock), s, logits, T, B, iters);
}

int birkhoff_fwd_bf16(const uint16_t* logits, uint16_t* T, float* dual, int64_t B, int n, float tol, int max_iter,
                      void* stream) {
    return fwd_entry<uint16_t>(logits, T, dual, nullptr, nullptr, false, B, n, tol, max_iter, stream);
}

int birkhoff_bwd_bf16(const uint16_t* logits, const float* dual, const uint16_t* dT, uint16_t* dH, int64_t B, int n,
                      void* stream) {
    return bwd_entry<uint16_t>(logits, dual, dT, dH, B, n, stream);
}

int birkhoff_bwd_from_T(const float* T, const float* dT, float* dH, int64_t B, int n, void* stream) {
    const int rc = birk::abi::validate_bwd_from_T(T, dT, dH, B, n);
    if (rc != BIRKHOFF_OK || B == 0) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (n == 4) return launch(birk::implicit_bwd_from_T_kernel<4>, grid_for(B, 4), dim3(kBlock), s, T, dT, dH, B);
    return launch(birk::implicit_bwd_from_T_kernel<8>, grid_for(B, 8), dim3(kBlock), s, T, dT, dH, B);
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
        case BIRKHOFF_EALIGN: return "a pointer is not 16-byte aligned (iters, fallbacks: 4-byte aligned)";
        case BIRKHOFF_ELAUNCH: return "the HIP runtime rejected the kernel launch";
        default: return "unknown birkhoff error code";
    }
}

int birkhoff_abi_version(void) { return 2; }

}  // extern "C"
