// eot_launch.hpp -- launch helpers for the general entropic-OT kernels, shared
// by eot.hip (the C ABI) and the eot_rows_*.hip units that instantiate the
// kernels for a few row counts each (so that the shapes compile in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "eot.hpp"

namespace birk {
namespace eot {

template <int N, int M>
dim3 grid_for(int64_t B) {
    const int64_t t = Waves<N * M>::threads;
    return dim3((unsigned)((B + t - 1) / t));
}

struct FwdArgs {
    const float *cost, *a, *b;
    int shared;
    float *T, *dual;
    int32_t* iters;
    int64_t B;
    float eta, tol;
    int max_iter;
    hipStream_t s;
};

struct BwdArgs {
    const float *T, *G, *a;
    int shared;
    float* D;
    int64_t B;
    float eta;
    hipStream_t s;
};

template <int N, int M>
void launch(const FwdArgs& x) {
    const dim3 g = grid_for<N, M>(x.B), blk(Waves<N * M>::threads);
    if (x.iters)
        hipLaunchKernelGGL((birk::eot::eot_fwd_kernel<N, M, true>), g, blk, 0, x.s, x.cost, x.a, x.b, x.shared, x.T,
                           x.dual, x.iters, x.B, x.eta, x.tol, x.max_iter);
    else
        hipLaunchKernelGGL((birk::eot::eot_fwd_kernel<N, M, false>), g, blk, 0, x.s, x.cost, x.a, x.b, x.shared, x.T,
                           x.dual, x.iters, x.B, x.eta, x.tol, x.max_iter);
}

template <int N, int M>
void launch(const BwdArgs& x) {
    const dim3 g = grid_for<N, M>(x.B), blk(Waves<N * M>::threads);
    hipLaunchKernelGGL((birk::eot::eot_bwd_kernel<N, M>), g, blk, 0, x.s, x.T, x.G, x.a, x.shared, x.D, x.B, x.eta);
}

// launches the kernel for n = N rows and m columns, m in [2, 8]
template <int N, typename Args>
void by_m(int m, const Args& x) {
    switch (m) {
        case 2: launch<N, 2>(x); break;
        case 3: launch<N, 3>(x); break;
        case 4: launch<N, 4>(x); break;
        case 5: launch<N, 5>(x); break;
        case 6: launch<N, 6>(x); break;
        case 7: launch<N, 7>(x); break;
        default: launch<N, 8>(x); break;
    }
}

// each instantiated in one of the eot_rows_*.hip units
#define BIRK_EOT_ROWS(N)                                   \
    extern template void by_m<N, FwdArgs>(int, const FwdArgs&); \
    extern template void by_m<N, BwdArgs>(int, const BwdArgs&);
BIRK_EOT_ROWS(1)
BIRK_EOT_ROWS(2)
BIRK_EOT_ROWS(3)
BIRK_EOT_ROWS(4)
BIRK_EOT_ROWS(5)
BIRK_EOT_ROWS(6)
BIRK_EOT_ROWS(7)
BIRK_EOT_ROWS(8)
#undef BIRK_EOT_ROWS

}  // namespace eot
}  // namespace birk
