// eot_launch.hpp -- launch helpers for the general entropic-OT kernels, shared
// by eot.hip (the C ABI) and the eot_rows_*.hip units that instantiate the
// kernels for a few row counts each (so that the shapes compile in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "eot.hpp"
#include "launch.hpp"

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
int launch_shape(const FwdArgs& x) {
    const dim3 g = grid_for<N, M>(x.B), blk(Waves<N * M>::threads);
    if (x.iters)
        return birk::launch(eot_fwd_kernel<N, M, true>, g, blk, x.s, x.cost, x.a, x.b, x.shared, x.T, x.dual,
                            x.iters, x.B, x.eta, x.tol, x.max_iter);
    return birk::launch(eot_fwd_kernel<N, M, false>, g, blk, x.s, x.cost, x.a, x.b, x.shared, x.T, x.dual, x.iters,
                        x.B, x.eta, x.tol, x.max_iter);
}

template <int N, int M>
int launch_shape(const BwdArgs& x) {
    const dim3 g = grid_for<N, M>(x.B), blk(Waves<N * M>::threads);
    return birk::launch(eot_bwd_kernel<N, M>, g, blk, x.s, x.T, x.G, x.a, x.shared, x.D, x.B, x.eta);
}

// launches the kernel for n = N rows and m columns, m in [2, 8]; returns
// BIRKHOFF_OK or BIRKHOFF_ELAUNCH
template <int N, typename Args>
int by_m(int m, const Args& x) {
    switch (m) {
        case 2: return launch_shape<N, 2>(x);
        case 3: return launch_shape<N, 3>(x);
        case 4: return launch_shape<N, 4>(x);
        case 5: return launch_shape<N, 5>(x);
        case 6: return launch_shape<N, 6>(x);
        case 7: return launch_shape<N, 7>(x);
        default: return launch_shape<N, 8>(x);
    }
}

// each instantiated in one of the eot_rows_*.hip units
#define BIRK_EOT_ROWS(N)                                   \
    extern template int by_m<N, FwdArgs>(int, const FwdArgs&); \
    extern template int by_m<N, BwdArgs>(int, const BwdArgs&);
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
