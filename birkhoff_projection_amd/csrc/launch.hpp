// launch.hpp -- kernel launch for the C ABI entry points.
//
// hipLaunchKernel returns the launch's own status, so a call reports
// BIRKHOFF_ELAUNCH exactly when its own launch failed: an error left by an
// earlier, unrelated HIP call on the thread is neither taken for this call's
// failure nor consumed (hipGetLastError after the launch would do both).  As
// for any failed HIP call, a failed launch also leaves its error in the
// thread's last-error state.
#pragma once

#include <hip/hip_runtime.h>

#include "birkhoff.h"

namespace birk {

template <typename... P>
int launch_args(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, P... args) {
    void* argv[] = {static_cast<void*>(&args)...};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
    return e == hipSuccess ? BIRKHOFF_OK : BIRKHOFF_ELAUNCH;
}

// Launches `kernel` on `grid` x `block` on `stream` with the arguments converted
// to the kernel's parameter types; returns BIRKHOFF_OK or BIRKHOFF_ELAUNCH.
template <typename... P, typename... A>
int launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A... args) {
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    return launch_args<P...>(kernel, grid, block, stream, static_cast<P>(args)...);
}

}  // namespace birk
