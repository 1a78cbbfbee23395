// clock_probe.hip -- the engine clock at which kernels actually run.
//
// A measurement aid, not part of the projection: the driver's reported clock
// is a sampled figure that can lag the load by a long way, while the VALU-bound
// kernels' times scale with the clock they get.  Each workgroup's first wave
// counts shader-clock cycles (s_memtime) against the constant-rate counter
// (s_memrealtime) over `ticks` of the latter; the caller divides the sums and
// multiplies by the constant counter's rate.  Enqueued right behind a timed
// region on the same stream, it reads the clock the region ended on.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "birkhoff.h"
#include "launch.hpp"

namespace {

constexpr int kProbeThreads = 64;
constexpr int kProbeMaxBlocks = 1 << 16;
constexpr int kProbeMaxTicks = 1 << 20;   // about 10 ms at 100 MHz

__global__ void __launch_bounds__(kProbeThreads) clock_probe_kernel(uint64_t* __restrict__ counts, uint32_t ticks) {
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    uint64_t r1 = r0;
    // ends after `ticks` of the constant counter, and in any case after 2^22 reads
    for (uint32_t i = 0; i < (1u << 22) && r1 - r0 < ticks; ++i) r1 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) {
        counts[2 * blockIdx.x] = c1 - c0;
        counts[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" {

int birkhoff_clock_probe(uint64_t* counts, int blocks, int ticks, int* wall_khz, void* stream) {
    if (counts == nullptr || wall_khz == nullptr || blocks < 1 || blocks > kProbeMaxBlocks || ticks < 1 ||
        ticks > kProbeMaxTicks)
        return BIRKHOFF_EINVAL;
    if (reinterpret_cast<uintptr_t>(counts) % 16 != 0) return BIRKHOFF_EALIGN;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        return BIRKHOFF_ELAUNCH;
    *wall_khz = khz;
    return birk::launch(clock_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads),
                        static_cast<hipStream_t>(stream), counts, (uint32_t)ticks);
}

}  // extern "C"
