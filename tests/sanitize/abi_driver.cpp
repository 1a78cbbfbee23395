// Host driver for a sanitizer build (address and undefined-behaviour) of the
// C ABI's argument validation, birkhoff_projection_amd/csrc/abi_checks.hpp,
// compiled by the host compiler without HIP: each validator is called at the
// edges of its ranges -- batch sizes at and beyond the limits, INT64_MAX, NaN
// and infinite tolerances, NULL and misaligned pointers, empty batches with
// NULL pointers, the size products of the fused mixing near overflow -- and
// its return code is compared with the documented one.  Exits non-zero on a
// wrong code; the sanitizers abort on any undefined operation.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "abi_checks.hpp"

using namespace birk::abi;

static int failures = 0;

static void expect(int got, int want, const char* what) {
    if (got != want) {
        std::fprintf(stderr, "FAIL %s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

int main() {
    alignas(16) static float buf[64];
    const float* p = buf;
    const float* q = buf + 4;   // 16-byte aligned
    const float* mis = buf + 1; // 4-byte aligned only
    const int32_t* it = reinterpret_cast<const int32_t*>(buf + 8);
    const int32_t* it_mis = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(buf) + 2);
    const int64_t big = std::numeric_limits<int64_t>::max();
    const float nan = std::numeric_limits<float>::quiet_NaN(), inf = std::numeric_limits<float>::infinity();

    // forward
    expect(validate_fwd(p, q, p, nullptr, nullptr, false, 5, 4, 1e-6f, 50), BIRKHOFF_OK, "fwd ok");
    expect(validate_fwd(p, q, p, nullptr, nullptr, false, kMaxBatch, 8, 1e-6f, 50), BIRKHOFF_OK, "fwd max B");
    expect(validate_fwd(p, q, p, nullptr, nullptr, false, kMaxBatch + 1, 4, 1e-6f, 50), BIRKHOFF_EINVAL, "fwd B+1");
    expect(validate_fwd(p, q, p, nullptr, nullptr, false, big, 4, 1e-6f, 50), BIRKHOFF_EINVAL, "fwd INT64_MAX");
    expect(validate_fwd(p, q, p, nullptr, nullptr, false, -1, 4, 1e-6f, 50), BIRKHOFF_EINVAL, "fwd B<0");
    for (int n : {0, 3, 5, 16, -4}) expect(validate_fwd(p, q, p, nullptr, nullptr, false, 5, n, 1e-6f, 50),
                                          BIRKHOFF_EINVAL, "fwd n");
    for (float tol : {0.0f, -1e-6f, nan, inf, -inf}) expect(validate_fwd(p, q, p, nullptr, nullptr, false, 5, 4, tol, 50),
                                                            BIRKHOFF_EINVAL, "fwd tol");
    expect(validate_fwd(p, q, p, nullptr, nullptr, false, 5, 4, 1e-6f, 0), BIRKHOFF_EINVAL, "fwd max_iter 0");
    expect(validate_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, false, 0, 4, 1e-6f, 50), BIRKHOFF_OK, "fwd empty");
    expect(validate_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, false, 0, 4, nan, 50), BIRKHOFF_EINVAL,
           "fwd empty bad tol");
    expect(validate_fwd(p, nullptr, p, nullptr, nullptr, false, 5, 4, 1e-6f, 50), BIRKHOFF_EINVAL, "fwd NULL T");
    expect(validate_fwd(p, mis, p, nullptr, nullptr, false, 5, 4, 1e-6f, 50), BIRKHOFF_EALIGN, "fwd misaligned T");
    expect(validate_fwd(p, mis, nullptr, nullptr, nullptr, false, 5, 4, 1e-6f, 50), BIRKHOFF_EINVAL,
           "fwd NULL before misaligned");
    expect(validate_fwd(p, q, p, nullptr, nullptr, true, 5, 4, 1e-6f, 50), BIRKHOFF_EINVAL, "fwd_ex NULL iters");
    expect(validate_fwd(p, q, p, it, nullptr, true, 5, 4, 1e-6f, 50), BIRKHOFF_OK, "fwd_ex no fallbacks");
    expect(validate_fwd(p, q, p, it, it, true, 5, 4, 1e-6f, 50), BIRKHOFF_OK, "fwd_ex fallbacks");
    expect(validate_fwd(p, q, p, it_mis, nullptr, true, 5, 4, 1e-6f, 50), BIRKHOFF_EALIGN, "fwd_ex iters align");
    expect(validate_fwd(p, q, p, it, it_mis, true, 5, 4, 1e-6f, 50), BIRKHOFF_EALIGN, "fwd_ex fallbacks align");

    // backward, backward from T, Sinkhorn, fused
    expect(validate_bwd(p, p, q, q, 5, 8), BIRKHOFF_OK, "bwd ok");
    expect(validate_bwd(p, p, q, nullptr, 5, 8), BIRKHOFF_EINVAL, "bwd NULL dH");
    expect(validate_bwd(p, p, q, mis, 5, 8), BIRKHOFF_EALIGN, "bwd misaligned");
    expect(validate_bwd(nullptr, nullptr, nullptr, nullptr, 0, 8), BIRKHOFF_OK, "bwd empty");
    expect(validate_bwd(p, p, q, q, big, 4), BIRKHOFF_EINVAL, "bwd INT64_MAX");
    expect(validate_bwd_from_T(p, q, q, 5, 4), BIRKHOFF_OK, "bwd_from_T ok");
    expect(validate_bwd_from_T(p, q, mis, 5, 4), BIRKHOFF_EALIGN, "bwd_from_T misaligned");
    expect(validate_bwd_from_T(p, q, q, 5, 6), BIRKHOFF_EINVAL, "bwd_from_T n");
    expect(validate_sinkhorn(p, q, 5, 4, 20), BIRKHOFF_OK, "sinkhorn ok");
    expect(validate_sinkhorn(p, q, 5, 4, 0), BIRKHOFF_EINVAL, "sinkhorn iters 0");
    expect(validate_sinkhorn(nullptr, nullptr, 0, 4, 0), BIRKHOFF_EINVAL, "sinkhorn empty bad iters");
    expect(validate_fused(p, q, p, p, q, 5, 4, 1e-6f, 50), BIRKHOFF_OK, "fused ok");
    expect(validate_fused(p, q, p, mis, q, 5, 4, 1e-6f, 50), BIRKHOFF_EALIGN, "fused misaligned dual");
    expect(validate_fused(p, q, p, p, q, kMaxBatch + 1, 8, 1e-6f, 50), BIRKHOFF_EINVAL, "fused B+1");

    // entropic OT
    expect(validate_eot_fwd(p, p, p, 0, q, q, nullptr, 5, 3, 5, 0.5f, 1e-6f, 50), BIRKHOFF_OK, "eot ok");
    expect(validate_eot_fwd(p, mis, mis, 1, q, q, it, 5, 3, 5, 0.5f, 1e-6f, 50), BIRKHOFF_OK, "eot shared 4B");
    expect(validate_eot_fwd(p, mis, p, 0, q, q, nullptr, 5, 3, 5, 0.5f, 1e-6f, 50), BIRKHOFF_EALIGN, "eot a align");
    expect(validate_eot_fwd(p, p, p, 0, q, q, it_mis, 5, 3, 5, 0.5f, 1e-6f, 50), BIRKHOFF_EALIGN, "eot iters align");
    expect(validate_eot_fwd(p, p, p, 0, q, q, nullptr, kMaxEotBatch + 1, 3, 5, 0.5f, 1e-6f, 50), BIRKHOFF_EINVAL,
           "eot B+1");
    expect(validate_eot_fwd(p, p, p, 0, q, q, nullptr, big, 3, 5, 0.5f, 1e-6f, 50), BIRKHOFF_EINVAL, "eot INT64_MAX");
    for (int n : {0, 9}) expect(validate_eot_fwd(p, p, p, 0, q, q, nullptr, 5, n, 5, 0.5f, 1e-6f, 50),
                                BIRKHOFF_EINVAL, "eot n");
    for (int m : {1, 9}) expect(validate_eot_fwd(p, p, p, 0, q, q, nullptr, 5, 3, m, 0.5f, 1e-6f, 50),
                                BIRKHOFF_EINVAL, "eot m");
    for (float eta : {0.0f, -1.0f, nan, inf}) expect(validate_eot_fwd(p, p, p, 0, q, q, nullptr, 5, 3, 5, eta, 1e-6f, 50),
                                                     BIRKHOFF_EINVAL, "eot eta");
    expect(validate_eot_fwd(nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, 0, 1, 2, 1.0f, 1e-6f, 50),
           BIRKHOFF_OK, "eot empty");
    expect(validate_eot_bwd(p, q, p, 0, q, 5, 8, 8, 1.0f), BIRKHOFF_OK, "eot bwd ok");
    expect(validate_eot_bwd(p, q, nullptr, 0, q, 5, 8, 8, 1.0f), BIRKHOFF_EINVAL, "eot bwd NULL a");
    expect(validate_eot_bwd(p, q, p, 0, q, 5, 8, 8, nan), BIRKHOFF_EINVAL, "eot bwd eta");

    // the projection fused with the residual mixing
    expect(validate_mix_fwd(p, q, p, p, q, 5, 4, 64, 4, 1e-6f, 50), BIRKHOFF_OK, "mix ok");
    expect(validate_mix_fwd(p, nullptr, p, p, nullptr, 5, 4, 0, 4, 1e-6f, 50), BIRKHOFF_OK, "mix C=0");
    expect(validate_mix_fwd(p, q, p, p, q, 5, 4, 6, 4, 1e-6f, 50), BIRKHOFF_EINVAL, "mix C not a multiple");
    expect(validate_mix_fwd(p, q, p, p, q, 5, 8, 64, 4, 1e-6f, 50), BIRKHOFF_EINVAL, "mix n");
    expect(validate_mix_fwd(p, q, p, p, q, 5, 4, kMaxMixC + 4, 4, 1e-6f, 50), BIRKHOFF_EINVAL, "mix C max");
    expect(validate_mix_fwd(p, q, p, p, q, kMaxMixTokens + 1, 4, 64, 4, 1e-6f, 50), BIRKHOFF_EINVAL, "mix B+1");
    expect(validate_mix_fwd(p, q, p, p, q, big, 4, kMaxMixC, 4, 1e-6f, 50), BIRKHOFF_EINVAL, "mix INT64_MAX");
    // B * 4 * C just above and at the element limit (2^60)
    expect(validate_mix_fwd(p, q, p, p, q, ((int64_t)1 << 32) + 1, 4, (int64_t)1 << 26, 4, 1e-6f, 50),
           BIRKHOFF_EINVAL, "mix elements above");
    expect(validate_mix_fwd(p, q, p, p, q, (int64_t)1 << 32, 4, (int64_t)1 << 26, 4, 1e-6f, 50), BIRKHOFF_OK,
           "mix elements at");
    expect(validate_mix_fwd(p, mis, p, p, q, 5, 4, 64, 4, 1e-6f, 50), BIRKHOFF_EALIGN, "mix x align");
    expect(validate_mix_bwd(p, q, q, q, p, 5, 4, 64, 8), BIRKHOFF_OK, "mix bwd ok");
    expect(validate_mix_bwd(p, q, q, q, p, 5, 4, 12, 8), BIRKHOFF_EINVAL, "mix bwd bf16 chunk");
    expect(validate_mix_bwd(p, nullptr, nullptr, nullptr, p, 5, 4, 0, 8), BIRKHOFF_OK, "mix bwd C=0");
    expect(validate_mix_bwd(p, q, q, nullptr, p, 5, 4, 64, 8), BIRKHOFF_EINVAL, "mix bwd NULL dx");

    if (failures) return 1;
    std::puts("abi driver: ok");
    return 0;
}
