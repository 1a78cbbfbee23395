// device_math.hpp -- scalar helpers for the per-lane projection kernels (gfx950).
//
// Transcendentals map to single hardware instructions: v_exp_f32 (2^x),
// v_log_f32 (log2 x), v_rcp_f32 (1/x), v_rsq_f32.  Each is accurate to about
// one ulp, which is well inside the 1e-5 forward tolerance; nothing here
// reproduces a vendor math library.  expm1 and log1p for small arguments use
// their Taylor series (textbook), so that differences of log-sum-exp values
// near the optimum keep their relative accuracy in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace birk {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float rsq(float x) { return __builtin_amdgcn_rsqf(x); }

// e^x - 1 with relative accuracy for small |x|: degree-8 Taylor polynomial on
// |x| < 1/2 (truncation below 2e-8 relative), e^x - 1 elsewhere (no cancellation
// there: |e^x - 1| > 0.39).  `ex` must be e^x.
__device__ __forceinline__ float expm1_from(float x, float ex) {
    float p = fmaf(x, 1.0f / 40320.0f, 1.0f / 5040.0f);
    p = fmaf(x, p, 1.0f / 720.0f);
    p = fmaf(x, p, 1.0f / 120.0f);
    p = fmaf(x, p, 1.0f / 24.0f);
    p = fmaf(x, p, 1.0f / 6.0f);
    p = fmaf(x, p, 0.5f);
    float small = fmaf(x * x, p, x);
    return fabsf(x) < 0.5f ? small : ex - 1.0f;
}

// log(1 + s) with relative accuracy for small |s|: Taylor series on |s| < 1/16
// (truncation below 1e-9 relative), log2(1 + s) * ln 2 elsewhere.
__device__ __forceinline__ float log1p_acc(float s) {
    float p = fmaf(s, -1.0f / 8.0f, 1.0f / 7.0f);
    p = fmaf(s, p, -1.0f / 6.0f);
    p = fmaf(s, p, 1.0f / 5.0f);
    p = fmaf(s, p, -1.0f / 4.0f);
    p = fmaf(s, p, 1.0f / 3.0f);
    p = fmaf(s, p, -0.5f);
    float small = fmaf(s * s, p, s);
    return fabsf(s) < 0.0625f ? small : lg2(1.0f + s) * kLn2;
}

// ---- storage types -------------------------------------------------------

// bf16 <-> fp32.  Decoding is exact; encoding rounds to nearest, ties to even,
// and keeps NaN a (quiet) NaN.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return (x != x) ? 0x7FC0u : r;
}

// Load / store K consecutive elements of a lane's own matrix (K a multiple of 8),
// as 16-byte vector accesses.
template <typename IO>
struct Storage;

template <>
struct Storage<float> {
    template <int K>
    __device__ __forceinline__ static void load(const float* __restrict__ p, float (&v)[K]) {
        const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
        for (int k = 0; k < K / 4; ++k) {
            float4 t = q[k];
            v[4 * k + 0] = t.x;
            v[4 * k + 1] = t.y;
            v[4 * k + 2] = t.z;
            v[4 * k + 3] = t.w;
        }
    }
    template <int K>
    __device__ __forceinline__ static void store(float* __restrict__ p, const float (&v)[K]) {
        float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
        for (int k = 0; k < K / 4; ++k) q[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    }
};

template <>
struct Storage<uint16_t> {
    template <int K>
    __device__ __forceinline__ static void load(const uint16_t* __restrict__ p, float (&v)[K]) {
        const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int k = 0; k < K / 8; ++k) {
            uint4 t = q[k];
            uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[8 * k + 2 * h + 0] = bf16_to_f32(w[h] & 0xFFFFu);
                v[8 * k + 2 * h + 1] = bf16_to_f32(w[h] >> 16);
            }
        }
    }
    template <int K>
    __device__ __forceinline__ static void store(uint16_t* __restrict__ p, const float (&v)[K]) {
        uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
        for (int k = 0; k < K / 8; ++k) {
            uint32_t w[4];
#pragma unroll
            for (int h = 0; h < 4; ++h)
                w[h] = f32_to_bf16(v[8 * k + 2 * h]) | (f32_to_bf16(v[8 * k + 2 * h + 1]) << 16);
            q[k] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
};

}  // namespace birk
