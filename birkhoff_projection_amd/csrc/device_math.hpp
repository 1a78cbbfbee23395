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

// e^x - 1 with relative accuracy for small |x|: degree-5 Taylor polynomial on
// |x| < 1/16 (truncation below 1.4e-9 relative, far below fp32's 6e-8),
// e^x - 1 elsewhere (there the relative rounding error stays below 1.2e-6, and
// it only enters through quantities that are not close to cancelling).  `ex`
// must be e^x.
__device__ __forceinline__ float expm1_from(float x, float ex) {
    float p = fmaf(x, 1.0f / 120.0f, 1.0f / 24.0f);
    p = fmaf(x, p, 1.0f / 6.0f);
    p = fmaf(x, p, 0.5f);
    const float small = fmaf(x * x, p, x);
    return fabsf(x) < 0.0625f ? small : ex - 1.0f;
}

// log(1 + s) for |s| < 1/16 by its Taylor series to degree 6 (truncation below
// 1e-8 relative, far below fp32's 6e-8); keeps full relative accuracy as s -> 0.
__device__ __forceinline__ float log1p_series(float s) {
    float p = fmaf(s, -1.0f / 6.0f, 1.0f / 5.0f);
    p = fmaf(s, p, -1.0f / 4.0f);
    p = fmaf(s, p, 1.0f / 3.0f);
    p = fmaf(s, p, -0.5f);
    return fmaf(s * s, p, s);
}

// ---- storage types -------------------------------------------------------

// bf16 <-> fp32.  Decoding is exact.  Encoding is gfx950's v_cvt_pk_bf16_f32,
// two values per instruction, rounding to nearest, ties to even (denormals
// included); NaN stays a quiet NaN.  Measured on the device against the
// bit-level definition (add 0x7FFF plus the kept lsb, shift) over 2^22 random
// patterns, every low-bit pattern of the smallest denormals and the tie,
// overflow and infinity cases: identical except for NaN payloads.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// lo in bits 0..15, hi in bits 16..31
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Decode / encode one matrix between its storage chunks (16-byte words, as
// loaded from memory) and fp32 registers.  K elements, K * sizeof(IO) a
// multiple of 16.
template <typename IO>
struct Storage;

template <>
struct Storage<float> {
    template <int K>
    __device__ __forceinline__ static void decode(const uint4 (&w)[K / 4], float (&v)[K]) {
#pragma unroll
        for (int k = 0; k < K / 4; ++k) {
            v[4 * k + 0] = __uint_as_float(w[k].x);
            v[4 * k + 1] = __uint_as_float(w[k].y);
            v[4 * k + 2] = __uint_as_float(w[k].z);
            v[4 * k + 3] = __uint_as_float(w[k].w);
        }
    }
    template <int K>
    __device__ __forceinline__ static void encode(const float (&v)[K], uint4 (&w)[K / 4]) {
#pragma unroll
        for (int k = 0; k < K / 4; ++k)
            w[k] = make_uint4(__float_as_uint(v[4 * k]), __float_as_uint(v[4 * k + 1]),
                              __float_as_uint(v[4 * k + 2]), __float_as_uint(v[4 * k + 3]));
    }
};

template <>
struct Storage<uint16_t> {
    template <int K>
    __device__ __forceinline__ static void decode(const uint4 (&w)[K / 8], float (&v)[K]) {
#pragma unroll
        for (int k = 0; k < K / 8; ++k) {
            const uint32_t u[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[8 * k + 2 * h + 0] = bf16_to_f32(u[h] & 0xFFFFu);
                v[8 * k + 2 * h + 1] = bf16_to_f32(u[h] >> 16);
            }
        }
    }
    template <int K>
    __device__ __forceinline__ static void encode(const float (&v)[K], uint4 (&w)[K / 8]) {
#pragma unroll
        for (int k = 0; k < K / 8; ++k) {
            uint32_t u[4];
#pragma unroll
            for (int h = 0; h < 4; ++h)
                u[h] = pack_bf16x2(v[8 * k + 2 * h], v[8 * k + 2 * h + 1]);
            w[k] = make_uint4(u[0], u[1], u[2], u[3]);
        }
    }
};

// ---- streaming global accesses -------------------------------------------
//
// Every byte of a batch is read or written exactly once per launch, so matrix
// and dual traffic uses non-temporal 16-byte accesses (the caches do not keep
// lines that will not be touched again).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 stream_load(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void stream_store(uint4* p, const uint4& v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

// A copy of v that the compiler cannot see through (an empty asm statement that
// claims to modify the register; no instruction is emitted): addresses derived
// from it are recomputed where they are used, a few instructions, instead of
// being kept live -- or spilled -- across a long iteration between the load
// and the store of a tile.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// ---- movement of one matrix per lane between HBM and registers ------------
//
// A wave owns 64 consecutive matrices, one per lane, each C 16-byte chunks long
// and stored back to back.
//
// Items of up to 128 bytes (C <= 8): loading them lane by lane would make
// every load instruction touch 64 scattered 16-byte pieces of a
// 64*C*16-byte span (64 distinct cache lines per instruction, each visited
// C times), which starves the address path.  Instead the wave reads (and
// writes) the span with fully coalesced 16-byte accesses -- chunk
// c = k*64 + lane in instruction k -- and swaps the chunks into their owners'
// registers through a private region of LDS.  Within an item, chunk q sits at
// slot q ^ f(m), f(m) = (m / (16/C)) mod C, so that the 16 lanes of any LDS
// access phase hit 16 different 16-byte bank groups on both sides.  Only the
// issuing wave touches its region, so ordering inside the wave needs no
// workgroup barrier.  (Larger items would be read and written by their owners
// directly; none of the kernels has them.)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int C>
struct WaveTile {
    static_assert(C == 2 || C == 4 || C == 8 || C == 16, "chunks per matrix");
    static constexpr bool kStaged = C <= 8;
    static constexpr int kLdsChunks = kStaged ? 64 * C : 1;   // LDS tile per wave, in 16-byte chunks
    // (unsigned arithmetic: the divisions and remainders by powers of two are
    // shifts and masks, and the chunk offsets k * 64 fold into immediates)
    __device__ __forceinline__ static unsigned slot(unsigned m, unsigned q) {
        return m * C + (q ^ ((m / (16 / C)) & (C - 1)));
    }
    // chunk that a lane handles in access k: coalesced order when staged, its own chunk k otherwise
    __device__ __forceinline__ static unsigned chunk(unsigned k, unsigned lane) {
        return kStaged ? k * 64 + lane : lane * C + k;
    }

    // Issue the global loads of one wave tile.  `src` points at the wave's first
    // matrix; `valid` (wave-uniform, >= 1) chunks exist.  A full tile loads
    // unconditionally; in a partial one, chunks at or beyond `valid` read the
    // last valid chunk instead and are then zeroed.  Either way every load is
    // issued before any is waited for.
    __device__ __forceinline__ static void fetch(const uint4* __restrict__ src, int valid, int lane, uint4 (&t)[C]) {
        if (valid == 64 * C) {
#pragma unroll
            for (int k = 0; k < C; ++k) t[k] = stream_load(src + chunk(k, lane));
        } else {
#pragma unroll
            for (int k = 0; k < C; ++k) {
                const unsigned c = chunk(k, lane);
                t[k] = stream_load(src + (c < (unsigned)valid ? c : (unsigned)valid - 1));
            }
#pragma unroll
            for (int k = 0; k < C; ++k) {
                const bool keep = chunk(k, lane) < (unsigned)valid;
                t[k].x = keep ? t[k].x : 0u;
                t[k].y = keep ? t[k].y : 0u;
                t[k].z = keep ? t[k].z : 0u;
                t[k].w = keep ? t[k].w : 0u;
            }
        }
    }

    // Fetched chunks -> registers of their owners.
    __device__ __forceinline__ static void route(const uint4 (&t)[C], uint4* lds, int lane, uint4 (&own)[C]) {
        if constexpr (kStaged) {
#pragma unroll
            for (int k = 0; k < C; ++k) {
                const unsigned c = chunk(k, lane);
                lds[slot(c / C, c % C)] = t[k];
            }
            wave_lds_sync();
#pragma unroll
            for (int q = 0; q < C; ++q) own[q] = lds[slot(lane, q)];
            wave_lds_sync();
        } else {
#pragma unroll
            for (int q = 0; q < C; ++q) own[q] = t[q];
        }
    }

    __device__ __forceinline__ static void load(const uint4* __restrict__ src, int valid, uint4* lds, int lane,
                                                uint4 (&own)[C]) {
        uint4 t[C];
        fetch(src, valid, lane, t);
        route(t, lds, lane, own);
    }

    // Asynchronous variant of fetch + route for a staged tile whose contents
    // are needed much later: the wave's span is copied from global memory
    // straight into its LDS region (global_load_lds_dwordx4: lane i of access k
    // writes chunk k*64 + i at byte 16*(k*64 + i) of the region, unswizzled),
    // holding no registers while it is in flight.  Chunks at or beyond `valid`
    // repeat the last valid chunk.  The region must not be touched until
    // read_prefetched.
    __device__ __forceinline__ static void prefetch(const uint4* __restrict__ src, int valid, uint4* lds, int lane) {
        static_assert(kStaged, "only staged tiles are prefetched through LDS");
        typedef __attribute__((address_space(3))) uint4 lds_u4;
        typedef __attribute__((address_space(3))) void lds_void;
        lds_u4* base = reinterpret_cast<lds_u4*>(
            __builtin_amdgcn_readfirstlane(static_cast<int>(reinterpret_cast<uintptr_t>(lds))));
        wave_lds_sync();   // earlier reads of the region are complete
#pragma unroll
        for (int k = 0; k < C; ++k) {
            const int c = k * 64 + lane;
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + (c < valid ? c : valid - 1)),
                                             reinterpret_cast<lds_void*>(base + k * 64), 16, 0, 0);
        }
    }

    // Waits for a prefetch and hands each lane its own C chunks.  kPin: the
    // addresses are recomputed from the lane here (opaque) instead of being kept
    // from the load, which kernels near their register limit need; others spend
    // fewer instructions without it.
    template <bool kPin = true>
    __device__ __forceinline__ static void read_prefetched(uint4* lds, int lane, uint4 (&own)[C]) {
        if constexpr (kPin) lane = opaque(lane);
        __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0): the LDS copies have landed
        wave_lds_sync();
#pragma unroll
        for (int q = 0; q < C; ++q) own[q] = lds[lane * C + q];
        wave_lds_sync();
    }

    // As store, but the items whose bit is set in the wave-uniform mask `skip`
    // (bit m = the wave's m-th item) are not written.
    template <bool kPin = true>
    __device__ __forceinline__ static void store_except(const uint4 (&own)[C], uint4* lds, int lane,
                                                        uint4* __restrict__ dst, int valid, uint64_t skip) {
        static_assert(kStaged, "staged tiles only");
        if constexpr (kPin) lane = opaque(lane);
#pragma unroll
        for (int q = 0; q < C; ++q) lds[slot(lane, q)] = own[q];
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < C; ++k) {
            const unsigned c = chunk(k, lane);
            const uint4 v = lds[slot(c / C, c % C)];
            if (c < (unsigned)valid && !((skip >> (c / C)) & 1u)) stream_store(dst + c, v);
        }
        wave_lds_sync();
    }

    // Registers of the owning lane -> global.  `valid` (wave-uniform) chunks
    // exist; the rest are not written.  A full tile stores unconditionally.
    // (kPin as in read_prefetched.)
    template <bool kPin = true>
    __device__ __forceinline__ static void store(const uint4 (&own)[C], uint4* lds, int lane, uint4* __restrict__ dst,
                                                 int valid) {
        if constexpr (kPin) lane = opaque(lane);
        const bool full = valid == 64 * C;
        if constexpr (kStaged) {
#pragma unroll
            for (int q = 0; q < C; ++q) lds[slot(lane, q)] = own[q];
            wave_lds_sync();
            if (full) {
#pragma unroll
                for (int k = 0; k < C; ++k) {
                    const unsigned c = chunk(k, lane);
                    stream_store(dst + c, lds[slot(c / C, c % C)]);
                }
            } else {
#pragma unroll
                for (int k = 0; k < C; ++k) {
                    const unsigned c = chunk(k, lane);
                    const uint4 v = lds[slot(c / C, c % C)];
                    if (c < (unsigned)valid) stream_store(dst + c, v);
                }
            }
            wave_lds_sync();
        } else {
            if (full) {
#pragma unroll
                for (int k = 0; k < C; ++k) stream_store(dst + chunk(k, lane), own[k]);
            } else {
#pragma unroll
                for (int k = 0; k < C; ++k) {
                    const unsigned c = chunk(k, lane);
                    if (c < (unsigned)valid) stream_store(dst + c, own[k]);
                }
            }
        }
    }
};

}  // namespace birk
