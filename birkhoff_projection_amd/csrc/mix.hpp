// mix.hpp -- the consumer of the projection in an mHC layer: the residual-stream
// mixing y = H_res x of the update x_{l+1} = H_res x_l + H_post^T F(H_pre x_l)
// ("Accelerating Birkhoff Projection for Manifold-Constrained Hyper-Connections",
// section 2.1), with H_res the projected 4 x 4 matrix of each token and x the
// token's n x C hidden matrix (n = 4 streams of C features).
//
// Forward (project_mix_kernel): a workgroup takes 4 tokens, one per wave.  Its first wave
// projects their logits exactly as birkhoff_fwd does (one matrix per
// lane) and stores T and the dual; the 4 projections go to LDS, and then all
// four waves stream the tokens' hidden matrices, one token each, through
// y_i = sum_j T_ij x_j (each wave's first loads are issued before the
// projection, so they are in flight while it runs).  T of the token being streamed is wave-uniform and is
// held in scalar registers; every lane owns 16-byte column chunks of the four
// rows, so each access instruction is a coalesced 1 KiB.  The epilogue never
// writes T to HBM and reads it back: the stored T is for the backward.
//
// Backward (mix_bwd_kernel): for upstream dy, dx = T^T dy and
// dT = dy x^T (a reduction over the C columns), then eq (13) turns dT into
// dL/dH.  The four waves stream x and dy and write dx, accumulating each
// token's 16 dT partial sums per lane, which one DPP / readlane reduction per
// entry completes; the 4 dT matrices meet in LDS, and the first wave runs the
// eq (13) backward of implicit_grad for them, one token per lane.
//
// The work is HBM-bound: 8 FMAs per element against 2 (fp32) or 1 (bf16)
// bytes moved per FMA.  No MFMA: the 4 x 4 by 4 x C product per token has
// K = 4, far below any matrix-core tile, and the same bytes bound it either way.
#pragma once

#include "projection.hpp"

namespace birk {
namespace mix {

constexpr int kTokens = 4;     // tokens per workgroup (one per wave): small, so that the grid has many
                               // workgroups and the last round of them is short
constexpr int kUnroll = 4;     // column chunks per lane in flight per row
constexpr int kTs = 17;        // LDS stride of a token's 16 entries (odd: no bank conflicts)

// 16-byte chunks of hidden-state storage <-> fp32
template <typename XT>
struct Vec;

template <>
struct Vec<float> {
    static constexpr int V = 4;
    __device__ __forceinline__ static void decode(const uint4& w, float (&v)[V]) {
        v[0] = __uint_as_float(w.x);
        v[1] = __uint_as_float(w.y);
        v[2] = __uint_as_float(w.z);
        v[3] = __uint_as_float(w.w);
    }
    __device__ __forceinline__ static uint4 encode(const float (&v)[V]) {
        return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    }
};

template <>
struct Vec<uint16_t> {
    static constexpr int V = 8;
    __device__ __forceinline__ static void decode(const uint4& w, float (&v)[V]) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            v[2 * h] = bf16_to_f32(u[h] & 0xFFFFu);
            v[2 * h + 1] = bf16_to_f32(u[h] >> 16);
        }
    }
    __device__ __forceinline__ static uint4 encode(const float (&v)[V]) {
        uint32_t u[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) u[h] = pack_bf16x2(v[2 * h], v[2 * h + 1]);
        return make_uint4(u[0], u[1], u[2], u[3]);
    }
};

__device__ __forceinline__ float uniform(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// sum over the 64 lanes, returned wave-uniform: quad and row DPP exchanges
// leave every lane of each 16-lane row with the row's sum, then the four row
// sums are read out of lanes 0, 16, 32, 48.
__device__ __forceinline__ float wave_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // half-row mirror
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// The loads of one batch of a token's columns: chunks q + 64u (u < kUnroll) of
// its four rows, all issued before any is used.
__device__ __forceinline__ void load_batch(const uint4* __restrict__ xr, int64_t Q, int64_t q,
                                           uint4 (&w)[kUnroll][4]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[u][j] = stream_load(xr + j * Q + q + 64 * u);
}

// y_i = sum_j T_ij x_j for the chunk whose four row pieces are w, stored at
// chunk q of each output row.
template <typename XT>
__device__ __forceinline__ void mix_chunk(const float (&t)[16], const uint4 (&w)[4], uint4* __restrict__ yr,
                                          int64_t Q, int64_t q) {
    using Vx = Vec<XT>;
    constexpr int V = Vx::V;
    float xv[4][V];
#pragma unroll
    for (int j = 0; j < 4; ++j) Vx::decode(w[j], xv[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e)
            o[e] = fmaf(t[4 * i + 3], xv[3][e], fmaf(t[4 * i + 2], xv[2][e],
                        fmaf(t[4 * i + 1], xv[1][e], t[4 * i] * xv[0][e])));
        stream_store(yr + i * Q + q, Vx::encode(o));
    }
}

// y_i = sum_j T_ij x_j for one token: rows of Q 16-byte chunks at xr + j*Q and
// yr + i*Q; lane l handles chunks l, l + 64, ...  T is wave-uniform.  When
// `pre` is set (per lane, only if lane + 64 (kUnroll - 1) < Q), the batch at
// q = lane has already been loaded into w0.
template <typename XT>
__device__ __forceinline__ void mix_token(const float (&t)[16], const uint4* __restrict__ xr, uint4* __restrict__ yr,
                                          int64_t Q, int lane, bool pre, const uint4 (&w0)[kUnroll][4]) {
    int64_t q = lane;
    if (pre) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) mix_chunk<XT>(t, w0[u], yr, Q, q + 64 * u);
        q += 64 * kUnroll;
    }
    for (; q + 64 * (kUnroll - 1) < Q; q += 64 * kUnroll) {
        uint4 w[kUnroll][4];
        load_batch(xr, Q, q, w);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) mix_chunk<XT>(t, w[u], yr, Q, q + 64 * u);
    }
    for (; q < Q; q += 64) {
        uint4 w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = stream_load(xr + j * Q + q);
        mix_chunk<XT>(t, w, yr, Q, q);
    }
}

// Projection of the workgroup's tokens' 4 x 4 logits (first wave) and the mixing of their
// hidden matrices (all waves).  Q = 16-byte chunks per hidden row (C / V).
template <typename XT>
__global__ void __launch_bounds__(kBlock)
project_mix_kernel(const float* __restrict__ logits, const XT* __restrict__ x, float* __restrict__ Tout,
                   float* __restrict__ dual, XT* __restrict__ y, int64_t B, int64_t Q, float tol, int max_iter) {
    using Gm = Geometry<4, float>;
    static_assert(kTokens == kWaves, "one token per wave");
    __shared__ uint4 tile[Gm::Tile::kLdsChunks];
    __shared__ float Ts[kTokens * kTs];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t first = (int64_t)blockIdx.x * kTokens;
    const int64_t left = B - first;
    const int ntok = left >= kTokens ? kTokens : (int)left;
    // this wave's token: its first batch of hidden-state loads is issued now, so
    // that it is in flight while the first wave projects
    const bool mine = wave < ntok;
    const bool pre = mine && lane + 64 * (kUnroll - 1) < Q;   // per lane: every chunk of the batch exists
    const int64_t row0 = (first + wave) * 4 * Q;
    uint4 w0[kUnroll][4];
    if (pre) load_batch(reinterpret_cast<const uint4*>(x) + row0, Q, lane, w0);
    if (wave == 0) {
        const Gm geo(B, first, kTokens);
        float T[16], yv[3], res;
        int sweeps;
        newton_solve<4, float>(geo, tile, logits, tol, max_iter, T, yv, res, sweeps);
        store_forward<4, float>(geo, tile, Tout, dual, T, yv);
        if (lane < kTokens)
#pragma unroll
            for (int k = 0; k < 16; ++k) Ts[lane * kTs + k] = T[k];
    }
    __syncthreads();
    if (mine) {
        float tm[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) tm[k] = uniform(Ts[wave * kTs + k]);
        mix_token<XT>(tm, reinterpret_cast<const uint4*>(x) + row0, reinterpret_cast<uint4*>(y) + row0, Q, lane, pre,
                      w0);
    }
}

// dx = T^T dy for one token, and this lane's share of dT = dy x^T (acc).
template <typename XT>
__device__ __forceinline__ void mix_token_bwd(const float (&t)[16], const uint4* __restrict__ xr,
                                              const uint4* __restrict__ dyr, uint4* __restrict__ dxr, int64_t Q,
                                              int lane, float (&acc)[16]) {
    using Vx = Vec<XT>;
    constexpr int V = Vx::V;
    // element by element (few values live at once): dT partial sums and the
    // four dx outputs of each column of the chunk
    auto chunk = [&](const uint4 (&wx)[4], const uint4 (&wd)[4], int64_t qq) {
        float xv[4][V], dv[4][V], o[4][V];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Vx::decode(wx[j], xv[j]);
            Vx::decode(wd[j], dv[j]);
        }
#pragma unroll
        for (int e = 0; e < V; ++e) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[4 * i + j] = fmaf(dv[i][e], xv[j][e], acc[4 * i + j]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j][e] = fmaf(t[12 + j], dv[3][e], fmaf(t[8 + j], dv[2][e], fmaf(t[4 + j], dv[1][e], t[j] * dv[0][e])));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) stream_store(dxr + j * Q + qq, Vx::encode(o[j]));
    };
    constexpr int U = 1;   // two input streams: 8 chunks in flight per lane
    int64_t q = lane;
    for (; q + 64 * (U - 1) < Q; q += 64 * U) {
        uint4 wx[U][4], wd[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wx[u][j] = stream_load(xr + j * Q + q + 64 * u);
                wd[u][j] = stream_load(dyr + j * Q + q + 64 * u);
            }
#pragma unroll
        for (int u = 0; u < U; ++u) chunk(wx[u], wd[u], q + 64 * u);
    }
    for (; q < Q; q += 64) {
        uint4 wx[4], wd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wx[j] = stream_load(xr + j * Q + q);
            wd[j] = stream_load(dyr + j * Q + q);
        }
        chunk(wx, wd, q);
    }
}

// Backward of the mixing and of the projection: dx = T^T dy, dT = dy x^T, and
// dH = dL/dH by eq (13) from (T, dT).
template <typename XT>
__global__ void __launch_bounds__(kBlock)
mix_bwd_kernel(const float* __restrict__ Tin, const XT* __restrict__ x, const XT* __restrict__ dy,
               XT* __restrict__ dx, float* __restrict__ dH, int64_t B, int64_t Q) {
    __shared__ float dTs[kTokens * kTs];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t first = (int64_t)blockIdx.x * kTokens;
    const int64_t left = B - first;
    const int ntok = left >= kTokens ? kTokens : (int)left;
    for (int t = wave; t < ntok; t += kWaves) {
        const int64_t tok = first + t;
        float tm[16], acc[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            tm[k] = uniform(Tin[tok * 16 + k]);
            acc[k] = 0.0f;
        }
        const int64_t row0 = tok * 4 * Q;
        mix_token_bwd<XT>(tm, reinterpret_cast<const uint4*>(x) + row0, reinterpret_cast<const uint4*>(dy) + row0,
                          reinterpret_cast<uint4*>(dx) + row0, Q, lane, acc);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const float s = wave_sum(acc[k]);
            if (lane == 0) dTs[t * kTs + k] = s;
        }
    }
    __syncthreads();
    if (wave == 0 && lane < ntok) {
        const int64_t tok = first + lane;
        const uint4* tp = reinterpret_cast<const uint4*>(Tin + tok * 16);
        float T[16], G[16], out[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4 v = stream_load(tp + k);
            T[4 * k] = __uint_as_float(v.x);
            T[4 * k + 1] = __uint_as_float(v.y);
            T[4 * k + 2] = __uint_as_float(v.z);
            T[4 * k + 3] = __uint_as_float(v.w);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) G[k] = dTs[lane * kTs + k];
        implicit_grad<4>(T, G, out);
        uint4* dp = reinterpret_cast<uint4*>(dH + tok * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            stream_store(dp + k, make_uint4(__float_as_uint(out[4 * k]), __float_as_uint(out[4 * k + 1]),
                                            __float_as_uint(out[4 * k + 2]), __float_as_uint(out[4 * k + 3])));
    }
}

}  // namespace mix
}  // namespace birk
