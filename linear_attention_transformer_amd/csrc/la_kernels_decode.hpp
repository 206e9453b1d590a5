// la_kernels_decode.hpp -- one recurrent (causal) step per head: the state
// update of the state-update pseudocode in section 2 of the cloud.baidu.com
// article ("Transformer Based Linear Attention with Optimized GPU Kernel
// Implementation"), followed by the normalised output of the new token
// (sciencestack.ai page, TL;DR: the normalisation scheme):
//
//     S' = S + k v^T,  z' = z + k,  u' = u + v,  n' = n + 1
//     den = n' + q.z',  o = (u' + S'^T q) / den
//
// The state moves as records [S (D x D, row-major) | z | u] (fp32), read from
// `rin` (null: the zero state of an empty prefix) and written to `rout`
// (distinct buffers: every workgroup of a head reads z while one of them
// writes z').  The step is bound by HBM: it reads and writes the D^2 + 2D
// floats of each head's record once.
//
// Work split: a workgroup takes one head and a block of CB columns of S.
// Thread (rg, cg) holds four consecutive columns (one 16-byte vector) and
// walks its rows rg, rg + RG, ...; so the CB/4 threads of a row read one
// contiguous run of the row.  The row partials of S'^T q meet in LDS.
// k_decode_any takes any head size up to 256 (one column per thread, scalar
// loads) and fp16 storage as well.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "la_kernels.hpp"
#include "la_kernels_stage.hpp"

namespace la {
namespace dec {

constexpr int kThreads = 256;

template <int D>
constexpr int cols_per_block()
{
    return D >= 32 ? 32 : D;
}

template <int D>
constexpr int blocks_per_head()
{
    return D / cols_per_block<D>();
}

template <class ST>
__device__ __forceinline__ float ld1(const typename ST::T *p)
{
    return ST::widen1(*p);
}

template <class ST, int D>
__global__ __launch_bounds__(kThreads) void k_decode(
    const typename ST::T *__restrict__ Q, const typename ST::T *__restrict__ K,
    const typename ST::T *__restrict__ V, typename ST::T *__restrict__ O,
    float *__restrict__ den_out, const float *__restrict__ rin, float *__restrict__ rout,
    const int64_t *__restrict__ counts, float n_all, int H)
{
    constexpr int CB = cols_per_block<D>();
    constexpr int NB = blocks_per_head<D>();
    constexpr int CG = CB / 4;             // 16-byte column groups of the block
    constexpr int RG = kThreads / CG;      // row groups
    constexpr int PS = D * D + 2 * D;
    static_assert(CB % 4 == 0 && kThreads % CG == 0, "column split");

    __shared__ float qs[D], ks[D];
    __shared__ float part[RG][CB];
    __shared__ float dots[2];               // q.k, q.z

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / NB;
    const int cb = blockIdx.x % NB;
    const int64_t io = bh * D;              // this head's token row
    const bool has_in = rin != nullptr;
    const float *r = has_in ? rin + bh * PS : nullptr;
    float *w = rout + bh * PS;

    for (int d = tid; d < D; d += kThreads) {
        qs[d] = ld1<ST>(Q + io + d);
        ks[d] = ld1<ST>(K + io + d);
    }
    // q.k and q.z over D, in wave 0 (each lane a strided part, then a
    // butterfly over the wave)
    if (tid < 64) {
        float qk = 0.f, qz = 0.f;
        for (int d = tid; d < D; d += 64) {
            const float q = ld1<ST>(Q + io + d);
            qk += q * ld1<ST>(K + io + d);
            qz += has_in ? q * r[D * D + d] : 0.f;
        }
        qk = wave_sum(qk);
        qz = wave_sum(qz);
        if (tid == 0) {
            dots[0] = qk;
            dots[1] = qz;
        }
    }
    __syncthreads();

    const int cg = tid % CG, rg = tid / CG;
    const int c0 = cb * CB + 4 * cg;
    float v4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v4[i] = ld1<ST>(V + io + c0 + i);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = rg; d < D; d += RG) {
        const float4 s = has_in ? *reinterpret_cast<const float4 *>(r + (int64_t)d * D + c0)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        const float kd = ks[d], qd = qs[d];
        float4 t;
        t.x = s.x + kd * v4[0];
        t.y = s.y + kd * v4[1];
        t.z = s.z + kd * v4[2];
        t.w = s.w + kd * v4[3];
        *reinterpret_cast<float4 *>(w + (int64_t)d * D + c0) = t;
        acc[0] += qd * t.x;
        acc[1] += qd * t.y;
        acc[2] += qd * t.z;
        acc[3] += qd * t.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        part[rg][4 * cg + i] = acc[i];
    if (cb == 0)
        for (int d = tid; d < D; d += kThreads)
            w[D * D + d] = (has_in ? r[D * D + d] : 0.f) + ks[d];
    __syncthreads();

    if (tid < CB) {
        const int e = cb * CB + tid;
        float num = 0.f;
        for (int g = 0; g < RG && g < D; ++g)
            num += part[g][tid];
        const float v = ld1<ST>(V + io + e);
        const float u1 = (has_in ? r[D * D + D + e] : 0.f) + v;
        w[D * D + D + e] = u1;
        const float n = counts ? (float)counts[bh / H] : n_all;
        // den = (n + 1) + q.z' with q.z' = q.z + q.k
        const float den = (n + 1.f) + (dots[1] + dots[0]);
        O[io + e] = ST::narrow((u1 + num) / den);
        if (den_out && cb == 0 && tid == 0)
            den_out[bh] = den;
    }
}

// Any head size D <= 256 (records of D*D + 2*D floats, no alignment beyond
// 4 bytes).  A workgroup takes one head and 32 columns; thread (rg, c) holds
// column c of the block and walks rows rg, rg + 8, ...
template <class ST>
__global__ __launch_bounds__(kThreads) void k_decode_any(
    const typename ST::T *__restrict__ Q, const typename ST::T *__restrict__ K,
    const typename ST::T *__restrict__ V, typename ST::T *__restrict__ O,
    float *__restrict__ den_out, const float *__restrict__ rin, float *__restrict__ rout,
    const int64_t *__restrict__ counts, float n_all, int H, int D)
{
    constexpr int CB = 32, RG = kThreads / CB;
    __shared__ float qs[256], ks[256];
    __shared__ float part[RG][CB];
    __shared__ float dots[2];

    const int nb = (D + CB - 1) / CB;
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x / nb;
    const int cb = blockIdx.x % nb;
    const int64_t ps = (int64_t)D * D + 2 * D;
    const int64_t io = bh * D;
    const bool has_in = rin != nullptr;
    const float *r = has_in ? rin + bh * ps : nullptr;
    float *w = rout + bh * ps;

    for (int d = tid; d < D; d += kThreads) {
        qs[d] = ld1<ST>(Q + io + d);
        ks[d] = ld1<ST>(K + io + d);
    }
    if (tid < 64) {
        float qk = 0.f, qz = 0.f;
        for (int d = tid; d < D; d += 64) {
            const float q = ld1<ST>(Q + io + d);
            qk += q * ld1<ST>(K + io + d);
            qz += has_in ? q * r[(int64_t)D * D + d] : 0.f;
        }
        qk = wave_sum(qk);
        qz = wave_sum(qz);
        if (tid == 0) {
            dots[0] = qk;
            dots[1] = qz;
        }
    }
    __syncthreads();

    const int c = tid % CB, rg = tid / CB;
    const int e = cb * CB + c;
    float acc = 0.f;
    if (e < D) {
        const float ve = ld1<ST>(V + io + e);
        for (int d = rg; d < D; d += RG) {
            const int64_t x = (int64_t)d * D + e;
            const float t = (has_in ? r[x] : 0.f) + ks[d] * ve;
            w[x] = t;
            acc += qs[d] * t;
        }
    }
    part[rg][c] = acc;
    if (cb == 0)
        for (int d = tid; d < D; d += kThreads)
            w[(int64_t)D * D + d] = (has_in ? r[(int64_t)D * D + d] : 0.f) + ks[d];
    __syncthreads();

    if (tid < CB && e < D) {
        float num = 0.f;
        for (int g = 0; g < RG; ++g)
            num += part[g][tid];
        const float v = ld1<ST>(V + io + e);
        const float u1 = (has_in ? r[(int64_t)D * D + D + e] : 0.f) + v;
        w[(int64_t)D * D + D + e] = u1;
        const float n = counts ? (float)counts[bh / H] : n_all;
        const float den = (n + 1.f) + (dots[1] + dots[0]);
        O[io + e] = ST::narrow((u1 + num) / den);
        if (den_out && cb == 0 && tid == 0)
            den_out[bh] = den;
    }
}

}  // namespace dec
}  // namespace la
