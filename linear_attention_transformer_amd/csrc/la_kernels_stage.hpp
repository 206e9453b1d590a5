// la_kernels_stage.hpp -- head sizes other than the native 32, 64, 128, 256.
//
// A head of size D runs as one of the next native size Dp > D with the extra
// columns zero.  That is exact: the zero columns of q and k add nothing to
// q.k; the zero columns of v give zero output columns (0 / den); the padded
// rows and columns of S, z, u, dS, r, t stay zero; and the padded columns of
// dQ, dK, dV come out zero and are dropped.  The staging kernels copy
// between the caller's [rows, D] layout and the padded [rows, Dp] one in the
// storage type of the call.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "la_kernels.hpp"

namespace la {
namespace stg {

constexpr int kThreads = 256;

// [rows, D] -> [rows, Dp] with zero columns D..Dp-1.  A thread writes one
// 16-byte chunk of a padded row; it reads the chunk as one vector when D is
// a multiple of the chunk (rows then stay 16-byte aligned), else element by
// element.
template <class ST>
__global__ __launch_bounds__(kThreads) void k_pad(const typename ST::T *__restrict__ src,
                                                  typename ST::T *__restrict__ dst,
                                                  int64_t rows, int D, int Dp)
{
    typedef typename ST::T T;
    constexpr int V = 16 / sizeof(T);
    const int cpr = Dp / V;
    const int64_t total = rows * cpr;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        const int64_t r = i / cpr;
        const int c0 = (int)(i - r * cpr) * V;
        uint4 out = {0u, 0u, 0u, 0u};
        if (D % V == 0) {
            if (c0 < D)
                out = *reinterpret_cast<const uint4 *>(src + r * D + c0);
        } else {
            T e[V];
#pragma unroll
            for (int x = 0; x < V; ++x)
                e[x] = c0 + x < D ? src[r * D + c0 + x] : T(0);
            out = __builtin_bit_cast(uint4, e);
        }
        *reinterpret_cast<uint4 *>(dst + r * Dp + c0) = out;
    }
}

// [rows, Dp] -> the first D columns of each padded row, written to row n of
// head bh (r = bh * N + n) in the output layout ol.  A thread reads one
// 16-byte chunk of a padded row and writes its part below D, as one 16-byte
// store when the columns and every stride of the layout allow it.
template <class ST>
__global__ __launch_bounds__(kThreads) void k_unpad(const typename ST::T *__restrict__ src,
                                                    typename ST::T *__restrict__ dst,
                                                    int64_t rows, int D, int Dp, int64_t N,
                                                    OutLay ol)
{
    typedef typename ST::T T;
    constexpr int V = 16 / sizeof(T);
    const int cpr = (D + V - 1) / V;          // chunks holding real columns
    const int64_t total = rows * cpr;
    const bool vec = D % V == 0 && ol.sn % V == 0 && ol.sh % V == 0 && ol.sb % V == 0;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        const int64_t r = i / cpr;
        const int c0 = (int)(i - r * cpr) * V;
        const uint4 in = *reinterpret_cast<const uint4 *>(src + r * Dp + c0);
        const int64_t bh = r / N;
        T *drow = dst + ol.head(bh) + (r - bh * N) * ol.sn;
        if (vec) {
            *reinterpret_cast<uint4 *>(drow + c0) = in;
        } else {
            T e[V];
            *reinterpret_cast<uint4 *>(e) = in;
#pragma unroll
            for (int x = 0; x < V; ++x)
                if (c0 + x < D)
                    drow[c0 + x] = e[x];
        }
    }
}

// A record [M (Ds x Ds) | x (Ds) | y (Ds)] per head re-laid for head size
// Dd, zero outside the source (src null: all zero).
__global__ __launch_bounds__(kThreads) void k_stage_record(const float *__restrict__ src,
                                                           float *__restrict__ dst,
                                                           int64_t heads, int Ds, int Dd)
{
    const int64_t ps = (int64_t)Dd * Dd + 2 * Dd, pss = (int64_t)Ds * Ds + 2 * Ds;
    const int64_t total = heads * ps;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        const int64_t h = i / ps;
        const int64_t e = i - h * ps;
        int64_t from = -1;
        if (e < (int64_t)Dd * Dd) {
            const int a = (int)(e / Dd), b = (int)(e % Dd);
            if (a < Ds && b < Ds)
                from = (int64_t)a * Ds + b;
        } else {
            const int64_t j = e - (int64_t)Dd * Dd;   // 0 .. 2 Dd - 1
            const int part = (int)(j / Dd), c = (int)(j % Dd);
            if (c < Ds)
                from = (int64_t)Ds * Ds + (int64_t)part * Ds + c;
        }
        dst[i] = (src != nullptr && from >= 0) ? src[h * pss + from] : 0.f;
    }
}

}  // namespace stg
}  // namespace la
