// la_kernels_bf16.hpp -- bf16-storage kernels on the bf16 matrix cores of
// gfx950 (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Same method and layout as la_kernels_nc.hpp (pages about "Transformer
// Based Linear Attention with Optimized GPU Kernel Implementation":
// sciencestack.ai TL;DR and Figure 1 caption; cloud.baidu.com article,
// section 2).  With bf16 storage every row of Q, K, V and dO is exactly a
// bf16 vector, so a product with it on the bf16 MFMA accumulates exact
// products in fp32.  The other factor of the apply products is an fp32 state
// (S, dS); it is carried as two bf16 terms, hi = bf16(x) and lo = bf16(x -
// hi), which represent x to about 2^-17 relative, and each k-step issues two
// MFMAs (hi, lo) against the same row operand.
//
// v_mfma_f32_32x32x16_bf16: lane l = 32 h + j supplies A[m = j][k = 8h ..
// 8h + 7] and B[k = 8h .. 8h + 7][n = j] (8 bf16 each) and holds accumulator
// element i at row 8 (i / 4) + 4 h + i % 4, column j -- the same output
// layout as the fp32 32x32x2 form, so the epilogues are unchanged.
#pragma once

#include "la_kernels_nc.hpp"

namespace la {
namespace bf {

using nc::dot4;
using nc::drain_loads;
using nc::f16v;
using nc::zero16;

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16v mma16(bf8 a, bf8 b, f16v c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// word 3 of a raw buffer resource descriptor on gfx9-family GPUs
constexpr int kBufferWord3 = 0x00020000;

// x = hi + lo with hi, lo bf16 (round to nearest even both times)
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo)
{
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

// the 8 bf16 of b as fp32
__device__ __forceinline__ void unpack8(bf8 b, float *o)
{
    const uint4 u = __builtin_bit_cast(uint4, b);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Element s of two 8 x bf16 vectors as one bf16 pair (t0's in the low half)
__device__ __forceinline__ uint32_t pair_bf16(const uint4 &t0, const uint4 &t1, int s)
{
    const uint32_t w0 = reinterpret_cast<const uint32_t *>(&t0)[s / 2];
    const uint32_t w1 = reinterpret_cast<const uint32_t *>(&t1)[s / 2];
    return (s & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u)
                   : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
}

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// sum of the 8 bf16 of b, added to c (bf16 dot2 against (1, 1): the
// products are exact, the sums fp32)
__device__ __forceinline__ float sum8(bf8 b, float c)
{
    const uint4 u = __builtin_bit_cast(uint4, b);
    const bf2 ones = {(__bf16)1.f, (__bf16)1.f};
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.x), ones, c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.y), ones, c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.z), ones, c, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.w), ones, c, false);
}

typedef short v4s __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 on gfx950: within each group of 16 lanes, lane p = 4e + f
// points at row r0 + e, columns c0 + 4f .. + 3 of a row-major bf16 tile;
// lane i of the group then receives rows r0 .. r0 + 3 of column c0 + i.
__device__ __forceinline__ v4s tr4(const uint16_t *tile, int pitch, int r0, int c0, int p)
{
    const uint16_t *a = tile + (r0 + (p >> 2)) * pitch + c0 + 4 * (p & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(a));
}

// the MFMA operand of lane (j, h) = 32 h + j: rows rb + 8 h .. + 7 of column
// cb0 + j (8 consecutive tokens of one column)
__device__ __forceinline__ bf8 col8(const uint16_t *tile, int pitch, int rb, int cb0, int lane)
{
    const int g = lane >> 4, p = lane & 15;
    const int r0 = rb + 8 * (g >> 1), c0 = cb0 + 16 * (g & 1);
    const v4s x = tr4(tile, pitch, r0, c0, p);
    const v4s y = tr4(tile, pitch, r0 + 4, c0, p);
    const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
    return __builtin_bit_cast(bf8, uint4{ux.x, ux.y, uy.x, uy.y});
}

// the MFMA operand of lane (j, h): row rb + j, columns c + 8 h .. + 7
__device__ __forceinline__ bf8 row8(const uint16_t *tile, int pitch, int rb, int c, int j, int h)
{
    return *reinterpret_cast<const bf8 *>(tile + (rb + j) * pitch + c + 8 * h);
}

// two fp32 as hi and lo bf16 pairs (a in the low halves): one paired
// round-to-nearest conversion for hi, the residuals, one for lo
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo)
{
    hi = StBF16::narrow2(a, b);
    lo = StBF16::narrow2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// four fp32 as hi and lo bf16 (two 8-byte words)
__device__ __forceinline__ void split4(float a, float b, float c, float d, uint2 &hi, uint2 &lo)
{
    split2(a, b, hi.x, lo.x);
    split2(c, d, hi.y, lo.y);
}

// eight fp32 as hi and lo bf16 MFMA operands (paired conversions)
__device__ __forceinline__ void split8v(const float *x, bf8 &hi, bf8 &lo)
{
    uint4 h, l;
    split2(x[0], x[1], h.x, l.x);
    split2(x[2], x[3], h.y, l.y);
    split2(x[4], x[5], h.z, l.z);
    split2(x[6], x[7], h.w, l.w);
    hi = __builtin_bit_cast(bf8, h);
    lo = __builtin_bit_cast(bf8, l);
}

constexpr int kApplyThreads = 256;

// ============================================================ apply
// KIND 0 forward : A = S^T, o_i = (u + A q_i) / (N + q_i.z), X = Q;
//                  den_out[i] = N + q_i.z (optional).  Each wave forms q_i.z
//                  over its own 32 columns; the partials meet in LDS at the
//                  round's barrier.
// KIND 1 dQ      : A = S, X = dO, X2 = Q: y_i = A g_i, den_i = N + q_i.z,
//                  c_i = (g_i.u + q_i.y_i) / den_i^2, dq_i = y_i / den_i - c_i z;
//                  cbuf[i] = (c_i, 1/den_i).  q_i.y_i, g_i.u and q_i.z are
//                  formed per column block and summed through LDS at the
//                  round's barrier.
// KIND 2 dK | dV : parity 0: A = dS, X = V, dk_j = A v_j - r;
//                  parity 1: A = dS^T, X2 = K, dv_j = A k_j + t.
// The structure is k_apply_nc's: waves own 32-column output blocks (and, for
// D < 128, row groups), hold their block of A in registers (as hi/lo bf16
// pairs: 8 per lane and k-step of 16), stage each round of rows in LDS
// (raw bf16, double-buffered, one barrier per round), and read the B operand
// as one 16-byte LDS read per k-step.  Stores of a round are issued during
// a later round's MFMAs.  Rows are loaded through a per-round buffer descriptor that
// covers only the rows before the segment end (zeros beyond it).
template <int D, int KIND>
__global__ __launch_bounds__(kApplyThreads) void k_apply_bf(
    const uint16_t *__restrict__ X, const uint16_t *__restrict__ X2, uint16_t *__restrict__ Out,
    uint16_t *__restrict__ Out2, float *__restrict__ den_out, float *__restrict__ cbuf,
    const float *__restrict__ rec, int64_t N, int64_t seg_len, int nseg, float n0, OutLay ol)
{
    static_assert(D >= 32 && D <= 128, "32-column output blocks");
    static_assert(KIND >= 0 && KIND <= 2, "forward, dQ or dK | dV");
    constexpr int KS = D / 16;               // k-steps of 16
    constexpr int NWAVE = kApplyThreads / 64;
    constexpr int NCB = D / 32;
    constexpr int NRG = NWAVE / NCB;
    constexpr int TR = 32 * NRG;             // rows per round
    constexpr int LDX = D + 8;               // LDS row pitch (bf16)
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int PER = TR * CPR / kApplyThreads;
    static_assert(PER >= 1 && TR * CPR % kApplyThreads == 0, "staging split");
    constexpr bool DQ = (KIND == 1);
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][TR * LDX];
    __shared__ __attribute__((aligned(16))) uint16_t qs[DQ ? 2 : 1][DQ ? TR * LDX : 8];
    __shared__ __attribute__((aligned(16))) float vz[KIND <= 1 ? D : 4];
    __shared__ __attribute__((aligned(16))) float vu[DQ ? D : 4];
    // per-row sums over the column blocks (forward: q.z; dQ: q.y), one
    // partial per wave, added up after the round's barrier
    constexpr bool XCH = (KIND <= 1);
    __shared__ float xch[XCH ? 2 : 1][NRG][NCB][32][DQ ? 2 : 1];
    // output rows of a round (bf16), stored as whole rows by the workgroup
    // LAG rounds later: the dK | dV tile is complete at the round's barrier,
    // the forward and dQ tiles (normalised after it) only at the next one
    constexpr int LAG = XCH ? 2 : 1;
    constexpr int OCH = TR * CPR / kApplyThreads;  // 16-byte output chunks per thread
    __shared__ __attribute__((aligned(16))) uint16_t ot[2][TR * LDX];

    // unit = segment (forward, dQ) or 2 segment + parity (dK | dV)
    int64_t bh;
    int unit;
    xcd_unit(blockIdx.x, KIND == 2 ? 2 * nseg : nseg, bh, unit);
    const int sub = (KIND == 2) ? (unit & 1) : 0;
    const int seg = (KIND == 2) ? (unit >> 1) : unit;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int cb = w % NCB, rg = w / NCB;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + bh * (int64_t)(D * D + 2 * D);
    const bool colread = (KIND == 0) || (KIND == 2 && sub == 1);
    const uint16_t *xh = ((KIND == 2 && sub == 1) ? X2 : X) + hoff;
    const uint16_t *qh = DQ ? X2 + hoff : nullptr;
    uint16_t *oh = ((KIND == 2 && sub == 1) ? Out2 : Out) + ol.head(bh);

    uint4 stg[PER], stq[DQ ? PER : 1];
    auto fetch_round = [&](int64_t r0) {
        const int rows = (int)(end - r0 < TR ? end - r0 : TR);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(xh + r0 * D), (short)0, rows * D * 2, kBufferWord3);
        __amdgpu_buffer_rsrc_t rq;
        if constexpr (DQ)
            rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(qh + r0 * D), (short)0,
                                                   rows * D * 2, kBufferWord3);
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * kApplyThreads;
            const int off = (c / CPR) * D * 2 + 16 * (c % CPR);
            stg[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
            if constexpr (DQ)
                stq[p] =
                    __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
        }
    };
    auto stage_round = [&](int buf) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * kApplyThreads;
            *reinterpret_cast<uint4 *>(&xs[buf][(c / CPR) * LDX + 8 * (c % CPR)]) = stg[p];
            if constexpr (DQ)
                *reinterpret_cast<uint4 *>(&qs[buf][(c / CPR) * LDX + 8 * (c % CPR)]) = stq[p];
        }
    };

    const int64_t nrounds = (end - beg + TR - 1) / TR;
    fetch_round(beg);

    // this wave's block of A as hi/lo bf16:
    // a?[ks][s] = A[32 cb + j][16 ks + 8 h + s]
    bf8 ahi[KS], alo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        float v[8];
        if (colread) {
#pragma unroll
            for (int s = 0; s < 8; ++s)
                v[s] = st[(16 * ks + 8 * h + s) * D + 32 * cb + j];
        } else {
            const f4 v0 = *reinterpret_cast<const f4 *>(st + (32 * cb + j) * D + 16 * ks + 8 * h);
            const f4 v1 =
                *reinterpret_cast<const f4 *>(st + (32 * cb + j) * D + 16 * ks + 8 * h + 4);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                v[s] = v0[s];
                v[s + 4] = v1[s];
            }
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            __bf16 hi, lo;
            split_bf16(v[s], hi, lo);
            ahi[ks][s] = hi;
            alo[ks][s] = lo;
        }
    }
    // epilogue vector at the lane's output columns 32*cb + 8*q + 4*h + (0..3):
    // u (forward), z (dQ), -r (dK) or t (dV)
    f4 ev[4];
    {
        const float *vec = st + D * D + ((KIND == 0 || (KIND == 2 && sub == 1)) ? D : 0);
        const float sgn = (KIND == 2 && sub == 0) ? -1.f : 1.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            ev[q] = sgn * *reinterpret_cast<const f4 *>(vec + 32 * cb + 8 * q + 4 * h);
    }
    if constexpr (KIND <= 1)
        for (int e = tid; e < D; e += kApplyThreads) {
            vz[e] = st[D * D + e];
            if constexpr (DQ)
                vu[e] = st[D * D + D + e];
        }
    stage_round(0);
    drain_loads();
    if (nrounds > 1)
        fetch_round(beg + TR);
    __syncthreads();

    // this lane's 4 x 4 output values of a round into its tile
    auto put_tile = [&](int tb, const f4 *o) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint2 r;
            r.x = StBF16::narrow2(o[q][0], o[q][1]);
            r.y = StBF16::narrow2(o[q][2], o[q][3]);
            *reinterpret_cast<uint2 *>(&ot[tb][(32 * rg + j) * LDX + 32 * cb + 8 * q + 4 * h]) = r;
        }
    };
    // chunk p of round rr's tile to global memory (16 bytes per lane;
    // consecutive lanes cover consecutive 16-byte pieces of a row)
    auto store_tile = [&](int64_t rr, int p) {
        const int c = tid + p * kApplyThreads;
        const int64_t grow = beg + rr * TR + c / CPR;
        if (grow < end)
            *reinterpret_cast<uint4 *>(oh + grow * ol.sn + 8 * (c % CPR)) =
                *reinterpret_cast<const uint4 *>(&ot[(int)(rr & 1)][(c / CPR) * LDX + 8 * (c % CPR)]);
    };

    for (int64_t round = 0; round < nrounds; ++round) {
        const int buf = (int)(round & 1);
        const uint16_t *xt = &xs[buf][(32 * rg + j) * LDX + 8 * h];
        f16v acc = zero16();
        bf8 xn = *reinterpret_cast<const bf8 *>(xt);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf8 x = xn;
            if (ks + 1 < KS)
                xn = *reinterpret_cast<const bf8 *>(xt + 16 * (ks + 1));
            acc = mma16(ahi[ks], x, acc);
            acc = mma16(alo[ks], x, acc);
#pragma unroll
            for (int p = 0; p < OCH; ++p)
                if (round >= LAG && ks == (p * KS) / OCH)
                    store_tile(round - LAG, p);
            __builtin_amdgcn_sched_barrier(0);
        }

        const int64_t row = beg + round * TR + 32 * rg + j;
        f4 pend[4];
        // a.b over this block's 32 columns of two staged rows (lane half h
        // sums 16 of them; both halves get the total)
        auto rowdot = [&](const uint16_t *a, const float *b) {
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < 16; e += 8) {
                float af[8];
                unpack8(*reinterpret_cast<const bf8 *>(a + 32 * cb + 16 * h + e), af);
                const float *br = b + 32 * cb + 16 * h + e;
                p += dot4(f4{af[0], af[1], af[2], af[3]}, *reinterpret_cast<const f4 *>(br)) +
                     dot4(f4{af[4], af[5], af[6], af[7]}, *reinterpret_cast<const f4 *>(br + 4));
            }
            return swap32_sum(p);
        };
        if constexpr (KIND == 0) {
            const float p = rowdot(&xs[buf][(32 * rg + j) * LDX], vz);  // q.z
            if (h == 0)
                xch[buf][rg][cb][j][0] = p;
        } else if constexpr (KIND == 2) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pend[q] = f4{acc[4 * q] + ev[q][0], acc[4 * q + 1] + ev[q][1],
                             acc[4 * q + 2] + ev[q][2], acc[4 * q + 3] + ev[q][3]};
            put_tile(buf, pend);
        } else {
            // q.y over this block's 32 output columns (y = S g in the
            // accumulators), plus g.u and q.z over its 32 input columns
            const uint16_t *qr = &qs[buf][(32 * rg + j) * LDX + 32 * cb + 4 * h];
            float p = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint2 u = *reinterpret_cast<const uint2 *>(qr + 8 * q);
                p += __uint_as_float(u.x << 16) * acc[4 * q] +
                     __uint_as_float(u.x & 0xffff0000u) * acc[4 * q + 1] +
                     __uint_as_float(u.y << 16) * acc[4 * q + 2] +
                     __uint_as_float(u.y & 0xffff0000u) * acc[4 * q + 3];
            }
            p = swap32_sum(p);
            p += rowdot(&xs[buf][(32 * rg + j) * LDX], vu);               // g.u
            const float pz = rowdot(&qs[buf][(32 * rg + j) * LDX], vz);  // q.z
            if (h == 0) {
                xch[buf][rg][cb][j][0] = p;
                xch[buf][rg][cb][j][DQ ? 1 : 0] = pz;
            }
        }
        if (round + 1 < nrounds) {
            stage_round(buf ^ 1);
            if (round + 2 < nrounds)
                fetch_round(beg + (round + 2) * TR);
        }
        __syncthreads();
        if constexpr (KIND == 0) {
            float qz = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < NCB; ++c2)
                qz += xch[buf][rg][c2][j][0];
            const float den = (n0 + (float)N) + qz;
            const float inv = 1.f / den;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pend[q] = f4{(acc[4 * q] + ev[q][0]) * inv, (acc[4 * q + 1] + ev[q][1]) * inv,
                             (acc[4 * q + 2] + ev[q][2]) * inv, (acc[4 * q + 3] + ev[q][3]) * inv};
            if (den_out != nullptr && row < end && h == 0 && cb == 0)
                den_out[bh * N + row] = den;
            put_tile(buf, pend);
        }
        if constexpr (DQ) {
            float sy = 0.f, qz = 0.f;  // g.u + q.y and q.z
#pragma unroll
            for (int c2 = 0; c2 < NCB; ++c2) {
                sy += xch[buf][rg][c2][j][0];
                qz += xch[buf][rg][c2][j][DQ ? 1 : 0];
            }
            const float inv = 1.f / ((n0 + (float)N) + qz);
            const float c = sy * inv * inv;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pend[q] = f4{acc[4 * q] * inv - c * ev[q][0], acc[4 * q + 1] * inv - c * ev[q][1],
                             acc[4 * q + 2] * inv - c * ev[q][2],
                             acc[4 * q + 3] * inv - c * ev[q][3]};
            if (row < end && h == 0 && cb == 0)
                reinterpret_cast<float2 *>(cbuf)[bh * N + row] = float2{c, inv};
            put_tile(buf, pend);
        }
    }
    __syncthreads();
    for (int64_t rr = nrounds - LAG < 0 ? 0 : nrounds - LAG; rr < nrounds; ++rr)
#pragma unroll
        for (int p = 0; p < OCH; ++p)
            store_tile(rr, p);
}

// ============================================================ reduction
// Record (bh, seg) as k_reduce_nc writes it: Mat[D][D] = sum_t X[t]^T Y'[t],
// cx = sum_t w_t X[t], cy = sum_t Y'[t] over the segment's rows, with
//   forward  (GRAD = false): X = K, Y' = V, w = 1        -> S, z, u
//   backward (GRAD = true) : X = Q, Y' = dO / den, w = c -> dS, r, t
// and (c_t, 1/den_t) from cbuf.  Each round of TT = 64 rows is loaded as
// whole rows (consecutive lanes take consecutive 16-byte pieces of a row)
// and staged as natural rows in LDS, one 16-byte write per piece; the
// contraction runs over tokens, and both MFMA operands (8 consecutive tokens
// of one column per lane) are read with the LDS transpose read.  Y' of the
// backward is an fp32 product, kept as hi and lo planes (two MFMAs per
// step).  The column sums are accumulated by the staging lanes (each keeps
// the same 8 columns in every round) and reduced once at the end.  Waves own
// 32x32 output tiles (D = 128: a 2 x 2 block each); for D = 32 the four
// waves split the k-steps of the single tile and add up in LDS.
template <int D, bool GRAD>
__global__ __launch_bounds__(256) void k_reduce_bf(
    const uint16_t *__restrict__ X, const uint16_t *__restrict__ Y,
    const float *__restrict__ cbuf, float *__restrict__ part, int64_t N, int64_t seg_len,
    int nseg)
{
    static_assert(D >= 32 && D <= 128, "32x32 tiles");
    constexpr int NT = 256, TT = 64;
    constexpr int LDP = D + 16;             // row pitch: 16-lane transpose reads conflict-free
    constexpr int NTILE1 = D / 32;          // tiles per dimension
    constexpr int NTILE = NTILE1 * NTILE1;
    constexpr int TPW1 = NTILE >= 4 ? NTILE1 / 2 : 1;  // tiles per wave per dimension
    constexpr int WPT = NTILE >= 4 ? 1 : 4;           // waves sharing a tile (k split)
    constexpr int CPR = D / 8;              // 16-byte pieces per row
    constexpr int PER = TT * CPR / NT;      // pieces per thread per round
    static_assert(PER >= 1 && TT * CPR % NT == 0 && NT % CPR == 0, "staging split");
    constexpr int NYP = GRAD ? 2 : 1;       // planes of Y'
    __shared__ __attribute__((aligned(16))) uint16_t xs[TT * LDP];
    __shared__ __attribute__((aligned(16))) uint16_t ys[NYP][TT * LDP];
    __shared__ float red[WPT > 1 ? (WPT - 1) * 16 * 64 : 1];
    __shared__ float csx[NT / 64][CPR][8], csy[NT / 64][CPR][8];

    const int64_t bh = blockIdx.x / nseg;
    const int seg = (int)(blockIdx.x % nseg);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = bh * N * D;
    const uint16_t *xh = X + hoff, *yh = Y + hoff;
    const float2 *ch = GRAD ? reinterpret_cast<const float2 *>(cbuf) + bh * N : nullptr;
    // output tiles of this wave
    const int m0 = (NTILE >= 4) ? (w / 2) * 32 * TPW1 : 0;
    const int n0 = (NTILE >= 4) ? (w % 2) * 32 * TPW1 : 0;
    const int ksplit = (NTILE >= 4) ? 0 : w;  // D = 32: this wave's k-step

    // staging pieces: q = tid + p * NT -> row q / CPR, columns 8 (q % CPR) ..
    // (the same 8 columns, tid % CPR, for every piece of the thread)
    uint4 sx[PER], sy[PER];
    float2 scb[PER];
    float cx[8], cy[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        cx[s] = cy[s] = 0.f;

    auto fetch = [&](int64_t r0) {
        const int rows = (int)(end - r0 < TT ? end - r0 : TT);
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(xh + r0 * D), (short)0, rows * D * 2, kBufferWord3);
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(yh + r0 * D), (short)0, rows * D * 2, kBufferWord3);
        __amdgpu_buffer_rsrc_t rc;
        if constexpr (GRAD)
            rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float2 *>(ch + r0), (short)0,
                                                   rows * 8, kBufferWord3);
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int q = tid + p * NT;
            const int off = (q / CPR) * D * 2 + 16 * (q % CPR);
            sx[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
            sy[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ry, off, 0, 0));
            if constexpr (GRAD)
                scb[p] = __builtin_bit_cast(
                    float2, __builtin_amdgcn_raw_buffer_load_b64(rc, (q / CPR) * 8, 0, 0));
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int q = tid + p * NT;
            const int o = (q / CPR) * LDP + 8 * (q % CPR);
            *reinterpret_cast<uint4 *>(&xs[o]) = sx[p];
            float xv[8], yv[8];
            StBF16::widen(sx[p], xv);
            StBF16::widen(sy[p], yv);
            if constexpr (!GRAD) {
                *reinterpret_cast<uint4 *>(&ys[0][o]) = sy[p];
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    cx[s] += xv[s];
                    cy[s] += yv[s];
                }
            } else {
                const float c = scb[p].x, inv = scb[p].y;
                uint4 hi, lo;
                split2(yv[0] * inv, yv[1] * inv, hi.x, lo.x);
                split2(yv[2] * inv, yv[3] * inv, hi.y, lo.y);
                split2(yv[4] * inv, yv[5] * inv, hi.z, lo.z);
                split2(yv[6] * inv, yv[7] * inv, hi.w, lo.w);
                *reinterpret_cast<uint4 *>(&ys[0][o]) = hi;
                *reinterpret_cast<uint4 *>(&ys[1][o]) = lo;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    cx[s] += c * xv[s];
                    cy[s] += yv[s] * inv;
                }
            }
        }
    };

    f16v acc[TPW1][TPW1];
#pragma unroll
    for (int a = 0; a < TPW1; ++a)
#pragma unroll
        for (int b = 0; b < TPW1; ++b)
            acc[a][b] = zero16();

    const int64_t nrounds = (end - beg + TT - 1) / TT;
    fetch(beg);
    for (int64_t round = 0; round < nrounds; ++round) {
        __syncthreads();  // the previous round's operands have been read
        stage();
        if (round + 1 < nrounds)
            fetch(beg + (round + 1) * TT);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TT / 16; ++kk) {
            if (WPT > 1 && kk != ksplit)
                continue;
            bf8 av[TPW1], bv[TPW1][NYP];
#pragma unroll
            for (int a = 0; a < TPW1; ++a)
                av[a] = col8(xs, LDP, 16 * kk, m0 + 32 * a, lane);
#pragma unroll
            for (int b = 0; b < TPW1; ++b)
#pragma unroll
                for (int y = 0; y < NYP; ++y)
                    bv[b][y] = col8(ys[y], LDP, 16 * kk, n0 + 32 * b, lane);
#pragma unroll
            for (int a = 0; a < TPW1; ++a)
#pragma unroll
                for (int b = 0; b < TPW1; ++b)
#pragma unroll
                    for (int y = 0; y < NYP; ++y)
                        acc[a][b] = mma16(av[a], bv[b][y], acc[a][b]);
        }
    }

    const int j = lane & 31, h = lane >> 5;
    float *out = part + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
    if constexpr (WPT > 1) {
        // D = 32: waves 1..3 hand their k-split partials to wave 0
        if (w > 0)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                red[((w - 1) * 16 + i) * 64 + lane] = acc[0][0][i];
        __syncthreads();
        if (w == 0)
            for (int o = 0; o < WPT - 1; ++o)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[0][0][i] += red[(o * 16 + i) * 64 + lane];
    }
    if (WPT == 1 || w == 0) {
#pragma unroll
        for (int a = 0; a < TPW1; ++a)
#pragma unroll
            for (int b = 0; b < TPW1; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    out[(m0 + 32 * a + 8 * (i / 4) + 4 * h + (i % 4)) * D + n0 + 32 * b + j] =
                        acc[a][b][i];
    }
    // column sums: the lanes l + k CPR of a wave hold the same 8 columns;
    // sum them (rotations within rows of 16 lanes, then the swaps across
    // rows), then the waves' sums meet in LDS
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        float a = cx[s], b = cy[s];
        if constexpr (CPR <= 4) {
            a += dpp_mov<0x124>(a);  // row_ror:4
            b += dpp_mov<0x124>(b);
        }
        if constexpr (CPR <= 8) {
            a += dpp_mov<0x128>(a);  // row_ror:8
            b += dpp_mov<0x128>(b);
        }
        cx[s] = swap32_sum(swap16_sum(a));
        cy[s] = swap32_sum(swap16_sum(b));
    }
    if (lane < CPR) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            csx[w][lane][s] = cx[s];
            csy[w][lane][s] = cy[s];
        }
    }
    __syncthreads();
    if (tid < D) {
        const int pc2 = tid / 8, s2 = tid % 8;
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int v = 0; v < NT / 64; ++v) {
            a += csx[v][pc2][s2];
            b += csy[v][pc2][s2];
        }
        out[D * D + tid] = a;
        out[D * D + D + tid] = b;
    }
}

// ============================================================ fused dQ + dS (non-causal)
// dQ and the segment's gradient record [dS | r | t] in one pass over Q and
// dO (D = 64, 128), eight waves in two roles over rounds of TR rows:
//   - staging (by the dS waves, two 16-byte pieces of Q and of dO per thread
//     and round, loaded three rounds ahead):
//     den_t = n0 + N + q_t.z from a 16-lane (D / 8-lane) row sum, then
//     a_t = dO_t / den_t as hi / lo planes; Q, dO, a staged as natural rows;
//   - waves 0..3 (dQ role): y_t = S dO_t as in k_apply_bf<D, 1> (S as hi /
//     lo operand registers), c_t = (dO_t.u + q_t.y_t) / den_t^2, dq_t =
//     y_t / den_t - c_t z; they also sum r = sum c_t q_t and t = sum a_t at
//     their output columns, from values kept in registers;
//   - waves 4..7 (dS role): dS += Q^T A over the round's tokens, both
//     operands read with the LDS transpose read (a: hi and lo).
// One barrier per round.  A round's staged rows are read before its barrier
// only (the epilogue after it works from registers and the exchange), so
// staging the next round into the other buffers never overwrites a value
// still to be read.  Rows read whole (dO, the dQ tile) have a pitch of D + 8
// (conflict-free 16-byte row reads), rows read by the transpose read a pitch
// of D + 16 (32 bytes mod 128: conflict-free 16-lane transpose reads).
template <int D>
struct BqBfLds {
    static constexpr int NCB = D / 32, NRG = 4 / NCB, TR = 32 * NRG, LDX = D + 8, LDT = D + 16;
    uint16_t xs[2][TR * LDX];   // dO rows
    uint16_t qs[2][TR * LDT];   // Q rows
    uint16_t ah[2][TR * LDT];   // a = dO / den, hi
    uint16_t al[2][TR * LDT];   // a, lo
    uint16_t ot[2][TR * LDX];   // dQ rows of a round, stored as whole rows
    float ivx[2][TR];           // 1 / den of the round's rows
    float xch[2][NRG][NCB][32]; // per column block: dO.u + q.y
    float vu[D];
    float csr[NRG][D], cst[NRG][D];  // r, t of each row group
};

template <int D>
__global__ __launch_bounds__(512) void k_bwd_q_bf(
    const uint16_t *__restrict__ G, const uint16_t *__restrict__ Q, uint16_t *__restrict__ dQ,
    float *__restrict__ part, const float *__restrict__ rec, int64_t N, int64_t seg_len,
    int nseg, float n0, OutLay ol)
{
    static_assert(D == 64 || D == 128, "two or four column blocks");
    typedef BqBfLds<D> Lt;
    constexpr int NT = 512, KS = D / 16, NCB = Lt::NCB, NRG = Lt::NRG, TR = Lt::TR;
    constexpr int LDX = Lt::LDX, LDT = Lt::LDT, CPR = D / 8;
    static_assert(TR * CPR == NT, "two staging pieces per staging thread and tensor");
    constexpr int TPW1 = NCB / 2;  // dS tiles per wave and dimension
    __shared__ __attribute__((aligned(16))) Lt L;

    int64_t bh;
    int seg;
    xcd_unit(blockIdx.x, nseg, bh, seg);
    const int tid = threadIdx.x, lane = tid & 63, j = lane & 31, h = lane >> 5;
    // the wave index as a scalar: the role branches below are uniform per
    // wave, and each role's loop passes the same barriers
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w4 = w & 3;
    const int cb = w4 % NCB, rg = w4 / NCB;
    const int64_t beg = (int64_t)seg * seg_len;
    const int len = (int)((beg + seg_len < N ? beg + seg_len : N) - beg);  // rows of the segment
    const int64_t hoff = bh * N * D + beg * D;
    const float *st = rec + bh * (int64_t)(D * D + 2 * D);
    const uint16_t *gh = G + hoff, *qh = Q + hoff;
    uint16_t *oh = dQ + ol.head(bh) + beg * ol.sn;
    const float ntot = n0 + (float)N;

    // store piece of this thread (dQ rows): row it, columns 8 ic .. 8 ic + 7
    const int it = tid / CPR, ic = tid % CPR;
    // staging pieces of the dS waves' threads: rows sr + (0, NT / 2 / CPR),
    // columns 8 ic .. (the same columns for both: NT / 2 is a multiple of CPR)
    const int sr = (tid - NT / 2) / CPR;
    constexpr int SR2 = NT / 2 / CPR;
    float zp[8];  // z at the pieces' columns (loaded by the dS waves)
    // three register sets (set x mod 3 holds round x's pieces): the loads of
    // a round are issued three rounds before it is staged
    uint4 pg[3][2], pq[3][2];
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    // round r's pieces (rounds past the end read nothing: their pieces are zero)
    auto fetch = [&](int r, auto set_) {
        constexpr int X = decltype(set_)::value;
        const int rb = r * TR < len ? r * TR : len;
        const int rows = len - rb < TR ? len - rb : TR;
        const int off = sr * D * 2 + 16 * ic;
        const __amdgpu_buffer_rsrc_t rgs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(gh + (int64_t)rb * D), (short)0, rows * D * 2, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rqs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(qh + (int64_t)rb * D), (short)0, rows * D * 2, kBufferWord3);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            pg[X][p] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rgs, off + p * SR2 * D * 2, 0, 0));
            pq[X][p] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rqs, off + p * SR2 * D * 2, 0, 0));
        }
    };
    // the fetched pieces into LDS: dO and Q as they are, 1 / den of their
    // rows, a = dO / den as hi and lo (rows past the end are zero: a = 0)
    auto stage = [&](int buf, auto set_) {
        constexpr int X = decltype(set_)::value;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int row = sr + p * SR2;
            const int o = row * LDT + 8 * ic;
            *reinterpret_cast<uint4 *>(&L.xs[buf][row * LDX + 8 * ic]) = pg[X][p];
            *reinterpret_cast<uint4 *>(&L.qs[buf][o]) = pq[X][p];
            float qf[8], gf[8];
            StBF16::widen(pq[X][p], qf);
            StBF16::widen(pg[X][p], gf);
            float qz = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                qz += qf[s] * zp[s];
            qz = group_sum<CPR>(qz);
            const float inv = 1.f / (ntot + qz);
            if (ic == 0)
                L.ivx[buf][row] = inv;
            uint4 hi, lo;
            split2(gf[0] * inv, gf[1] * inv, hi.x, lo.x);
            split2(gf[2] * inv, gf[3] * inv, hi.y, lo.y);
            split2(gf[4] * inv, gf[5] * inv, hi.z, lo.z);
            split2(gf[6] * inv, gf[7] * inv, hi.w, lo.w);
            *reinterpret_cast<uint4 *>(&L.ah[buf][o]) = hi;
            *reinterpret_cast<uint4 *>(&L.al[buf][o]) = lo;
        }
    };
    // round rr's dQ rows to global memory (one 16-byte piece per thread;
    // none for rr < 0 or rows past the end)
    auto store_tile = [&](int rr) {
        const int lr = rr * TR + it;
        if (rr >= 0 && lr < len)
            *reinterpret_cast<uint4 *>(oh + lr * ol.sn + 8 * ic) =
                *reinterpret_cast<const uint4 *>(&L.ot[(int)(rr & 1)][it * LDX + 8 * ic]);
    };
    for (int e = tid; e < D; e += NT)
        L.vu[e] = st[D * D + D + e];

    // The rounds are padded to a multiple of three: the padding rounds are
    // past the end (zero rows: no dQ rows, nothing added to dS, r, t).  The
    // loop body is then three rounds of straight-line code, with every load
    // and stage unconditional, so that each stage waits for its own loads
    // only (a branch around a load makes the compiler wait for all of them).
    const int nrounds = (len + TR - 1) / TR;
    const int nr3 = (nrounds + 2) / 3 * 3;
    // (dS waves) the next round into the other buffers from its register
    // set, whose loads are reissued for the round three later
    auto next = [&](int round, auto set_) {
        stage((round + 1) & 1, set_);
        fetch(round + 4, set_);
    };

    float *out = part + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
    if (w < 4) {
        // ---- dQ role: S's block as hi / lo operands,
        // s?[ks][s] = S[32 cb + j][16 ks + 8 h + s]
        bf8 shi[KS], slo[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const f4 v0 = *reinterpret_cast<const f4 *>(st + (32 * cb + j) * D + 16 * ks + 8 * h);
            const f4 v1 =
                *reinterpret_cast<const f4 *>(st + (32 * cb + j) * D + 16 * ks + 8 * h + 4);
            uint4 hi, lo;
            split2(v0[0], v0[1], hi.x, lo.x);
            split2(v0[2], v0[3], hi.y, lo.y);
            split2(v1[0], v1[1], hi.z, lo.z);
            split2(v1[2], v1[3], hi.w, lo.w);
            shi[ks] = __builtin_bit_cast(bf8, hi);
            slo[ks] = __builtin_bit_cast(bf8, lo);
        }
        f4 ez[4];  // z at the lane's output columns 32 cb + 8 q + 4 h ..
#pragma unroll
        for (int q = 0; q < 4; ++q)
            ez[q] = *reinterpret_cast<const f4 *>(st + D * D + 32 * cb + 8 * q + 4 * h);
        // r and t at the lane's output columns, summed over its rows
        float rsum[16], tsum[16];
#pragma unroll
        for (int e = 0; e < 16; ++e)
            rsum[e] = tsum[e] = 0.f;
        __syncthreads();  // the first round staged

        for (int round = 0; round < nr3; ++round) {
            const int buf = round & 1;
            store_tile(round - 2);
            const uint16_t *xr = &L.xs[buf][(32 * rg + j) * LDX];
            f16v acc = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf8 x = *reinterpret_cast<const bf8 *>(xr + 16 * ks + 8 * h);
                acc = mma16(shi[ks], x, acc);
                acc = mma16(slo[ks], x, acc);
            }
            // q.y over this block's output columns, dO.u over the same columns
            const uint16_t *qr = &L.qs[buf][(32 * rg + j) * LDT + 32 * cb + 4 * h];
            const uint16_t *gr = xr + 32 * cb + 4 * h;
            uint2 qv[4], gv[4];
            float p = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                qv[q] = *reinterpret_cast<const uint2 *>(qr + 8 * q);
                gv[q] = *reinterpret_cast<const uint2 *>(gr + 8 * q);
                float qf[4], gf[4];
                StBF16::widen2(qv[q].x, qf);
                StBF16::widen2(qv[q].y, qf + 2);
                StBF16::widen2(gv[q].x, gf);
                StBF16::widen2(gv[q].y, gf + 2);
                const f4 u = *reinterpret_cast<const f4 *>(&L.vu[32 * cb + 8 * q + 4 * h]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p += qf[r] * acc[4 * q + r] + gf[r] * u[r];
            }
            p = swap32_sum(p);
            if (h == 0)
                L.xch[buf][rg][cb][j] = p;
            const float inv = L.ivx[buf][32 * rg + j];
            __syncthreads();
            float sy = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < NCB; ++c2)
                sy += L.xch[buf][rg][c2][j];
            const float c = sy * inv * inv;
            const float cv = (round * TR + 32 * rg + j < len) ? c : 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 o = {acc[4 * q] * inv - c * ez[q][0], acc[4 * q + 1] * inv - c * ez[q][1],
                              acc[4 * q + 2] * inv - c * ez[q][2],
                              acc[4 * q + 3] * inv - c * ez[q][3]};
                uint2 r2;
                r2.x = StBF16::narrow2(o[0], o[1]);
                r2.y = StBF16::narrow2(o[2], o[3]);
                *reinterpret_cast<uint2 *>(
                    &L.ot[buf][(32 * rg + j) * LDX + 32 * cb + 8 * q + 4 * h]) = r2;
                float qf[4], gf[4];
                StBF16::widen2(qv[q].x, qf);
                StBF16::widen2(qv[q].y, qf + 2);
                StBF16::widen2(gv[q].x, gf);
                StBF16::widen2(gv[q].y, gf + 2);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    rsum[4 * q + r] += cv * qf[r];
                    tsum[4 * q + r] += gf[r] * inv;
                }
            }
        }
        // r and t over the wave's rows (the 32 lanes of each half)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float a = group_sum<32>(rsum[e]), b = group_sum<32>(tsum[e]);
            if (j == 0) {
                const int col = 32 * cb + 8 * (e / 4) + 4 * h + (e % 4);
                L.csr[rg][col] = a;
                L.cst[rg][col] = b;
            }
        }
    } else {
        // ---- dS role (and the staging): the first rounds in flight, the
        // first staged; everything any wave loads before the loops is loaded
        // in its own branch, so the loop's waits cover its own loads only
#pragma unroll
        for (int s = 0; s < 8; ++s)
            zp[s] = st[D * D + 8 * ic + s];
        fetch(0, S0{});
        fetch(1, S1{});
        fetch(2, S2{});
        stage(0, S0{});
        fetch(3, S0{});
        __syncthreads();  // the first round staged
        // tiles dS[tm0 + 32 a ..][tn0 + 32 b ..]
        const int tm0 = (w4 / 2) * 32 * TPW1, tn0 = (w4 % 2) * 32 * TPW1;
        f16v dacc[TPW1][TPW1];
#pragma unroll
        for (int a = 0; a < TPW1; ++a)
#pragma unroll
            for (int b = 0; b < TPW1; ++b)
                dacc[a][b] = zero16();
        // body(round, set of round + 1), unrolled over the three sets
        auto body = [&](int round, auto set_) {
            const int buf = round & 1;
            store_tile(round - 2);
#pragma unroll
            for (int kk = 0; kk < TR / 16; ++kk) {
                bf8 av[TPW1], bvh[TPW1], bvl[TPW1];
#pragma unroll
                for (int a = 0; a < TPW1; ++a)
                    av[a] = col8(L.qs[buf], LDT, 16 * kk, tm0 + 32 * a, lane);
#pragma unroll
                for (int b = 0; b < TPW1; ++b) {
                    bvh[b] = col8(L.ah[buf], LDT, 16 * kk, tn0 + 32 * b, lane);
                    bvl[b] = col8(L.al[buf], LDT, 16 * kk, tn0 + 32 * b, lane);
                }
#pragma unroll
                for (int a = 0; a < TPW1; ++a)
#pragma unroll
                    for (int b = 0; b < TPW1; ++b) {
                        dacc[a][b] = mma16(av[a], bvh[b], dacc[a][b]);
                        dacc[a][b] = mma16(av[a], bvl[b], dacc[a][b]);
                    }
            }
            next(round, set_);
            __syncthreads();
        };
        for (int round = 0; round < nr3; round += 3) {
            body(round, S1{});
            body(round + 1, S2{});
            body(round + 2, S0{});
        }
#pragma unroll
        for (int a = 0; a < TPW1; ++a)
#pragma unroll
            for (int b = 0; b < TPW1; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    out[(tm0 + 32 * a + 8 * (i / 4) + 4 * h + (i % 4)) * D + tn0 + 32 * b + j] =
                        dacc[a][b][i];
    }
    __syncthreads();  // the last tiles, r and t
    store_tile(nr3 - 2);
    store_tile(nr3 - 1);
    if (tid < D) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < NRG; ++g2) {
            a += L.csr[g2][tid];
            b += L.cst[g2][tid];
        }
        out[D * D + tid] = a;
        out[D * D + D + tid] = b;
    }
}

// ============================================================ causal
// The causal kernels of la_kernels_causal.hpp on the bf16 matrix cores, same
// chunking (C = 32 rows) and state layout: wave cb holds its D x 32 slice of
// the running state as fp32 accumulators st[t][i] <-> state[32 t + 8 (i/4) +
// 4 h + i % 4][32 cb + j].  For the bf16 MFMA the k-slots of lane (j, h) at
// k-step 2 t + p are taken as accumulator elements 8 p .. 8 p + 7 of st[t],
// i.e. d = 32 t + 16 p + 4 h + {0..3, 8..11}; the state operand is their
// hi/lo bf16 split (re-split every chunk, as the state changes), and the row
// operand is the row's bf16 values at the same d (two 8-byte LDS reads).
// Products over the chunk's tokens (the in-chunk block and the state update)
// read 8 consecutive tokens of a column from transposed LDS tiles.

constexpr int kCc = 32;            // rows per chunk
constexpr int kRT = kCc + 8;       // bf16 pitch of a transposed column

// the 8 bf16 of row r at d = d0 + {0..3, 8..11} (d0 = 32 t + 16 p + 4 h)
__device__ __forceinline__ bf8 row_at(const uint16_t *row, int d0)
{
    const uint2 a = *reinterpret_cast<const uint2 *>(row + d0);
    const uint2 b = *reinterpret_cast<const uint2 *>(row + d0 + 8);
    return __builtin_bit_cast(bf8, uint4{a.x, a.y, b.x, b.y});
}

// hi/lo bf16 operands of accumulator elements 8p .. 8p + 7 of a running
// state.  The residual x - hi of each element is one v_dot2_f32_bf16,
// x + (-1) hi.x + 0 hi.y (or the mirror): the products are exact and the
// residual of a round-to-nearest bf16 is representable in fp32, so it is
// exact, and it replaces an unpack and a subtraction.  Written as one asm
// block because the compiler neither selects this form (it uses the dot2c
// form plus a copy) nor encodes the (-1, 0) operand correctly as a constant
// (its inline constant -1.0 is read as the fp32 pattern, i.e. (0, -1)), and
// because a dot2 result needs three wait states before a VALU reads it,
// which the compiler does not insert after inline asm: the order below
// leaves at least three instructions between every dot2 and its reader,
// and two wait states after the last conversion (an MFMA may read it next).
// The inputs must not be fresh MFMA results (the compiler does not insert
// the MFMA-to-VALU wait states before inline asm either): here they are
// state accumulators last updated a whole chunk earlier.
__device__ __forceinline__ void split8(const f16v &a, int p, bf8 &hi, bf8 &lo)
{
    uint32_t m0, m1;
    asm("v_mov_b32 %0, 0xbf80" : "=v"(m0));      // (-1, 0)
    asm("v_mov_b32 %0, 0xbf800000" : "=v"(m1));  // (0, -1)
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    float r0, r1, r2, r3, r4, r5, r6, r7;
    asm("v_cvt_pk_bf16_f32 %0, %16, %17\n\t"
        "v_cvt_pk_bf16_f32 %1, %18, %19\n\t"
        "v_cvt_pk_bf16_f32 %2, %20, %21\n\t"
        "v_cvt_pk_bf16_f32 %3, %22, %23\n\t"
        "v_dot2_f32_bf16 %8, %0, %24, %16\n\t"
        "v_dot2_f32_bf16 %9, %0, %25, %17\n\t"
        "v_dot2_f32_bf16 %10, %1, %24, %18\n\t"
        "v_dot2_f32_bf16 %11, %1, %25, %19\n\t"
        "v_dot2_f32_bf16 %12, %2, %24, %20\n\t"
        "v_dot2_f32_bf16 %13, %2, %25, %21\n\t"
        "v_dot2_f32_bf16 %14, %3, %24, %22\n\t"
        "v_dot2_f32_bf16 %15, %3, %25, %23\n\t"
        "v_cvt_pk_bf16_f32 %4, %8, %9\n\t"
        "v_cvt_pk_bf16_f32 %5, %10, %11\n\t"
        "v_cvt_pk_bf16_f32 %6, %12, %13\n\t"
        "v_cvt_pk_bf16_f32 %7, %14, %15\n\t"
        "s_nop 1"
        : "=&v"(h0), "=&v"(h1), "=&v"(h2), "=&v"(h3), "=&v"(l0), "=&v"(l1), "=&v"(l2),
          "=&v"(l3), "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5),
          "=&v"(r6), "=&v"(r7)
        : "v"(a[8 * p]), "v"(a[8 * p + 1]), "v"(a[8 * p + 2]), "v"(a[8 * p + 3]),
          "v"(a[8 * p + 4]), "v"(a[8 * p + 5]), "v"(a[8 * p + 6]), "v"(a[8 * p + 7]), "v"(m0),
          "v"(m1));
    hi = __builtin_bit_cast(bf8, uint4{h0, h1, h2, h3});
    lo = __builtin_bit_cast(bf8, uint4{l0, l1, l2, l3});
}

// Staging of one chunk: item q = tid (+ NT) covers token pair pr = q % 16
// and 8-column chunk q / 16; loads two 16-byte pieces through a descriptor
// limited to the chunk's valid rows (zeros past the end).
template <int D, int NT>
struct ChunkRows {
    static constexpr int CH = D / 8;
    static constexpr int PC = (kCc / 2) * CH;
    static constexpr int PER = (PC + NT - 1) / NT;
    static constexpr int LDX = D + 8;  // bf16 pitch of a natural row
    uint4 r[PER][2];

    __device__ __forceinline__ void fetch(const uint16_t *src, int64_t r0, int64_t end, int tid)
    {
        const int rows = (int)(end - r0 < kCc ? end - r0 : kCc);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(src + r0 * D), (short)0, rows * D * 2, kBufferWord3);
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int q = tid + p * NT;
            if (PC % NT == 0 || q < PC) {
                const int chunk = q / (kCc / 2), pr = q % (kCc / 2);
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    r[p][u] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                   rs, (2 * pr + u) * D * 2 + 16 * chunk, 0, 0));
            }
        }
    }
    // natural rows [token][d]
    __device__ __forceinline__ void stage_nat(uint16_t *lds, int tid) const
    {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int q = tid + p * NT;
            if (PC % NT == 0 || q < PC) {
                const int chunk = q / (kCc / 2), pr = q % (kCc / 2);
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    *reinterpret_cast<uint4 *>(&lds[(2 * pr + u) * LDX + 8 * chunk]) = r[p][u];
            }
        }
    }
    // transposed [d][token], tokens 2 pr, 2 pr + 1 packed per 32-bit write
    __device__ __forceinline__ void stage_tr(uint16_t *lds, int tid) const
    {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int q = tid + p * NT;
            if (PC % NT == 0 || q < PC) {
                const int chunk = q / (kCc / 2), pr = q % (kCc / 2);
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    *reinterpret_cast<uint32_t *>(&lds[(8 * chunk + s) * kRT + 2 * pr]) =
                        pair_bf16(r[p][0], r[p][1], s);
            }
        }
    }
};

// (c_t, 1/den_t) of a chunk's rows for the staging items: item q covers
// tokens 2 (q % 16) and 2 (q % 16) + 1; rows past the end read as zeros
template <int D, int NT>
struct ChunkCb {
    static constexpr int PER = ChunkRows<D, NT>::PER, PC = ChunkRows<D, NT>::PC;
    float2 r[PER][2];
    __device__ __forceinline__ void fetch(const float2 *src, int64_t r0, int64_t end, int tid)
    {
        const int rows = (int)(end - r0 < kCc ? end - r0 : kCc);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float2 *>(src + r0), (short)0, rows * 8, kBufferWord3);
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int q = tid + p * NT;
            if (PC % NT == 0 || q < PC) {
                const int pr = q % (kCc / 2);
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    r[p][u] = __builtin_bit_cast(
                        float2, __builtin_amdgcn_raw_buffer_load_b64(rs, (2 * pr + u) * 8, 0, 0));
            }
        }
    }
};

// a_t = g_t / den_t of the staged dO rows, transposed, as hi and lo planes
template <int D, int NT>
__device__ __forceinline__ void stage_a_tr(const ChunkRows<D, NT> &rg, const ChunkCb<D, NT> &cb,
                                           uint16_t *hiT, uint16_t *loT, int tid)
{
    typedef ChunkRows<D, NT> R;
#pragma unroll
    for (int p = 0; p < R::PER; ++p) {
        const int q = tid + p * NT;
        if (R::PC % NT == 0 || q < R::PC) {
            const int chunk = q / (kCc / 2), pr = q % (kCc / 2);
            float g0[8], g1[8];
            StBF16::widen(rg.r[p][0], g0);
            StBF16::widen(rg.r[p][1], g1);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                // tokens 2 pr, 2 pr + 1 of column 8 chunk + s: hi and lo pairs
                const float a0 = g0[s] * cb.r[p][0].y, a1 = g1[s] * cb.r[p][1].y;
                const bf2 hv = {(__bf16)a0, (__bf16)a1};
                const uint32_t hw = __builtin_bit_cast(uint32_t, hv);
                const bf2 lv = {(__bf16)(a0 - __uint_as_float(hw << 16)),
                                (__bf16)(a1 - __uint_as_float(hw & 0xffff0000u))};
                *reinterpret_cast<uint32_t *>(&hiT[(8 * chunk + s) * kRT + 2 * pr]) = hw;
                *reinterpret_cast<uint32_t *>(&loT[(8 * chunk + s) * kRT + 2 * pr]) =
                    __builtin_bit_cast(uint32_t, lv);
            }
        }
    }
}

// One row's 32 output columns held by lanes (j, 0) and (j, 1) (lane h:
// columns 8 q + 4 h + 0..3 in v[q]) stored as bf16 in two 16-byte pieces per
// lane: a permlane32 swap per dword pair (q = 2 s, 2 s + 1) leaves lane h
// with columns 16 s + 8 h .. + 7 (h = 0: its own q = 2 s and the partner's;
// h = 1: the partner's q = 2 s + 1 and its own).  Every lane runs the swaps;
// ok guards the stores.
__device__ __forceinline__ void store_row32(uint16_t *p, const f4 *v, int h, bool ok)
{
    uint32_t w[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        w[q][0] = StBF16::narrow2(v[q][0], v[q][1]);
        w[q][1] = StBF16::narrow2(v[q][2], v[q][3]);
    }
    uint32_t o[2][4];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const auto r = __builtin_amdgcn_permlane32_swap(w[2 * s2][e], w[2 * s2 + 1][e], false,
                                                            false);
            o[s2][e] = (uint32_t)r[0];
            o[s2][2 + e] = (uint32_t)r[1];
        }
    if (ok) {
        *reinterpret_cast<uint4 *>(p + 8 * h) = uint4{o[0][0], o[0][1], o[0][2], o[0][3]};
        *reinterpret_cast<uint4 *>(p + 16 + 8 * h) = uint4{o[1][0], o[1][1], o[1][2], o[1][3]};
    }
}

// 8 consecutive tokens (16 kk + 8 h ..) of column c of a transposed tile
__device__ __forceinline__ bf8 col_at(const uint16_t *ldsT, int c, int kk, int h)
{
    return *reinterpret_cast<const bf8 *>(&ldsT[c * kRT + 16 * kk + 8 * h]);
}

// X_c Y_c^T over all D columns (natural rows), written to sh[i * (kCc + 1) +
// jj] by one wave: on the bf16 matrix cores the whole 32 x 32 block is D/16
// MFMAs, cheaper than exchanging per-wave shares through LDS
template <int D>
__device__ __forceinline__ void full_bf(const uint16_t *xs, const uint16_t *ys, float *sh,
                                        int j, int h)
{
    constexpr int LDX = D + 8, WP = kCc + 1;
    f16v a = zero16();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const bf8 x = *reinterpret_cast<const bf8 *>(&xs[j * LDX + 16 * ks + 8 * h]);
        const bf8 y = *reinterpret_cast<const bf8 *>(&ys[j * LDX + 16 * ks + 8 * h]);
        a = mma16(x, y, a);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e)
        sh[(8 * (e / 4) + 4 * h + (e % 4)) * WP + j] = a[e];
}

constexpr int kWP = kCc + 8;  // bf16 pitch of a [row][key] plane of a chunk

// W = M o (1 + Q_c K_c^T) of a chunk, quarter qd (rows 16 (qd / 2) ..,
// keys 16 (qd % 2) ..), as hi / lo bf16 planes [row][key] (pitch kWP) and
// its row sums over the quarter's keys (rsx[(qd % 2) kCc + row]).  The
// quarter is one product K_blk Q_blk^T on v_mfma_f32_16x16x32_bf16 (lane l
// supplies key / row l % 16 and columns 8 (l / 16) .. + 7 of each 32-column
// step, and receives keys 4 (l / 16) + 0..3 of row l % 16); the quarter
// above the diagonal is all zero and skips the product.
template <int D>
__device__ __forceinline__ void w_quarter(const uint16_t *qs, const uint16_t *ks, uint16_t *whi,
                                          uint16_t *wlo, float *rsx, int qd, int lane)
{
    constexpr int LDX = D + 8;
    const int rb0 = 16 * (qd >> 1), kb0 = 16 * (qd & 1);
    const int r = lane & 15, g = lane >> 4;
    f4 t = {0.f, 0.f, 0.f, 0.f};
    if (kb0 <= rb0) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            const bf8 a = *reinterpret_cast<const bf8 *>(&ks[(kb0 + r) * LDX + 32 * s + 8 * g]);
            const bf8 b = *reinterpret_cast<const bf8 *>(&qs[(rb0 + r) * LDX + 32 * s + 8 * g]);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, t, 0, 0, 0);
        }
    }
    const int row = rb0 + r, k0 = kb0 + 4 * g;
    float w[4], sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[i] = (k0 + i <= row) ? 1.f + t[i] : 0.f;
        sum += w[i];
    }
    uint2 hi, lo;
    split4(w[0], w[1], w[2], w[3], hi, lo);
    *reinterpret_cast<uint2 *>(&whi[row * kWP + k0]) = hi;
    *reinterpret_cast<uint2 *>(&wlo[row * kWP + k0]) = lo;
    sum = swap32_sum(swap16_sum(sum));
    if (g == 0)
        rsx[(qd & 1) * kCc + row] = sum;
}

// Forward (as cz::k_fwd_causal): per chunk (1) acc = S^T-block . Q_c^T and
// q.z; (2) the waves' quarters of W = M o (1 + Q_c K_c^T) as hi / lo planes,
// with their row sums; barrier; (3) acc += V_c-block^T . W^T (the row sums
// go to den), st += K_c^T . V_c-block; (4) normalised rows.
template <int D>
__global__ __launch_bounds__(64 * (D / 32)) void k_fwd_causal_bf(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ den_out,
    const float *__restrict__ rec, int64_t N, int64_t seg_len, int nseg, float n0, OutLay ol)
{
    typedef nc::IO<StBF16> io;
    static_assert(D >= 32 && D <= 128, "32-column blocks, state in registers");
    constexpr int NCB = D / 32, NT = 64 * NCB, LDX = D + 8;
    __shared__ __attribute__((aligned(16))) uint16_t qs[kCc * LDX];
    __shared__ __attribute__((aligned(16))) uint16_t ks[kCc * LDX];
    __shared__ __attribute__((aligned(16))) uint16_t kT[D * kRT];
    __shared__ __attribute__((aligned(16))) uint16_t vT[D * kRT];
    __shared__ __attribute__((aligned(16))) uint16_t whi[kCc * kWP];  // W, [row][key]
    __shared__ __attribute__((aligned(16))) uint16_t wlo[kCc * kWP];
    __shared__ float rsx[2 * kCc];   // row sums of W by key half
    __shared__ float qzx[NCB][kCc];  // q.z over each wave's 32 columns
    __shared__ __attribute__((aligned(16))) float vz[D];
    __shared__ __attribute__((aligned(16))) float vu[D];

    const int64_t bh = blockIdx.x / nseg;
    const int seg = (int)(blockIdx.x % nseg);
    const int tid = threadIdx.x, cb = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
    const uint16_t *qh = Q + hoff, *kh = K + hoff, *vh = V + hoff;
    uint16_t *oh = O + ol.head(bh);

    ChunkRows<D, NT> rq, rk, rv;
    const int64_t nrounds = (end - beg + kCc - 1) / kCc;
    rq.fetch(qh, beg, end, tid);
    rk.fetch(kh, beg, end, tid);
    rv.fetch(vh, beg, end, tid);
    f16v sacc[NCB];
#pragma unroll
    for (int t = 0; t < NCB; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            sacc[t][i] = st[(32 * t + 8 * (i / 4) + 4 * h + (i % 4)) * D + 32 * cb + j];
    for (int e = tid; e < D; e += NT) {
        vz[e] = st[D * D + e];
        vu[e] = st[D * D + D + e];
    }
    rq.stage_nat(qs, tid);
    rk.stage_nat(ks, tid);
    rk.stage_tr(kT, tid);
    rv.stage_tr(vT, tid);
    drain_loads();
    if (nrounds > 1)
        rq.fetch(qh, beg + kCc, end, tid);
    __syncthreads();

    f4 pend[4];
    int64_t prow = 0;
    bool pok = false;
    auto store_pending = [&]() { store_row32(oh + prow * ol.sn + 32 * cb, pend, h, pok); };

    for (int64_t round = 0; round < nrounds; ++round) {
        const int64_t t0 = beg + round * kCc;
        const bool more = round + 1 < nrounds;
        // (1) the prefix state applied to the chunk's queries, and q.z over
        // this wave's 32 columns (the partials meet in LDS at B1)
        f16v acc = zero16();
        {
            const uint16_t *qrow = &qs[j * LDX];
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < 16; e += 8) {
                float xf[8];
                unpack8(*reinterpret_cast<const bf8 *>(qrow + 32 * cb + 16 * h + e), xf);
                const float *zr = &vz[32 * cb + 16 * h + e];
                p += dot4(f4{xf[0], xf[1], xf[2], xf[3]}, *reinterpret_cast<const f4 *>(zr)) +
                     dot4(f4{xf[4], xf[5], xf[6], xf[7]}, *reinterpret_cast<const f4 *>(zr + 4));
            }
            p = swap32_sum(p);
            if (h == 0)
                qzx[cb][j] = p;
#pragma unroll
            for (int t = 0; t < NCB; ++t)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int d0 = 32 * t + 16 * p;
                    const bf8 x = row_at(qrow, d0 + 4 * h);
                    bf8 ahi, alo;
                    split8(sacc[t], p, ahi, alo);
                    acc = mma16(ahi, x, acc);
                    acc = mma16(alo, x, acc);
                    if (t == 0 && p == 0)
                        store_pending();
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        // (2) this wave's quarters of W
        for (int qd = cb; qd < 4; qd += NCB)
            w_quarter<D>(qs, ks, whi, wlo, rsx, qd, lane);
        __syncthreads();  // B1
        if (more)
            rq.stage_nat(qs, tid);  // Q is read only before B1
        if (more) {
            rk.fetch(kh, t0 + kCc, end, tid);
            rv.fetch(vh, t0 + kCc, end, tid);
        }
        // (3) in-chunk term over key rows 16 kk + 8 h .. and the state update
        float zc = 0.f, uc = 0.f;
#pragma unroll
        for (int kk = 0; kk < kCc / 16; ++kk) {
            // W[j][16 kk + 8 h ..]
            const bf8 wh = *reinterpret_cast<const bf8 *>(&whi[j * kWP + 16 * kk + 8 * h]);
            const bf8 wl = *reinterpret_cast<const bf8 *>(&wlo[j * kWP + 16 * kk + 8 * h]);
            const bf8 vcol = col_at(vT, 32 * cb + j, kk, h);  // V[16kk+8h..][32cb+j]
            acc = mma16(vcol, wh, acc);
            acc = mma16(vcol, wl, acc);
#pragma unroll
            for (int t = 0; t < NCB; ++t)
                sacc[t] = mma16(col_at(kT, 32 * t + j, kk, h), vcol, sacc[t]);
            // (this wave's K column read again: selecting it among the
            // unrolled operands would cost a sum per block)
            zc = sum8(col_at(kT, 32 * cb + j, kk, h), zc);
            uc = sum8(vcol, uc);
            __builtin_amdgcn_sched_barrier(0);
        }
        zc = swap32_sum(zc);
        uc = swap32_sum(uc);
        const float rs = rsx[j] + rsx[kCc + j];
        float qz = 0.f;
#pragma unroll
        for (int c2 = 0; c2 < NCB; ++c2)
            qz += qzx[c2][j];
        // (4) normalised rows of the chunk, stored during the next product
        const float den = (n0 + (float)t0) + qz + rs;
        const float inv = 1.f / den;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f4 u = *reinterpret_cast<const f4 *>(&vu[32 * cb + 8 * q + 4 * h]);
            pend[q] = f4{(acc[4 * q] + u[0]) * inv, (acc[4 * q + 1] + u[1]) * inv,
                         (acc[4 * q + 2] + u[2]) * inv, (acc[4 * q + 3] + u[3]) * inv};
        }
        prow = t0 + j;
        pok = prow < end;
        if (den_out != nullptr && pok && h == 0 && cb == 0)
            den_out[bh * N + prow] = den;
        __syncthreads();  // B2
        if (h == 0) {
            vz[32 * cb + j] += zc;
            vu[32 * cb + j] += uc;
        }
        if (more) {
            rk.stage_nat(ks, tid);
            rk.stage_tr(kT, tid);
            rv.stage_tr(vT, tid);
            if (round + 2 < nrounds)
                rq.fetch(qh, t0 + 2 * kCc, end, tid);
        }
        __syncthreads();  // B3
    }
    store_pending();
}

// The dQ pass's in-chunk blocks, quarter qd (as w_quarter): W = 1 + Q_c K_c^T
// and GV = G_c V_c^T under the mask M, the masked GV as hi / lo planes
// [row][key], and the row sums over the quarter's keys of W (rsx) and of
// W o GV (cwx), both at [(qd % 2) kCc + row].
template <int D>
__device__ __forceinline__ void wg_quarter(const uint16_t *qs, const uint16_t *ks,
                                           const uint16_t *gs, const uint16_t *vs, uint16_t *ghi,
                                           uint16_t *glo, float *rsx, float *cwx, int qd,
                                           int lane)
{
    constexpr int LDX = D + 8;
    const int rb0 = 16 * (qd >> 1), kb0 = 16 * (qd & 1);
    const int r = lane & 15, g = lane >> 4;
    f4 tw = {0.f, 0.f, 0.f, 0.f}, tg = {0.f, 0.f, 0.f, 0.f};
    if (kb0 <= rb0) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            const int ok = (kb0 + r) * LDX + 32 * s + 8 * g, orw = (rb0 + r) * LDX + 32 * s + 8 * g;
            tw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf8 *>(&ks[ok]),
                                                         *reinterpret_cast<const bf8 *>(&qs[orw]),
                                                         tw, 0, 0, 0);
            tg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf8 *>(&vs[ok]),
                                                         *reinterpret_cast<const bf8 *>(&gs[orw]),
                                                         tg, 0, 0, 0);
        }
    }
    const int row = rb0 + r, k0 = kb0 + 4 * g;
    float gm[4], rs = 0.f, cw = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool m = k0 + i <= row;
        const float w = m ? 1.f + tw[i] : 0.f;
        gm[i] = m ? tg[i] : 0.f;
        rs += w;
        cw += w * gm[i];
    }
    uint2 hi, lo;
    split4(gm[0], gm[1], gm[2], gm[3], hi, lo);
    *reinterpret_cast<uint2 *>(&ghi[row * kWP + k0]) = hi;
    *reinterpret_cast<uint2 *>(&glo[row * kWP + k0]) = lo;
    rs = swap32_sum(swap16_sum(rs));
    cw = swap32_sum(swap16_sum(cw));
    if (g == 0) {
        rsx[(qd & 1) * kCc + row] = rs;
        cwx[(qd & 1) * kCc + row] = cw;
    }
}

// dQ (as cz::k_bwd_q_causal): st[t] = S^T[32t.., 32cb..]; per chunk
// (1) acc = S-block . G_c^T with g.u and q.z; (2) the waves' quarters of the
// in-chunk blocks (wg_quarter), q.y over the wave's columns; barrier; (3)
// den, c, then acc += K_c-block^T . P^T with P = M o GV - c den M, formed as
// two products, K^T (M o GV)^T - c den K^T M^T (M exact in bf16), and st +=
// V_c^T . K_c-block; (4) dq rows and cbuf = (c, 1/den).
template <int D>
__global__ __launch_bounds__(64 * (D / 32)) void k_bwd_q_causal_bf(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ G, uint16_t *__restrict__ dQ,
    float *__restrict__ cbuf, const float *__restrict__ rec, int64_t N, int64_t seg_len,
    int nseg, float n0, OutLay ol)
{
    typedef nc::IO<StBF16> io;
    static_assert(D >= 32 && D <= 128, "32-column blocks, state in registers");
    constexpr int NCB = D / 32, NT = 64 * NCB, LDX = D + 8;
    __shared__ __attribute__((aligned(16))) uint16_t qs[kCc * LDX];
    __shared__ __attribute__((aligned(16))) uint16_t gs[kCc * LDX];
    __shared__ __attribute__((aligned(16))) uint16_t ks[kCc * LDX];
    __shared__ __attribute__((aligned(16))) uint16_t vs[kCc * LDX];
    __shared__ __attribute__((aligned(16))) uint16_t kT[D * kRT];
    __shared__ __attribute__((aligned(16))) uint16_t vT[D * kRT];
    __shared__ __attribute__((aligned(16))) uint16_t ghi[kCc * kWP];  // M o GV, [row][key]
    __shared__ __attribute__((aligned(16))) uint16_t glo[kCc * kWP];
    __shared__ float rsx[2 * kCc];       // row sums of W by key half
    __shared__ float cwx[2 * kCc];       // row sums of W o GV by key half
    __shared__ float xq[NCB][kCc];       // shares of q_i.y_i + g_i.u
    __shared__ float xz[NCB][kCc];       // shares of q_i.z
    __shared__ __attribute__((aligned(16))) float vz[D];
    __shared__ __attribute__((aligned(16))) float vu[D];

    const int64_t bh = blockIdx.x / nseg;
    const int seg = (int)(blockIdx.x % nseg);
    const int tid = threadIdx.x, cb = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
    const uint16_t *qh = Q + hoff, *kh = K + hoff, *vh = V + hoff, *gh = G + hoff;
    uint16_t *oh = dQ + ol.head(bh);

    ChunkRows<D, NT> rq, rg, rk, rv;
    const int64_t nrounds = (end - beg + kCc - 1) / kCc;
    rq.fetch(qh, beg, end, tid);
    rg.fetch(gh, beg, end, tid);
    rk.fetch(kh, beg, end, tid);
    rv.fetch(vh, beg, end, tid);
    // sacc[t][4q + r] = S[32cb + j][32t + 8q + 4h + r]
    f16v sacc[NCB];
#pragma unroll
    for (int t = 0; t < NCB; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f4 v = *reinterpret_cast<const f4 *>(st + (32 * cb + j) * D + 32 * t + 8 * q +
                                                       4 * h);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[t][4 * q + r] = v[r];
        }
    for (int e = tid; e < D; e += NT) {
        vz[e] = st[D * D + e];
        vu[e] = st[D * D + D + e];
    }
    rq.stage_nat(qs, tid);
    rg.stage_nat(gs, tid);
    rk.stage_nat(ks, tid);
    rk.stage_tr(kT, tid);
    rv.stage_nat(vs, tid);
    rv.stage_tr(vT, tid);
    drain_loads();
    if (nrounds > 1) {
        rq.fetch(qh, beg + kCc, end, tid);
        rg.fetch(gh, beg + kCc, end, tid);
    }
    __syncthreads();

    f4 pend[4];
    int64_t prow = 0;
    bool pok = false;
    auto store_pending = [&]() { store_row32(oh + prow * ol.sn + 32 * cb, pend, h, pok); };

    for (int64_t round = 0; round < nrounds; ++round) {
        const int64_t t0 = beg + round * kCc;
        const bool more = round + 1 < nrounds;
        // (1) y = S g for the chunk's rows; g.u and q.z over this wave's 32
        // columns (the shares meet in LDS at B1)
        f16v acc = zero16();
        float gu = 0.f, qz = 0.f;
        {
            const uint16_t *grow = &gs[j * LDX], *qrow = &qs[j * LDX];
#pragma unroll
            for (int e = 0; e < 16; e += 8) {
                const int d = 32 * cb + 16 * h + e;
                float xf[8], qf[8];
                unpack8(*reinterpret_cast<const bf8 *>(grow + d), xf);
                unpack8(*reinterpret_cast<const bf8 *>(qrow + d), qf);
                gu += dot4(f4{xf[0], xf[1], xf[2], xf[3]}, *reinterpret_cast<const f4 *>(&vu[d])) +
                      dot4(f4{xf[4], xf[5], xf[6], xf[7]}, *reinterpret_cast<const f4 *>(&vu[d + 4]));
                qz += dot4(f4{qf[0], qf[1], qf[2], qf[3]}, *reinterpret_cast<const f4 *>(&vz[d])) +
                      dot4(f4{qf[4], qf[5], qf[6], qf[7]}, *reinterpret_cast<const f4 *>(&vz[d + 4]));
            }
#pragma unroll
            for (int t = 0; t < NCB; ++t)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int d0 = 32 * t + 16 * p;
                    const bf8 x = row_at(grow, d0 + 4 * h);
                    bf8 ahi, alo;
                    split8(sacc[t], p, ahi, alo);
                    acc = mma16(ahi, x, acc);
                    acc = mma16(alo, x, acc);
                    if (t == 0 && p == 0)
                        store_pending();
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        // (2) this wave's quarters of the in-chunk blocks, q.y over this
        // wave's columns
        for (int qd = cb; qd < 4; qd += NCB)
            wg_quarter<D>(qs, ks, gs, vs, ghi, glo, rsx, cwx, qd, lane);
        {
            const uint16_t *qr = &qs[j * LDX + 32 * cb + 4 * h];
            float pq = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint2 u = *reinterpret_cast<const uint2 *>(qr + 8 * q);
                pq += __uint_as_float(u.x << 16) * acc[4 * q] +
                      __uint_as_float(u.x & 0xffff0000u) * acc[4 * q + 1] +
                      __uint_as_float(u.y << 16) * acc[4 * q + 2] +
                      __uint_as_float(u.y & 0xffff0000u) * acc[4 * q + 3];
            }
            pq += gu;
            pq = swap32_sum(pq);
            qz = swap32_sum(qz);
            if (h == 0) {
                xq[cb][j] = pq;
                xz[cb][j] = qz;
            }
        }
        __syncthreads();  // B1
        if (more) {
            rq.stage_nat(qs, tid);  // Q and dO are read only before B1
            rg.stage_nat(gs, tid);
            rk.fetch(kh, t0 + kCc, end, tid);
            rv.fetch(vh, t0 + kCc, end, tid);
        }
        // (3) den and c of row j, then the in-chunk term and the update over
        // key rows 16 kk + 8 h + s
        const float rs = rsx[j] + rsx[kCc + j], cw = cwx[j] + cwx[kCc + j];
        float qyu = 0.f, qzs = 0.f;  // q.y + g.u and q.z over all columns
#pragma unroll
        for (int pp = 0; pp < NCB; ++pp) {
            qyu += xq[pp][j];
            qzs += xz[pp][j];
        }
        const float den = (n0 + (float)t0) + qzs + rs;
        const float inv = 1.f / den;
        const float c = (qyu + cw) * inv * inv;
        const float cden = c * den;
        float zc = 0.f, uc = 0.f;
        f16v kcum = zero16();  // K^T M^T: sums of K over the keys up to row j
#pragma unroll
        for (int kk = 0; kk < kCc / 16; ++kk) {
            const bf8 gh = *reinterpret_cast<const bf8 *>(&ghi[j * kWP + 16 * kk + 8 * h]);
            const bf8 gl = *reinterpret_cast<const bf8 *>(&glo[j * kWP + 16 * kk + 8 * h]);
            bf8 mk;
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2)
                mk[s2] = (16 * kk + 8 * h + s2 <= j) ? (__bf16)1.f : (__bf16)0.f;
            const bf8 kcol = col_at(kT, 32 * cb + j, kk, h);  // K[16kk+8h..][32cb+j]
            acc = mma16(kcol, gh, acc);
            acc = mma16(kcol, gl, acc);
            kcum = mma16(kcol, mk, kcum);
#pragma unroll
            for (int t = 0; t < NCB; ++t)
                sacc[t] = mma16(col_at(vT, 32 * t + j, kk, h), kcol, sacc[t]);
            uc = sum8(col_at(vT, 32 * cb + j, kk, h), uc);  // (as in the forward)
            zc = sum8(kcol, zc);
            __builtin_amdgcn_sched_barrier(0);
        }
        zc = swap32_sum(zc);
        uc = swap32_sum(uc);
        // (4) dq rows (z of the rows before the chunk)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f4 z = *reinterpret_cast<const f4 *>(&vz[32 * cb + 8 * q + 4 * h]);
            f4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                o[r] = (acc[4 * q + r] - cden * kcum[4 * q + r]) * inv - c * z[r];
            pend[q] = o;
        }
        prow = t0 + j;
        pok = prow < end;
        if (pok && h == 0 && cb == 0)
            reinterpret_cast<float2 *>(cbuf)[bh * N + prow] = float2{c, inv};
        __syncthreads();  // B2
        if (h == 0) {
            vz[32 * cb + j] += zc;
            vu[32 * cb + j] += uc;
        }
        if (more) {
            rk.stage_nat(ks, tid);
            rk.stage_tr(kT, tid);
            rv.stage_nat(vs, tid);
            rv.stage_tr(vT, tid);
            if (round + 2 < nrounds) {
                rq.fetch(qh, t0 + 2 * kCc, end, tid);
                rg.fetch(gh, t0 + 2 * kCc, end, tid);
            }
        }
        __syncthreads();  // B3
    }
    store_pending();
}

// dK | dV (as cz::k_bwd_kv_causal), chunks in reverse order with the running
// suffix state (R, r, t).  Parity 0 (dK): st[t] = R^T[32t.., 32cb..];
// acc = R-block . V_c^T + Q_c-block^T . P with P[i][j] = g_i.v_j / den_i -
// c_i (i >= j), from shares of G_c V_c^T; R += Q_c^T A_c.  Parity 1 (dV):
// st[t] = R[32t.., 32cb..]; acc = R^T-block . K_c^T + A_c-block^T . W with
// W[i][j] = 1 + q_i.k_j (i >= j), from shares of Q_c K_c^T.  A_c = G_c /
// den is formed at staging as transposed hi/lo planes.
template <int D>
struct KvBfLds {
    static constexpr int LDX = D + 8, WP = kCc + 1, NCB = D / 32;
    uint16_t xs[kCc * LDX];  // V (dK) or K (dV), natural
    uint16_t ys[kCc * LDX];  // dO (dK) or Q (dV), natural
    uint16_t qT[D * kRT];
    uint16_t aT[2][D * kRT];  // a = dO / den, hi and lo
    float sh[kCc * WP];
    float cs[kCc], is[kCc];
    float vr[D];  // r (dK) or t (dV)
};

template <int D, int PAR>
__device__ __forceinline__ void kv_pass_bf(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ G, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, const float *__restrict__ cbuf, const float *__restrict__ rec,
    int64_t N, int64_t seg_len, int nseg, OutLay ol, KvBfLds<D> &L)
{
    typedef nc::IO<StBF16> io;
    constexpr int NCB = D / 32, NT = 64 * NCB, LDX = D + 8, WP = kCc + 1;
    const int64_t b = blockIdx.x >> 1;
    const int64_t bh = b / nseg;
    const int seg = (int)(b % nseg);
    const int tid = threadIdx.x, cb = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
    const uint16_t *xh = (PAR == 0 ? V : K) + hoff, *qh = Q + hoff, *gh = G + hoff;
    uint16_t *oh = (PAR == 0 ? dK : dV) + ol.head(bh);
    const float2 *ch = reinterpret_cast<const float2 *>(cbuf) + bh * N;

    ChunkRows<D, NT> rx, rq, rg;
    ChunkCb<D, NT> rc;
    auto fetch = [&](int64_t r0) {
        rx.fetch(xh, r0, end, tid);
        rq.fetch(qh, r0, end, tid);
        rg.fetch(gh, r0, end, tid);
        rc.fetch(ch, r0, end, tid);
    };
    auto stage = [&](int64_t r0) {
        rx.stage_nat(L.xs, tid);
        if (PAR == 0)
            rg.stage_nat(L.ys, tid);
        else
            rq.stage_nat(L.ys, tid);
        rq.stage_tr(L.qT, tid);
        stage_a_tr<D, NT>(rg, rc, L.aT[0], L.aT[1], tid);
        // (c, 1/den) of the chunk's rows
        if (tid < kCc) {
            const bool ok = r0 + tid < end;
            const float2 v = ok ? ch[r0 + tid] : float2{0.f, 0.f};
            L.cs[tid] = v.x;
            L.is[tid] = v.y;
        }
    };

    const int64_t nrounds = (end - beg + kCc - 1) / kCc;
    const int64_t last = beg + (nrounds - 1) * kCc;
    fetch(last);
    f16v sacc[NCB];
#pragma unroll
    for (int t = 0; t < NCB; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int a = 32 * t + 8 * (i / 4) + 4 * h + (i % 4), o = 32 * cb + j;
            sacc[t][i] = (PAR == 0) ? st[o * D + a] : st[a * D + o];
        }
    for (int e = tid; e < D; e += NT)
        L.vr[e] = st[D * D + (PAR == 0 ? 0 : D) + e];
    stage(last);
    drain_loads();
    if (nrounds > 1)
        fetch(last - kCc);
    __syncthreads();

    for (int64_t round = 0; round < nrounds; ++round) {
        const int64_t t0 = last - round * kCc;
        // (1) the suffix state applied to the chunk's rows of V (dK) or K (dV)
        f16v acc = zero16();
        {
            const uint16_t *xrow = &L.xs[j * LDX];
#pragma unroll
            for (int t = 0; t < NCB; ++t)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const bf8 x = row_at(xrow, 32 * t + 16 * p + 4 * h);
                    bf8 ahi, alo;
                    split8(sacc[t], p, ahi, alo);
                    acc = mma16(ahi, x, acc);
                    acc = mma16(alo, x, acc);
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        // (2) G_c V_c^T (dK) or Q_c K_c^T (dV), one wave
        if (cb == 0)
            full_bf<D>(L.ys, L.xs, L.sh, j, h);
        __syncthreads();  // B1
        // (3) in-chunk term over query rows ir = 16 kk + 8 h + s >= j, and the
        // state update
        float vc = 0.f;
#pragma unroll
        for (int kk = 0; kk < kCc / 16; ++kk) {
            float bm[8];
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2) {
                const int ir = 16 * kk + 8 * h + s2;
                const float sv = L.sh[ir * WP + j];
                if (PAR == 0)
                    bm[s2] = (ir >= j) ? sv * L.is[ir] - L.cs[ir] : 0.f;
                else
                    bm[s2] = (ir >= j) ? 1.f + sv : 0.f;
            }
            bf8 bhi, blo;
            split8v(bm, bhi, blo);
            if constexpr (PAR == 0) {
                const bf8 qcol = col_at(L.qT, 32 * cb + j, kk, h);  // Q[ir][32cb+j]
                acc = mma16(qcol, bhi, acc);
                acc = mma16(qcol, blo, acc);
#pragma unroll
                for (int t = 0; t < NCB; ++t) {
                    sacc[t] = mma16(col_at(L.aT[0], 32 * t + j, kk, h), qcol, sacc[t]);
                    sacc[t] = mma16(col_at(L.aT[1], 32 * t + j, kk, h), qcol, sacc[t]);
                }
                float qf[8];
                unpack8(qcol, qf);
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2)
                    vc += L.cs[16 * kk + 8 * h + s2] * qf[s2];
            } else {
                const bf8 ahi = col_at(L.aT[0], 32 * cb + j, kk, h);  // a[ir][32cb+j]
                const bf8 alo = col_at(L.aT[1], 32 * cb + j, kk, h);
                acc = mma16(ahi, bhi, acc);
                acc = mma16(ahi, blo, acc);
                acc = mma16(alo, bhi, acc);
#pragma unroll
                for (int t = 0; t < NCB; ++t) {
                    const bf8 qcol = col_at(L.qT, 32 * t + j, kk, h);
                    sacc[t] = mma16(qcol, ahi, sacc[t]);
                    sacc[t] = mma16(qcol, alo, sacc[t]);
                }
                vc = sum8(alo, sum8(ahi, vc));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        vc = swap32_sum(vc);
        // (4) rows of dK (- r) or dV (+ t) with the vector of the rows after
        // the chunk
        const float sg = (PAR == 0) ? -1.f : 1.f;
        if (t0 + j < end)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 v = *reinterpret_cast<const f4 *>(&L.vr[32 * cb + 8 * q + 4 * h]);
                io::store4(oh + (t0 + j) * ol.sn + 32 * cb + 8 * q + 4 * h,
                           f4{acc[4 * q] + sg * v[0], acc[4 * q + 1] + sg * v[1],
                              acc[4 * q + 2] + sg * v[2], acc[4 * q + 3] + sg * v[3]});
            }
        __syncthreads();  // B2
        if (h == 0)
            L.vr[32 * cb + j] += vc;
        if (round + 1 < nrounds) {
            stage(t0 - kCc);
            if (round + 2 < nrounds)
                fetch(t0 - 2 * kCc);
        }
        __syncthreads();  // B3
    }
}

template <int D>
__global__ __launch_bounds__(64 * (D / 32)) void k_bwd_kv_causal_bf(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ G, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, const float *__restrict__ cbuf, const float *__restrict__ rec,
    int64_t N, int64_t seg_len, int nseg, OutLay ol)
{
    __shared__ __attribute__((aligned(16))) KvBfLds<D> lds;
    if (blockIdx.x & 1)
        kv_pass_bf<D, 1>(Q, K, V, G, dK, dV, cbuf, rec, N, seg_len, nseg, ol, lds);
    else
        kv_pass_bf<D, 0>(Q, K, V, G, dK, dV, cbuf, rec, N, seg_len, nseg, ol, lds);
}

// ============================================================ causal dK | dV, one pass
// The causal dK | dV pass of one segment in a single workgroup (D = 64, 128):
// waves 0 .. NCB-1 form the 32-column blocks of dK, waves NCB .. 2 NCB - 1
// those of dV, over the segment's chunks in reverse order.  The suffix state R
// (sum over the rows after the chunk of q_i a_i^T) is kept once: every wave
// owns NCB/2 of its 32 x 32 tiles as fp32 MFMA accumulators, updates them by
// the chunk (R += Q_c^T A_c) and writes them after each chunk as hi and lo
// bf16 planes in LDS, laid out [b][a] (column-major R, columns swizzled by
// rsw), from which both
// products read their operand: dK = V_c R^T - r (8 consecutive b of a row of
// R, gathered by the LDS transpose read) and dV = K_c R + t (contiguous runs
// of 8 a).  The chunk's rows of Q, K, V and A = dO / den (hi and lo) are
// staged once, as natural rows; the in-chunk blocks P = M o (A V^T - c) and
// W = M o (1 + Q K^T) are formed by 16 x 16 quarters over the waves and
// stored [j][i] as hi / lo planes.  Products over the chunk's tokens (R's
// update, P^T Q, W^T A) read 8 consecutive tokens of a column with two
// ds_read_b64_tr_b16.  The column sums r = sum c_i q_i and t = sum a_i of a
// chunk are formed at its staging, per wave by lane exchanges, and added
// over the waves by the 2 D threads that carry the running vectors.  When
// the launch has more workgroups than one batch holds (one workgroup per CU
// at D = 128), a workgroup walks several consecutive segments, starting
// from the suffix record of the last of them.

// Column of element (row r, column c) of an R plane: 4-element granule c / 4
// XOR sig(r), sig(r) = 4 (r & 3) + 2 ((r >> 2) & 1).  With rows a multiple of
// 32 banks apart, the 2-dword bank slot of a granule is its index mod 16, and
//   - the transpose read (16 lanes: rows r0 + 0..3, granules 4m + 0..3, r0 a
//     multiple of 4) hits 4 ((m ^ e) & 3) + (f ^ 2 s): 16 distinct slots;
//   - a 16-byte row read by 8 lanes (rows j = 0..7, one even granule pair)
//     hits 8 distinct even slots and their odd neighbours (sig is even, so
//     a pair stays whole and in order);
//   - an 8-byte write by 16 lanes (rows j = 0..15, one granule) hits 8
//     slots, twice each (4 times without the swizzle at pitch D + 16).
__device__ __forceinline__ int rsw(int r, int c)
{
    return c ^ (((r & 3) << 4) | ((r & 4) << 1));
}

// col8 on an R plane (swizzled columns)
__device__ __forceinline__ bf8 col8_rsw(const uint16_t *tile, int pitch, int rb, int cb0,
                                        int lane)
{
    const int g = lane >> 4, p = lane & 15;
    const int ra = rb + 8 * (g >> 1) + (p >> 2), c = cb0 + 16 * (g & 1) + 4 * (p & 3);
    typedef __attribute__((address_space(3))) v4s *lp;
    const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(tile + ra * pitch + rsw(ra, c)));
    const v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lp)(tile + (ra + 4) * pitch + rsw(ra + 4, c)));
    const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
    return __builtin_bit_cast(bf8, uint4{ux.x, ux.y, uy.x, uy.y});
}

template <int D>
struct KvBf2Lds {
    // Row pitches (bf16): D + 8 (16 mod 128 bytes) for the rows read whole
    // only (K, V: conflict-free 16-byte row reads), D + 16 (32 mod 128 bytes)
    // for the planes read mostly with the transpose read (Q and a:
    // conflict-free 16-lane transpose reads).  D = 64 keeps D + 8 there: the
    // wider planes would cost it a third resident workgroup per CU.  The R
    // planes are read both ways and written by columns (8 bytes per lane, one
    // row per lane), so they take pitch D (a multiple of 128 bytes) and the
    // XOR swizzle of rsw instead.
    static constexpr int LDX = D + 8;
    static constexpr int LDT = D == 64 ? D + 8 : D + 16;
    static constexpr int RP = D;         // R planes: element (a, b) at b * RP + rsw(b, a)
    static constexpr int PP = kCc + 8;   // P, W planes: element (i, j) at j * PP + i
    uint16_t q[kCc * LDT], k[kCc * LDX], v[kCc * LDX], ahi[kCc * LDT], alo[kCc * LDT];
    uint16_t rhi[D * RP], rlo[D * RP];
    uint16_t phi[kCc * PP], plo[kCc * PP], whi[kCc * PP], wlo[kCc * PP];
    float cs[kCc];
    float vr[D], vt[D];
    float csp[D / 16][2][D];  // each wave's column sums of c q and a over its rows
};

template <int D>
__global__ __launch_bounds__(128 * (D / 32)) void k_bwd_kv_causal_bf2(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, const uint16_t *__restrict__ G, uint16_t *__restrict__ dK,
    uint16_t *__restrict__ dV, const float *__restrict__ cbuf, const float *__restrict__ rec,
    int64_t N, int64_t seg_len, int nseg, int merge, OutLay ol)
{
    typedef nc::IO<StBF16> io;
    static_assert(D == 64 || D == 128, "two or four 32-column blocks");
    constexpr int NCB = D / 32, NW = 2 * NCB, NT = 64 * NW, KS = D / 16, CPR = D / 8;
    constexpr int TPW = NCB * NCB / NW;  // R tiles per wave
    constexpr int LDX = KvBf2Lds<D>::LDX, LDT = KvBf2Lds<D>::LDT, RP = KvBf2Lds<D>::RP,
                  PP = KvBf2Lds<D>::PP;
    static_assert(NT == kCc * CPR, "one staging item per thread");
    __shared__ __attribute__((aligned(16))) KvBf2Lds<D> L;

    // a workgroup walks `merge` consecutive segments of the plan, starting
    // from the suffix record of the last of them
    const int nsm = (nseg + merge - 1) / merge;
    const int64_t bh = blockIdx.x / nsm;
    const int sm = (int)(blockIdx.x % nsm);
    const int seg = (sm + 1) * merge - 1 < nseg ? (sm + 1) * merge - 1 : nseg - 1;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const bool isk = w < NCB;
    const int cb = isk ? w : w - NCB;
    const int64_t beg = (int64_t)sm * merge * seg_len;
    const int64_t end = (beg + merge * seg_len < N) ? beg + merge * seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
    const uint16_t *qh = Q + hoff, *kh = K + hoff, *vh = V + hoff, *gh = G + hoff;
    uint16_t *oh = (isk ? dK : dV) + ol.head(bh);
    const float2 *ch = reinterpret_cast<const float2 *>(cbuf) + bh * N;

    // staging item of this thread: row it of the chunk, 8-column piece ic;
    // two register sets (set x & 1 holds chunk x of the walk), so the loads
    // of the next two chunks are in flight while one is computed
    const int it = tid / CPR, ic = tid % CPR;
    uint4 pq[2], pk[2], pv[2], pg[2];
    float2 pc[2];
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    // (chunks before the segment, the walk's padding, read nothing: zero rows)
    auto fetch = [&](int64_t r0, auto set_) {
        constexpr int X = decltype(set_)::value;
        const int rows = r0 < beg ? 0 : (int)(end - r0 < kCc ? end - r0 : kCc);
        const int64_t rb = r0 < beg ? beg : r0;
        const int off = it * D * 2 + 16 * ic;
        auto rs = [&](const uint16_t *x) {
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(x + rb * D), (short)0,
                                                     rows * D * 2, kBufferWord3);
        };
        pq[X] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs(qh), off, 0, 0));
        pk[X] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs(kh), off, 0, 0));
        pv[X] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs(vh), off, 0, 0));
        pg[X] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs(gh), off, 0, 0));
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float2 *>(ch + rb), (short)0, rows * 8, kBufferWord3);
        pc[X] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rc, it * 8, 0, 0));
    };
    auto stage = [&](auto set_) {
        constexpr int X = decltype(set_)::value;
        const int o = it * LDT + 8 * ic, ox = it * LDX + 8 * ic;
        *reinterpret_cast<uint4 *>(&L.q[o]) = pq[X];
        *reinterpret_cast<uint4 *>(&L.k[ox]) = pk[X];
        *reinterpret_cast<uint4 *>(&L.v[ox]) = pv[X];
        float gf[8], qf[8];
        StBF16::widen(pg[X], gf);
        StBF16::widen(pq[X], qf);
        const float c = pc[X].x, inv = pc[X].y;
        float v[16];  // c q and a at the item's 8 columns
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            v[s] = c * qf[s];
            v[8 + s] = gf[s] * inv;
        }
        uint2 h0, l0, h1, l1;
        split4(v[8], v[9], v[10], v[11], h0, l0);
        split4(v[12], v[13], v[14], v[15], h1, l1);
        *reinterpret_cast<uint4 *>(&L.ahi[o]) = uint4{h0.x, h0.y, h1.x, h1.y};
        *reinterpret_cast<uint4 *>(&L.alo[o]) = uint4{l0.x, l0.y, l1.x, l1.y};
        if (ic == 0)
            L.cs[it] = c;
        // the sums of v over the wave's rows of the chunk: (D = 64: the two
        // rows of each 16-lane row first), then pairwise exchanges across
        // rows 2r, 2r + 1 and across the halves, each of which sums two
        // values at once; lane (g = lane / 16, ic) ends with v[4 n + g]
        if constexpr (CPR == 8) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                v[e] += dpp_mov<0x128>(v[e]);  // row_ror:8
        }
        float u[8], x[4];
#pragma unroll
        for (int m = 0; m < 8; ++m)
            u[m] = pair16_sum(v[2 * m], v[2 * m + 1]);
#pragma unroll
        for (int n = 0; n < 4; ++n)
            x[n] = pair32_sum(u[2 * n], u[2 * n + 1]);
        if ((lane & 15) < CPR) {
            const int g = lane >> 4;
            L.csp[w][0][8 * ic + g] = x[0];
            L.csp[w][0][8 * ic + 4 + g] = x[1];
            L.csp[w][1][8 * ic + g] = x[2];
            L.csp[w][1][8 * ic + 4 + g] = x[3];
        }
    };

    // this wave's tiles of R: tile u <-> R[32 ta .., 32 tb ..], accumulator
    // element i of lane (j, h) at a = 32 ta + 8 (i / 4) + 4 h + i % 4, b = 32 tb + j
    f16v racc[TPW];
    auto write_r = [&]() {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int tau = w * TPW + u, ta = tau / NCB, tb = tau % NCB;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint2 hi, lo;
                split4(racc[u][4 * q], racc[u][4 * q + 1], racc[u][4 * q + 2], racc[u][4 * q + 3],
                       hi, lo);
                const int o = (32 * tb + j) * RP + rsw(j, 32 * ta + 8 * q + 4 * h);
                *reinterpret_cast<uint2 *>(&L.rhi[o]) = hi;
                *reinterpret_cast<uint2 *>(&L.rlo[o]) = lo;
            }
        }
    };

    // The walk is padded to an even number of chunks (a padding chunk lies
    // before the segment: zero rows, no output rows, nothing added to the
    // state), so that its loop body is two chunks of straight-line code with
    // every load and stage unconditional: each stage then waits for its own
    // loads only (a branch around a load makes the compiler wait for all).
    const int64_t nrounds = (end - beg + kCc - 1) / kCc;
    const int64_t nr2 = (nrounds + 1) / 2 * 2;
    const int64_t last = beg + (nrounds - 1) * kCc;
    fetch(last, S0{});
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tau = w * TPW + u, ta = tau / NCB, tb = tau % NCB;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            racc[u][i] = st[(32 * ta + 8 * (i / 4) + 4 * h + (i % 4)) * D + 32 * tb + j];
    }
    // the vector threads: the first 2 D of the workgroup, thread e holds
    // element e of [r | t] of the rows after the chunk
    const bool vth = tid < 2 * D;
    float rt = vth ? st[D * D + tid] : 0.f;
    write_r();
    stage(S0{});
    drain_loads();
    fetch(last - kCc, S1{});
    fetch(last - 2 * kCc, S0{});
    __syncthreads();

    // one chunk; set_ holds the next chunk's rows (round + 1 = set_ mod 2)
    auto round_body = [&](int64_t round, auto set_) {
        const int64_t t0 = last - round * kCc;
        // (1) the suffix state applied to the chunk's rows: dK^T block
        // C[a][t] = sum_b R[a][b] V[t][b], or dV^T block C[b][t] = sum_a
        // R[a][b] K[t][a]
        // (the role tests stay outside the k-loops: a branch inside one would
        // split it into blocks and keep the LDS reads from running ahead)
        f16v acc = zero16();
        if (isk) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf8 x = row8(L.v, LDX, 0, 16 * ks, j, h);
                acc = mma16(col8_rsw(L.rhi, RP, 16 * ks, 32 * cb, lane), x, acc);
                acc = mma16(col8_rsw(L.rlo, RP, 16 * ks, 32 * cb, lane), x, acc);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf8 x = row8(L.k, LDX, 0, 16 * ks, j, h);
                const int o = (32 * cb + j) * RP + rsw(j, 16 * ks + 8 * h);
                acc = mma16(*reinterpret_cast<const bf8 *>(&L.rhi[o]), x, acc);
                acc = mma16(*reinterpret_cast<const bf8 *>(&L.rlo[o]), x, acc);
            }
        }
        // the in-chunk blocks, [j][i] planes: P = A V^T - c and W = 1 + Q K^T,
        // masked to i >= j, by 16 x 16 quarters (i block 16 (qd / 2), j block
        // 16 (qd % 2)) on v_mfma_f32_16x16x32_bf16: lane l supplies row l % 16
        // of each block and columns 8 (l / 16) .. + 7 of a 32-column step, and
        // receives i = 4 (l / 16) + 0..3 of j = l % 16.  Wave w forms quarter
        // w % 4 of P (w < 4) or of W; with four waves, both.  The quarter
        // above the diagonal is all zero and skips the product.
#pragma unroll
        for (int pw = 0; pw < 2; ++pw) {
            if (NW == 8 && pw != (w >> 2))
                continue;
            const int qd = w & 3, ib0 = 16 * (qd >> 1), jb0 = 16 * (qd & 1);
            const int r16 = lane & 15, g4 = lane >> 4;
            f4 t = {0.f, 0.f, 0.f, 0.f};
            if (jb0 <= ib0) {
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    const int oi = (ib0 + r16) * LDT + 32 * ks + 8 * g4;
                    const int oj = (jb0 + r16) * LDX + 32 * ks + 8 * g4;
                    if (pw == 0) {
                        const bf8 vj = *reinterpret_cast<const bf8 *>(&L.v[oj]);
                        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            *reinterpret_cast<const bf8 *>(&L.ahi[oi]), vj, t, 0, 0, 0);
                        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            *reinterpret_cast<const bf8 *>(&L.alo[oi]), vj, t, 0, 0, 0);
                    } else {
                        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            *reinterpret_cast<const bf8 *>(&L.q[oi]),
                            *reinterpret_cast<const bf8 *>(&L.k[oj]), t, 0, 0, 0);
                    }
                }
            }
            const int jj = jb0 + r16, i0 = ib0 + 4 * g4;
            float x4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x4[r] = (i0 + r >= jj) ? ((pw == 0) ? t[r] - L.cs[i0 + r] : 1.f + t[r]) : 0.f;
            uint2 hi, lo;
            split4(x4[0], x4[1], x4[2], x4[3], hi, lo);
            *reinterpret_cast<uint2 *>(&(pw == 0 ? L.phi : L.whi)[jj * PP + i0]) = hi;
            *reinterpret_cast<uint2 *>(&(pw == 0 ? L.plo : L.wlo)[jj * PP + i0]) = lo;
        }
        // the vectors of the rows after the chunk go to LDS for the
        // epilogue; then the chunk's column sums (the waves' partials from
        // its staging) join them
        if (vth) {
            const int vi = tid / D, cd = tid % D;
            (vi ? L.vt : L.vr)[cd] = rt;
            float sc = 0.f;
#pragma unroll
            for (int u = 0; u < NW; ++u)
                sc += L.csp[u][vi][cd];
            rt += sc;
        }
        __syncthreads();  // B1
        // (2) in-chunk terms: dK^T += Q^T P (C[a][j] += sum_i Q[i][a] P[i][j]),
        // dV^T += A^T W (C[b][j] += sum_i A[i][b] W[i][j])
        if (isk) {
#pragma unroll
            for (int kk = 0; kk < kCc / 16; ++kk) {
                const bf8 qa = col8(L.q, LDT, 16 * kk, 32 * cb, lane);
                acc = mma16(qa, row8(L.phi, PP, 0, 16 * kk, j, h), acc);
                acc = mma16(qa, row8(L.plo, PP, 0, 16 * kk, j, h), acc);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < kCc / 16; ++kk) {
                const bf8 ah = col8(L.ahi, LDT, 16 * kk, 32 * cb, lane);
                const bf8 al = col8(L.alo, LDT, 16 * kk, 32 * cb, lane);
                const bf8 wh = row8(L.whi, PP, 0, 16 * kk, j, h);
                acc = mma16(ah, wh, acc);
                acc = mma16(ah, row8(L.wlo, PP, 0, 16 * kk, j, h), acc);
                acc = mma16(al, wh, acc);
            }
        }
        // rows of dK (- r) or dV (+ t) with the vectors of the rows after the chunk
        {
            const float sg = isk ? -1.f : 1.f;
            const float *vec = isk ? L.vr : L.vt;
            f4 o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 v = *reinterpret_cast<const f4 *>(&vec[32 * cb + 8 * q + 4 * h]);
                o[q] = f4{acc[4 * q] + sg * v[0], acc[4 * q + 1] + sg * v[1],
                          acc[4 * q + 2] + sg * v[2], acc[4 * q + 3] + sg * v[3]};
            }
            store_row32(oh + (t0 + j) * ol.sn + 32 * cb, o, h, t0 + j >= beg && t0 + j < end);
        }
        // the suffix state takes the chunk in: R += Q_c^T A_c (also after the
        // last chunk, where it is not read again)
        {
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int tau = w * TPW + u, ta = tau / NCB, tb = tau % NCB;
#pragma unroll
                for (int kk = 0; kk < kCc / 16; ++kk) {
                    const bf8 qa = col8(L.q, LDT, 16 * kk, 32 * ta, lane);
                    racc[u] = mma16(qa, col8(L.ahi, LDT, 16 * kk, 32 * tb, lane), racc[u]);
                    racc[u] = mma16(qa, col8(L.alo, LDT, 16 * kk, 32 * tb, lane), racc[u]);
                }
            }
            write_r();
        }
        __syncthreads();  // B2
        stage(set_);
        fetch(t0 - 3 * kCc, set_);
        __syncthreads();  // B3
    };
    for (int64_t round = 0; round < nr2; round += 2) {
        round_body(round, S1{});
        round_body(round + 1, S0{});
    }
}

}  // namespace bf
}  // namespace la
