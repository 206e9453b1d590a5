// la_kernels_nc.hpp -- non-causal linear attention for D <= 128 on gfx950.
//
// Same method as la_kernels.hpp (similarity 1 + q.k, normalised rows; state
// S = K^T V, z = sum k, u = sum v; gradient state dS = Q^T A, r = sum c q,
// t = sum a), laid out for the non-causal case, where every row of a head
// sees the same state:
//
//   k_reduce_nc : Mat = X^T Y over a segment of rows plus column sums.  The
//                 contraction runs over tokens, which are the row index of
//                 X and Y in memory, so MFMA operands are loaded straight
//                 from global memory (16 consecutive columns of one row per
//                 16 lanes) with a several-steps-deep register prefetch; no
//                 LDS, no barriers in the loop.
//   k_apply_nc  : out_i = epilogue(M-applied row i) for every row of a
//                 segment.  The D x D matrix sits in LDS (loaded once per
//                 workgroup), and each wave streams its own 16-row tiles
//                 with no barrier.  The product is formed transposed
//                 (out^T = M . X^T): the row tile is the MFMA B operand,
//                 read from global as 16-byte vectors along the row, and
//                 the result comes back as 4 consecutive columns of one
//                 row per lane, so stores are 16-byte vectors too and every
//                 per-row scalar (den_i, c_i) stays inside the lane.
//
// MFMA: v_mfma_f32_16x16x4_f32.  Lane l = 16*lg + lr supplies A[m=lr][k=lg]
// and B[k=lg][n=lr] and receives C[m=4*lg+r][n=lr], r = 0..3.  In the apply
// kernel the four accumulator steps r use k = 4*lg + r inside a 16-block,
// for which both operands are contiguous 16-byte reads.
#pragma once

#include "la_kernels.hpp"

namespace la {
namespace nc {

// ------------------------------------------------------------ element I/O
template <class ST>
struct IO;

template <>
struct IO<StF32> {
    __device__ static __forceinline__ float load1(const float *p) { return *p; }
    __device__ static __forceinline__ f4 load4(const float *p)
    {
        return *reinterpret_cast<const f4 *>(p);
    }
    __device__ static __forceinline__ void store4(float *p, f4 v)
    {
        *reinterpret_cast<f4 *>(p) = v;
    }
};

template <>
struct IO<StBF16> {
    __device__ static __forceinline__ float load1(const uint16_t *p)
    {
        return __uint_as_float((uint32_t)*p << 16);
    }
    __device__ static __forceinline__ f4 load4(const uint16_t *p)
    {
        const uint2 r = *reinterpret_cast<const uint2 *>(p);
        return f4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                  __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u)};
    }
    __device__ static __forceinline__ void store4(uint16_t *p, f4 v)
    {
        uint2 r;
        r.x = (uint32_t)StBF16::narrow(v[0]) | ((uint32_t)StBF16::narrow(v[1]) << 16);
        r.y = (uint32_t)StBF16::narrow(v[2]) | ((uint32_t)StBF16::narrow(v[3]) << 16);
        *reinterpret_cast<uint2 *>(p) = r;
    }
};

__device__ __forceinline__ float dot4(f4 a, f4 b)
{
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// sum over the four lane groups (lanes with equal l % 16)
__device__ __forceinline__ float lg_sum(float v)
{
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

constexpr int kReduceThreads = 256;
constexpr int kApplyThreads = 256;

// v_mfma_f32_32x32x2_f32: lane l = 32*h + j supplies A[m=j][k=h] and
// B[k=h][n=j] and holds accumulator element i at row 8*(i/4) + 4*h + i%4,
// column j.  (The 16x16x4 form issues at a lower sustained rate.)
typedef float f16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f16v mma32(float a, float b, f16v c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16v zero16()
{
    f16v z;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        z[i] = 0.f;
    return z;
}

// VW consecutive elements at p, widened to fp32 into o[0..VW)
template <class ST, int VW>
__device__ __forceinline__ void load_vec(const typename ST::T *p, float *o)
{
    if constexpr (sizeof(typename ST::T) == 4) {
        if constexpr (VW == 2) {
            const float2 x = *reinterpret_cast<const float2 *>(p);
            o[0] = x.x;
            o[1] = x.y;
        } else {
            o[0] = *reinterpret_cast<const float *>(p);
        }
    } else {
        if constexpr (VW == 2) {
            const uint32_t x = *reinterpret_cast<const uint32_t *>(p);
            o[0] = __uint_as_float(x << 16);
            o[1] = __uint_as_float(x & 0xffff0000u);
        } else {
            o[0] = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(p) << 16);
        }
    }
}

// ============================================================ reduction
// Record (bh, seg): Mat[D][D] = sum_t X[t]^T Y'[t], cx[D] = sum_t w_t X[t],
// cy[D] = sum_t Y'[t] over the rows t of the segment, where
//   forward  (GRAD = false): Y' = Y, w = 1          -> S, z, u
//   backward (GRAD = true) : Y' = Y * inv_den_t, w = c_t  -> dS, r, t
// with (c_t, inv_den_t) read from cbuf.  Waves own square output tiles
// (TM x TM, TM = min(D, 64)); when there are fewer tiles than waves, the
// waves of a tile split the token steps and add their partials in LDS.
//
// One MFMA step covers two tokens (k = h).  Lane j loads VW = TM/32
// consecutive columns of its token's row, so 32 lanes read 32*VW columns:
// MFMA (ca, cb) pairs column m0 + VW*j + ca of X with column n0 + VW*j + cb
// of Y, and accumulator (ca, cb) element i holds
// Mat[m0 + VW*(8*(i/4) + 4*h + i%4) + ca][n0 + VW*j + cb].
template <class ST, int D, bool GRAD>
__global__ __launch_bounds__(kReduceThreads) void k_reduce_nc(
    const typename ST::T *__restrict__ X, const typename ST::T *__restrict__ Y,
    const float *__restrict__ cbuf, float *__restrict__ part, int64_t N, int64_t seg_len,
    int nseg)
{
    typedef typename ST::T T;
    static_assert(D >= 32, "32x32 tiles");
    constexpr int TM = D < 64 ? D : 64;
    constexpr int NQ1 = D / TM;
    constexpr int NQ = NQ1 * NQ1;
    constexpr int NWAVE = kReduceThreads / 64;
    static_assert(NQ <= NWAVE && NWAVE % NQ == 0, "tile split");
    constexpr int TS = NWAVE / NQ;  // waves per output tile
    constexpr int VW = TM / 32;     // columns per lane
    constexpr int U = GRAD ? 16 : 24;  // prefetched steps (<= 48 loads in flight)
    __shared__ float red[(TS > 1) ? (TS - 1) * (TM * TM + 2 * TM) : 1];

    const int64_t bh = blockIdx.x / nseg;
    const int seg = (int)(blockIdx.x % nseg);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int quad = w % NQ, tsi = w / NQ;
    const int m0 = (quad / NQ1) * TM, n0 = (quad % NQ1) * TM;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const T *xh = X + bh * N * D + m0 + VW * j;
    const T *yh = Y + bh * N * D + n0 + VW * j;
    const float2 *ch = GRAD ? reinterpret_cast<const float2 *>(cbuf) + bh * N : nullptr;
    const int64_t nsteps = (end - beg + 1) / 2;

    f16v acc[VW][VW];
#pragma unroll
    for (int a = 0; a < VW; ++a)
#pragma unroll
        for (int b = 0; b < VW; ++b)
            acc[a][b] = zero16();
    float csx[VW], csy[VW];
#pragma unroll
    for (int a = 0; a < VW; ++a)
        csx[a] = csy[a] = 0.f;

    float ra[U][VW], rb[U][VW], rc[U], rs[U];
    // Prefetch ring over this wave's complete 2-token steps.  Addresses are
    // clamped into the segment and no loaded value is masked: slots past the
    // last step are fetched but never consumed, so nothing waits on a load
    // before its use.  An odd last token is handled after the loop.
    auto fetch = [&](int u, int64_t s) {
        int64_t t = beg + 2 * s + h;
        t = t < end ? t : end - 1;
        load_vec<ST, VW>(xh + t * D, ra[u]);
        load_vec<ST, VW>(yh + t * D, rb[u]);
        if constexpr (GRAD) {
            const float2 cs = ch[t];
            rc[u] = cs.x;
            rs[u] = cs.y;
        }
    };
    auto consume = [&](const float *xa, const float *yb, float c, float sc) {
        float y2[VW];
#pragma unroll
        for (int b = 0; b < VW; ++b)
            y2[b] = GRAD ? yb[b] * sc : yb[b];
#pragma unroll
        for (int a = 0; a < VW; ++a)
#pragma unroll
            for (int b = 0; b < VW; ++b)
                acc[a][b] = mma32(xa[a], y2[b], acc[a][b]);
#pragma unroll
        for (int a = 0; a < VW; ++a) {
            csx[a] += GRAD ? c * xa[a] : xa[a];
            csy[a] += y2[a];
        }
    };

    const int64_t npairs = (end - beg) / 2;
    // trip counts in scalar registers: the unrolled loop body has no branch,
    // so each consume waits only for its own slot's loads
    const int mine = __builtin_amdgcn_readfirstlane(
        (int)(npairs > tsi ? (npairs - tsi + TS - 1) / TS : 0));
    const int full = mine / U;
#pragma unroll
    for (int u = 0; u < U; ++u)
        fetch(u, tsi + (int64_t)u * TS);
    for (int it = 0; it < full; ++it) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            consume(ra[u], rb[u], GRAD ? rc[u] : 1.f, GRAD ? rs[u] : 1.f);
            fetch(u, tsi + ((int64_t)(it + 1) * U + u) * TS);
            // keep step u's work and its refill together: the scheduler would
            // otherwise sink the refills to the end of the body and hoist the
            // column-sum adds of later steps, each forcing an early wait
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (u < mine - full * U)
            consume(ra[u], rb[u], GRAD ? rc[u] : 1.f, GRAD ? rs[u] : 1.f);
    if (((end - beg) & 1) && tsi == (int)(npairs % TS)) {
        // last, unpaired token: lane half h = 1 contributes zeros
        const int64_t t = end - 1;
        float xa[VW], yb[VW];
        load_vec<ST, VW>(xh + t * D, xa);
        load_vec<ST, VW>(yh + t * D, yb);
        float c = 1.f, sc = 1.f;
        if constexpr (GRAD) {
            const float2 cs = ch[t];
            c = cs.x;
            sc = cs.y;
        }
#pragma unroll
        for (int a = 0; a < VW; ++a) {
            xa[a] = h == 0 ? xa[a] : 0.f;
            yb[a] = h == 0 ? yb[a] : 0.f;
        }
        consume(xa, yb, h == 0 ? c : 0.f, sc);
    }
#pragma unroll
    for (int a = 0; a < VW; ++a) {
        csx[a] += __shfl_xor(csx[a], 32, 64);
        csy[a] += __shfl_xor(csy[a], 32, 64);
    }

    if constexpr (TS > 1) {
        // waves tsi > 0 hand their partials to wave tsi == 0 of the same tile
        if (tsi > 0) {
            float *dst = red + (tsi - 1) * (TM * TM + 2 * TM);
#pragma unroll
            for (int a = 0; a < VW; ++a)
#pragma unroll
                for (int b = 0; b < VW; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        dst[((a * VW + b) * 16 + i) * 64 + lane] = acc[a][b][i];
            if (h == 0)
#pragma unroll
                for (int a = 0; a < VW; ++a) {
                    dst[TM * TM + a * 32 + j] = csx[a];
                    dst[TM * TM + TM + a * 32 + j] = csy[a];
                }
        }
        __syncthreads();
        if (tsi == 0) {
            for (int o = 0; o < TS - 1; ++o) {
                const float *src = red + o * (TM * TM + 2 * TM);
#pragma unroll
                for (int a = 0; a < VW; ++a)
#pragma unroll
                    for (int b = 0; b < VW; ++b)
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            acc[a][b][i] += src[((a * VW + b) * 16 + i) * 64 + lane];
#pragma unroll
                for (int a = 0; a < VW; ++a) {
                    csx[a] += src[TM * TM + a * 32 + j];
                    csy[a] += src[TM * TM + TM + a * 32 + j];
                }
            }
        }
    }
    if (tsi != 0)
        return;
    float *out = part + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
#pragma unroll
    for (int a = 0; a < VW; ++a)
#pragma unroll
        for (int b = 0; b < VW; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                out[(m0 + VW * (8 * (i / 4) + 4 * h + (i % 4)) + a) * D + n0 + VW * j + b] =
                    acc[a][b][i];
    if (h == 0) {
        if (n0 == 0)
#pragma unroll
            for (int a = 0; a < VW; ++a)
                out[D * D + m0 + VW * j + a] = csx[a];
        if (m0 == 0)
#pragma unroll
            for (int a = 0; a < VW; ++a)
                out[D * D + D + n0 + VW * j + a] = csy[a];
    }
}

// ============================================================ apply
// A is the MFMA left operand applied to each row x_i of X:
// KIND 0 forward : A = S^T;  o_i = (u + A q_i) / (N + q_i.z);
//                  X = Q.  den_out[i] = N + q_i.z (optional).
// KIND 1 dQ      : A = S;  a_i = g_i / den_i, y_i = A a_i,
//                  c_i = (a_i.u + q_i.y_i) / den_i, dq_i = y_i - c_i z;
//                  X = dO, X2 = Q; cbuf[i] = (c_i, 1/den_i).
// KIND 2 dK | dV : blockIdx parity 0: A = dS, X = V, dk_j = A v_j - r;
//                  parity 1: A = dS^T, X2 = K, dv_j = A k_j + t.
// rec: total record of the head: Mat[D][D], vec1[D], vec2[D] =
//      (S, z, u) for KIND 0/1 and (dS, r, t) for KIND 2.
//
// The workgroup's waves split the output columns into 32-column blocks
// (and, for D < 128, the rows into row groups).  Each wave keeps its block
// of A in registers (D/2 values per lane, loaded once).  The workgroup
// stages each round of 32-row tiles of X in LDS (fp32, double-buffered:
// the next round is fetched into registers while the current one is
// computed, one barrier per round), and every wave reads its MFMA B operand
// from there: column n = tile row j, k-block kb = columns kb*8 .. kb*8+7
// (lane half h reads 4*h .. 4*h+3 as one 16-byte LDS read feeding four
// MFMAs).  The accumulator returns 4 groups of 4 consecutive output columns
// per lane (16-byte stores).  The normalisation is linear, so per-row
// scalars are applied in the epilogue; row sums over all columns (q.z, and
// for dQ also dO.u and q.y) are formed per column block and exchanged
// through LDS at the same barrier.  Rows past the end of the segment are
// staged as zeros and not stored.
template <class ST, int D, int KIND>
__global__ __launch_bounds__(kApplyThreads) void k_apply_nc(
    const typename ST::T *__restrict__ X, const typename ST::T *__restrict__ X2,
    typename ST::T *__restrict__ Out, typename ST::T *__restrict__ Out2,
    float *__restrict__ den_out, float *__restrict__ cbuf, const float *__restrict__ rec,
    int64_t N, int64_t seg_len, int nseg)
{
    typedef typename ST::T T;
    typedef IO<ST> io;
    static_assert(D >= 32, "32-column output blocks");
    constexpr int KB = D / 8;                // k-blocks of 8
    constexpr int NWAVE = kApplyThreads / 64;
    constexpr int NCB = D / 32;              // column blocks
    static_assert(NCB <= NWAVE && NWAVE % NCB == 0, "column split");
    constexpr int NRG = NWAVE / NCB;         // row groups
    constexpr int TR = 32 * NRG;             // rows staged per round
    constexpr int LDX = D + 4;               // LDS row pitch (floats)
    constexpr int VEC = 16 / sizeof(T);      // elements per 16-byte load
    constexpr int CPR = D / VEC;             // 16-byte chunks per row
    constexpr int PER = TR * CPR / kApplyThreads;  // chunks per thread per round
    static_assert(TR * CPR % kApplyThreads == 0, "staging split");
    __shared__ __attribute__((aligned(16))) float xs[2][TR * LDX];
    __shared__ float xch[2][NRG][NCB][32][3];  // per-row partial sums of the blocks

    const int sub = (KIND == 2) ? (int)(blockIdx.x & 1) : 0;
    const int64_t b = (KIND == 2) ? (blockIdx.x >> 1) : blockIdx.x;
    const int64_t bh = b / nseg;
    const int seg = (int)(b % nseg);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int cb = w % NCB, rg = w / NCB;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + bh * (int64_t)(D * D + 2 * D);
    const bool colread = (KIND == 0) || (KIND == 2 && sub == 1);

    const T *xh = ((KIND == 2 && sub == 1) ? X2 : X) + hoff;
    const T *qh = (KIND == 1) ? X2 + hoff : nullptr;
    T *oh = ((KIND == 2 && sub == 1) ? Out2 : Out) + hoff;

    // staging: thread's chunk p of a round covers row (tid + p*NT) / CPR,
    // columns VEC*((tid + p*NT) % CPR) ..
    uint4 stg[PER];
    auto fetch_round = [&](int64_t r0) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * kApplyThreads;
            int64_t row = r0 + c / CPR;
            row = row < end ? row : end - 1;  // valid address; zeroed when staged
            stg[p] = *reinterpret_cast<const uint4 *>(xh + row * D + VEC * (c % CPR));
        }
    };
    auto stage_round = [&](int buf, int64_t r0) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * kApplyThreads;
            const bool ok = r0 + c / CPR < end;
            float v[VEC];
            if constexpr (VEC == 4)
                StF32::widen(stg[p], v);
            else
                StBF16::widen(stg[p], v);
            float *dst = &xs[buf][(c / CPR) * LDX + VEC * (c % CPR)];
#pragma unroll
            for (int x = 0; x < VEC; x += 4)
                *reinterpret_cast<f4 *>(dst + x) =
                    ok ? f4{v[x], v[x + 1], v[x + 2], v[x + 3]} : f4{0.f, 0.f, 0.f, 0.f};
        }
    };

    const int64_t nrounds = (end - beg + TR - 1) / TR;
    fetch_round(beg);

    // this wave's block of A: am[kb][r] = A[32*cb + j][kb*8 + 4*h + r]
    float am[KB][4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        if (colread) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                am[kb][r] = st[(kb * 8 + 4 * h + r) * D + 32 * cb + j];
        } else {
            const f4 v = *reinterpret_cast<const f4 *>(st + (32 * cb + j) * D + kb * 8 + 4 * h);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                am[kb][r] = v[r];
        }
    }
    // epilogue vector at the lane's output columns 32*cb + 8*q + 4*h + (0..3)
    f4 ev[4];
    {
        const float *vec = st + D * D + ((KIND == 0 || (KIND == 2 && sub == 1)) ? D : 0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            ev[q] = *reinterpret_cast<const f4 *>(vec + 32 * cb + 8 * q + 4 * h);
    }
    // second vector at the same columns: z (forward, for q.z) or u (dQ, for dO.u)
    f4 ew[4];
    if constexpr (KIND == 0 || KIND == 1) {
        const float *vec = st + D * D + (KIND == 0 ? 0 : D);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            ew[q] = *reinterpret_cast<const f4 *>(vec + 32 * cb + 8 * q + 4 * h);
    }
    stage_round(0, beg);
    if (nrounds > 1)
        fetch_round(beg + TR);
    __syncthreads();

    for (int64_t round = 0; round < nrounds; ++round) {
        const int buf = (int)(round & 1);
        const int64_t t0 = beg + round * TR + 32 * rg;  // this row group's tile
        const float *xt = &xs[buf][(32 * rg + j) * LDX + 4 * h];
        f4 qv[4];
        if constexpr (KIND == 1) {
            int64_t r = t0 + j;
            r = r < end ? r : end - 1;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                qv[q] = io::load4(qh + r * D + 32 * cb + 8 * q + 4 * h);
        }

        f16v acc = zero16();
        // LDS operand one k-block ahead of the MFMAs; the scheduling barrier
        // per k-block stops the compiler from hoisting every read of the tile
        f4 xn = *reinterpret_cast<const f4 *>(xt);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const f4 x = xn;
            if (kb + 1 < KB)
                xn = *reinterpret_cast<const f4 *>(xt + (kb + 1) * 8);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc = mma32(am[kb][r], x[r], acc);
            __builtin_amdgcn_sched_barrier(0);
        }

        const int64_t row = t0 + j;
        const bool ok = row < end;
        float c = 0.f, inv = 0.f;
        if constexpr (KIND == 0 || KIND == 1) {
            // partial row sums over this block's 32 columns, exchanged below:
            // forward: q.z;  dQ: dO.u, q.z, q.(S dO)
            const float *xr = &xs[buf][(32 * rg + j) * LDX + 32 * cb + 4 * h];
            float p0 = 0.f, p1 = 0.f, p2 = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                p0 += dot4(*reinterpret_cast<const f4 *>(xr + 8 * q), ew[q]);
            if constexpr (KIND == 1) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    p1 += dot4(qv[q], ev[q]);
                    p2 += qv[q][0] * acc[4 * q] + qv[q][1] * acc[4 * q + 1] +
                          qv[q][2] * acc[4 * q + 2] + qv[q][3] * acc[4 * q + 3];
                }
            }
            p0 += __shfl_xor(p0, 32, 64);
            p1 += __shfl_xor(p1, 32, 64);
            p2 += __shfl_xor(p2, 32, 64);
            if (h == 0) {
                xch[buf][rg][cb][j][0] = p0;
                xch[buf][rg][cb][j][1] = p1;
                xch[buf][rg][cb][j][2] = p2;
            }
        }
        // stage the next round (its buffer was last read before the previous
        // barrier) and fetch the one after
        if (round + 1 < nrounds) {
            stage_round(buf ^ 1, beg + (round + 1) * TR);
            if (round + 2 < nrounds)
                fetch_round(beg + (round + 2) * TR);
        }
        __syncthreads();

        if constexpr (KIND == 0) {
            float qz = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < NCB; ++c2)
                qz += xch[buf][rg][c2][j][0];
            const float den = (float)N + qz;
            inv = 1.f / den;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 o = {(acc[4 * q] + ev[q][0]) * inv, (acc[4 * q + 1] + ev[q][1]) * inv,
                              (acc[4 * q + 2] + ev[q][2]) * inv, (acc[4 * q + 3] + ev[q][3]) * inv};
                if (ok)
                    io::store4(oh + row * D + 32 * cb + 8 * q + 4 * h, o);
            }
            if (den_out != nullptr && ok && h == 0 && cb == 0)
                den_out[bh * N + row] = den;
        } else if constexpr (KIND == 1) {
            float rz = 0.f, qz = 0.f, qy = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < NCB; ++c2) {
                rz += xch[buf][rg][c2][j][0];
                qz += xch[buf][rg][c2][j][1];
                qy += xch[buf][rg][c2][j][2];
            }
            inv = 1.f / ((float)N + qz);
            c = (rz + qy) * inv * inv;  // (a.u + q.y_true) / den
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 o = {acc[4 * q] * inv - c * ev[q][0], acc[4 * q + 1] * inv - c * ev[q][1],
                              acc[4 * q + 2] * inv - c * ev[q][2],
                              acc[4 * q + 3] * inv - c * ev[q][3]};
                if (ok)
                    io::store4(oh + row * D + 32 * cb + 8 * q + 4 * h, o);
            }
            if (ok && h == 0 && cb == 0)
                reinterpret_cast<float2 *>(cbuf)[bh * N + row] = float2{c, inv};
        } else {
            const float sgn = (sub == 0) ? -1.f : 1.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 o = {acc[4 * q] + sgn * ev[q][0], acc[4 * q + 1] + sgn * ev[q][1],
                              acc[4 * q + 2] + sgn * ev[q][2], acc[4 * q + 3] + sgn * ev[q][3]};
                if (ok)
                    io::store4(oh + row * D + 32 * cb + 8 * q + 4 * h, o);
            }
        }
    }
}

}  // namespace nc
}  // namespace la
