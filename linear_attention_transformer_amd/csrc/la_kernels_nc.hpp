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
//                 from global memory (32 lanes per token row, consecutive
//                 columns per lane) with a several-steps-deep register
//                 prefetch; no LDS, no barriers in the loop.
//   k_apply_nc  : out_i = epilogue(A x_i) for every row x_i of a segment
//                 (forward: A = S^T; dK: A = dS; dV: A = dS^T).  Each wave
//                 keeps a 32-column block of A in registers; the workgroup
//                 stages 32-row tiles of X in LDS (double-buffered, one
//                 barrier per round) and every wave reads its MFMA B operand
//                 from there.
//   k_bwd_q_nc  : dQ and the segment's gradient record in one pass over Q
//                 and dO: one role of waves forms dQ as k_apply_nc does, the
//                 other accumulates dS = Q^T A from the same staged tiles.
//
// MFMA: v_mfma_f32_32x32x2_f32 throughout (layout below).
#pragma once

#include <type_traits>

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
        r.x = StBF16::narrow2(v[0], v[1]);
        r.y = StBF16::narrow2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(p) = r;
    }
};

template <>
struct IO<StF16> {
    __device__ static __forceinline__ float load1(const uint16_t *p) { return StF16::widen1(*p); }
    __device__ static __forceinline__ f4 load4(const uint16_t *p)
    {
        const uint2 r = *reinterpret_cast<const uint2 *>(p);
        float v[4];
        StF16::widen2(r.x, v);
        StF16::widen2(r.y, v + 2);
        return f4{v[0], v[1], v[2], v[3]};
    }
    __device__ static __forceinline__ void store4(uint16_t *p, f4 v)
    {
        uint2 r;
        r.x = StF16::narrow2(v[0], v[1]);
        r.y = StF16::narrow2(v[2], v[3]);
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
    return swap32_sum(swap16_sum(v));
}

constexpr int kReduceThreads = 256;
constexpr int kApplyThreads = 256;
// apply workgroups: four waves, or one wave per 32-column block when D > 128
template <int D>
constexpr int apply_threads()
{
    return D > 128 ? 64 * (D / 32) : kApplyThreads;
}

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

// Wait until every global load issued so far has returned.  Called once,
// before a loop whose body reads registers loaded ahead of it: otherwise the
// compiler keeps those loads pending across the loop's back edge and waits
// on them inside the loop, which also drains the loop's own prefetches.
__device__ __forceinline__ void drain_loads()
{
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); expcnt, lgkmcnt not waited on
    __builtin_amdgcn_sched_barrier(0);
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
        if constexpr (VW == 2)
            ST::widen2(*reinterpret_cast<const uint32_t *>(p), o);
        else
            o[0] = ST::widen1(*reinterpret_cast<const uint16_t *>(p));
    }
}

// load_vec through a raw buffer descriptor (voffset per lane, soffset uniform)
template <class ST, int VW>
__device__ __forceinline__ void buf_load_vec(__amdgpu_buffer_rsrc_t rs, int vo, int so, float *o)
{
    if constexpr (sizeof(typename ST::T) == 4) {
        if constexpr (VW == 2) {
            const float2 x =
                __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rs, vo, so, 0));
            o[0] = x.x;
            o[1] = x.y;
        } else {
            o[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, vo, so, 0));
        }
    } else {
        if constexpr (VW == 2)
            ST::widen2(__builtin_amdgcn_raw_buffer_load_b32(rs, vo, so, 0), o);
        else
            o[0] = ST::widen1((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, vo, so, 0));
    }
}

// ============================================================ reduction
// Record (bh, seg): Mat[D][D] = sum_t X[t]^T Y'[t], cx[D] = sum_t w_t X[t],
// cy[D] = sum_t Y'[t] over the rows t of the segment, where
//   forward  (GRAD = false): Y' = Y, w = 1          -> S, z, u
//   backward (GRAD = true) : Y' = Y * inv_den_t, w = c_t  -> dS, r, t
// with (c_t, inv_den_t) read from cbuf.  A workgroup forms one DB x DB block
// of Mat (DB = min(D, 128); D = 256 takes 4 workgroups per segment, block
// index fastest in blockIdx).  Waves own square output tiles (TM x TM,
// TM = min(DB, 64)); when there are fewer tiles than waves, the waves of a
// tile split the token steps and add their partials in LDS.
//
// One MFMA step covers two tokens (k = h).  Lane j loads VW = TM/32
// consecutive columns of its token's row, so 32 lanes read 32*VW columns:
// MFMA (ca, cb) pairs column m0 + VW*j + ca of X with column n0 + VW*j + cb
// of Y, and accumulator (ca, cb) element i holds
// Mat[m0 + VW*(8*(i/4) + 4*h + i%4) + ca][n0 + VW*j + cb].
template <int D>
constexpr int reduce_blocks()
{
    return D > 128 ? (D / 128) * (D / 128) : 1;
}

template <class ST, int D, bool GRAD>
__global__ __launch_bounds__(kReduceThreads) void k_reduce_nc(
    const typename ST::T *__restrict__ X, const typename ST::T *__restrict__ Y,
    const float *__restrict__ cbuf, float *__restrict__ part, int64_t N, int64_t seg_len,
    int nseg)
{
    typedef typename ST::T T;
    static_assert(D >= 32, "32x32 tiles");
    constexpr int DB = D < 128 ? D : 128;  // this workgroup's block of Mat
    constexpr int NB1 = D / DB;
    constexpr int TM = DB < 64 ? DB : 64;
    constexpr int NQ1 = DB / TM;
    constexpr int NQ = NQ1 * NQ1;
    constexpr int NWAVE = kReduceThreads / 64;
    static_assert(NQ <= NWAVE && NWAVE % NQ == 0, "tile split");
    constexpr int TS = NWAVE / NQ;  // waves per output tile
    constexpr int VW = TM / 32;     // columns per lane
    constexpr int U = GRAD ? 16 : 24;  // prefetched steps (<= 48 loads in flight)
    __shared__ float red[(TS > 1) ? (TS - 1) * (TM * TM + 2 * TM) : 1];

    const int blk = (int)(blockIdx.x % (NB1 * NB1));
    const int64_t bs = blockIdx.x / (NB1 * NB1);
    const int64_t bh = bs / nseg;
    const int seg = (int)(bs % nseg);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int quad = w % NQ, tsi = w / NQ;
    const int m0 = (blk / NB1) * DB + (quad / NQ1) * TM, n0 = (blk % NB1) * DB + (quad % NQ1) * TM;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const T *xh = X + bh * N * D + m0 + VW * j;
    const T *yh = Y + bh * N * D + n0 + VW * j;
    const float2 *ch = GRAD ? reinterpret_cast<const float2 *>(cbuf) + bh * N : nullptr;
    // The ring loads go through buffer descriptors over the segment's rows:
    // the lane's offset is fixed and each step adds a uniform (scalar) one,
    // and steps past the end read zeros.
    const uint32_t rows = (uint32_t)(end - beg);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(X + (bh * N + beg) * D), (short)0, (int)(rows * D * sizeof(T)), 0x00020000);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(Y + (bh * N + beg) * D), (short)0, (int)(rows * D * sizeof(T)), 0x00020000);
    __amdgpu_buffer_rsrc_t rcb;
    if constexpr (GRAD)
        rcb = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(cbuf + 2 * (bh * N + beg)),
                                                (short)0, (int)(rows * 8), 0x00020000);
    const int ox = (int)((h * D + m0 + VW * j) * sizeof(T));
    const int oy = (int)((h * D + n0 + VW * j) * sizeof(T));

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

    // The ring holds the loaded words as they are (fp32 values, or pairs of
    // 16-bit elements widened only when consumed, so that no load is waited
    // for before its slot comes round).
    constexpr bool WIDE = sizeof(T) == 4;
    constexpr int RW = WIDE ? VW : 1;
    typedef typename std::conditional<WIDE, float, uint32_t>::type RT;
    RT ra[U][RW], rb[U][RW];
    float rc[U], rs[U];
    auto raw_load = [&](__amdgpu_buffer_rsrc_t r, int vo, int so, RT *o) {
        if constexpr (WIDE)
            buf_load_vec<ST, VW>(r, vo, so, o);
        else if constexpr (VW == 2)
            o[0] = __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0);
        else
            o[0] = __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0);
    };
    auto widen_slot = [&](const RT *r, float *o) {
        if constexpr (WIDE) {
#pragma unroll
            for (int a = 0; a < VW; ++a)
                o[a] = r[a];
        } else if constexpr (VW == 2) {
            ST::widen2(r[0], o);
        } else {
            o[0] = ST::widen1((uint16_t)r[0]);
        }
    };
    // Prefetch ring over this wave's complete 2-token steps.  Slots past the
    // last step are fetched (as zeros) but never consumed, so nothing waits on
    // a load before its use.  An odd last token is handled after the loop.
    auto fetch = [&](int u, int s) {
        const int so = __builtin_amdgcn_readfirstlane(s) * (int)(2 * D * sizeof(T));
        raw_load(rx, ox, so, ra[u]);
        raw_load(ry, oy, so, rb[u]);
        if constexpr (GRAD) {
            const float2 cs = __builtin_bit_cast(
                float2, __builtin_amdgcn_raw_buffer_load_b64(
                            rcb, h * 8, __builtin_amdgcn_readfirstlane(s) * 16, 0));
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
        fetch(u, tsi + u * TS);
    for (int it = 0; it < full; ++it) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float xa[VW], yb[VW];
            widen_slot(ra[u], xa);
            widen_slot(rb[u], yb);
            consume(xa, yb, GRAD ? rc[u] : 1.f, GRAD ? rs[u] : 1.f);
            fetch(u, tsi + ((it + 1) * U + u) * TS);
            // keep step u's work and its refill together: the scheduler would
            // otherwise sink the refills to the end of the body and hoist the
            // column-sum adds of later steps, each forcing an early wait
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (u < mine - full * U) {
            float xa[VW], yb[VW];
            widen_slot(ra[u], xa);
            widen_slot(rb[u], yb);
            consume(xa, yb, GRAD ? rc[u] : 1.f, GRAD ? rs[u] : 1.f);
        }
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
        csx[a] = swap32_sum(csx[a]);
        csy[a] = swap32_sum(csy[a]);
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

// ============================================================ split products
// An fp32 value is the exact sum of three bf16 terms, x = hi + mid + lo, each
// rounded to nearest from what the previous ones leave (8 + 8 + 8 bits of
// the 24-bit significand; the differences are exact in fp32).  A product of
// two such values on the bf16 matrix cores keeps the six term products down
// to 2^-16 of the leading one (hi.hi, hi.mid, mid.hi, hi.lo, lo.hi, mid.mid)
// and drops the rest, which lie near 2^-24 relative, below fp32 rounding;
// every term product is exact in the fp32 accumulator.
typedef __bf16 bf8x __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16v mma_bf16(bf8x a, bf8x b, f16v c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split3(const float *x, bf8x &hi, bf8x &mid, bf8x &lo)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 a = (__bf16)x[e];
        const float r = x[e] - (float)a;
        const __bf16 b = (__bf16)r;
        hi[e] = a;
        mid[e] = b;
        lo[e] = (__bf16)(r - (float)b);
    }
}

// the six term products of a (three planes) and b (three planes), smallest
// first
__device__ __forceinline__ f16v mma_split3(const bf8x &a1, const bf8x &a2, const bf8x &a3,
                                           const bf8x &b1, const bf8x &b2, const bf8x &b3,
                                           f16v acc)
{
    acc = mma_bf16(a2, b2, acc);
    acc = mma_bf16(a1, b3, acc);
    acc = mma_bf16(a3, b1, acc);
    acc = mma_bf16(a1, b2, acc);
    acc = mma_bf16(a2, b1, acc);
    return mma_bf16(a1, b1, acc);
}

// ============================================================ apply
// A is the MFMA left operand applied to each row x_i of X:
// KIND 0 forward : A = S^T;  o_i = (u + A q_i) / (N + q_i.z);
//                  X = Q.  den_out[i] = N + q_i.z (optional).
// KIND 2 dK | dV : blockIdx parity 0: A = dS, X = V, dk_j = A v_j - r;
//                  parity 1: A = dS^T, X2 = K, dv_j = A k_j + t.
// rec: total record of the head: Mat[D][D], vec1[D], vec2[D] =
//      (S, z, u) for KIND 0 and (dS, r, t) for KIND 2.
// (dQ is k_bwd_q_nc below.)
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
// per lane (16-byte stores).  Rows past the end of the segment are staged
// as zeros and not stored.
//
// The round loop is software-pipelined so that the MFMA chain of a round
// runs with the other work in its shadow: the stores of the previous
// round's rows are issued between its k-blocks.  In the forward each wave
// forms q_j.z over its own 32 columns of the staged row only; the partials
// meet in LDS at the round's barrier, after which the rows are normalised.
template <class ST, int D, int KIND>
__global__ __launch_bounds__(apply_threads<D>()) void k_apply_nc(
    const typename ST::T *__restrict__ X, const typename ST::T *__restrict__ X2,
    typename ST::T *__restrict__ Out, typename ST::T *__restrict__ Out2,
    float *__restrict__ den_out, const float *__restrict__ rec, int64_t N, int64_t seg_len,
    int nseg, float n0, OutLay ol)
{
    typedef typename ST::T T;
    typedef IO<ST> io;
    static_assert(D >= 32, "32-column output blocks");
    static_assert(KIND == 0 || KIND == 2, "forward or dK | dV");
    constexpr int NT = apply_threads<D>();
    constexpr int KB = D / 8;                // k-blocks of 8
    constexpr int NWAVE = NT / 64;
    constexpr int NCB = D / 32;              // column blocks
    static_assert(NCB <= NWAVE && NWAVE % NCB == 0, "column split");
    constexpr int NRG = NWAVE / NCB;         // row groups
    constexpr int TR = 32 * NRG;             // rows staged per round
    constexpr int LDX = D + 4;               // LDS row pitch (floats)
    constexpr int VEC = 16 / sizeof(T);      // elements per 16-byte load
    constexpr int CPR = D / VEC;             // 16-byte chunks per row
    constexpr int PER = TR * CPR / NT;  // chunks per thread per round
    static_assert(TR * CPR % NT == 0, "staging split");
    __shared__ __attribute__((aligned(16))) float xs[2][TR * LDX];
    __shared__ __attribute__((aligned(16))) float vz[KIND == 0 ? D : 4];  // z
    // forward: q.z of each row over each wave's 32 columns (added up after
    // the round's barrier)
    __shared__ float xch[KIND == 0 ? 2 : 1][NRG][NCB][32];
    // D = 64 (few matrix steps per row, the output stores weigh most): a
    // round's output rows go to an LDS tile and the workgroup stores them as
    // whole 16-byte row pieces LAG rounds later (the dK | dV tile is complete
    // at the round's barrier, the forward's, normalised after it, at the
    // next one).  In the MFMA layout a lane's own stores cover 32 bytes of
    // each of 32 rows per instruction.  (fp32 step at B4 H16 N4096 D64:
    // 0.195 -> 0.182 ms, at two workgroups per CU instead of four; D = 32
    // measured the same either way, D = 128 spends its time on the products.)
    constexpr bool OT = D == 64;
    constexpr int LDO = D + VEC;  // tile row pitch (elements)
    constexpr int LAG = KIND == 0 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) T ot[OT ? 2 : 1][OT ? TR * LDO : VEC];

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

    const T *xh = ((KIND == 2 && sub == 1) ? X2 : X) + hoff;
    T *oh = ((KIND == 2 && sub == 1) ? Out2 : Out) + ol.head(bh);

    // staging: thread's chunk p of a round covers row (tid + p*NT) / CPR,
    // columns VEC*((tid + p*NT) % CPR) ..
    // rows load through a descriptor over the segment (rows past its end read
    // zeros); the lane's offsets are fixed, the round's is a scalar
    const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(xh + beg * D), (short)0, (int)((end - beg) * D * sizeof(T)), 0x00020000);
    uint4 stg[PER];
    auto fetch_round = [&](int64_t r0) {
        const int so = __builtin_amdgcn_readfirstlane((int)((r0 - beg) * D * sizeof(T)));
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            stg[p] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           rsx, (int)(((c / CPR) * D + VEC * (c % CPR)) * sizeof(T)), so, 0));
        }
    };
    // (rows past the segment end were loaded as zeros)
    auto stage_round = [&](int buf) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            float v[VEC];
            ST::widen(stg[p], v);
            float *dst = &xs[buf][(c / CPR) * LDX + VEC * (c % CPR)];
#pragma unroll
            for (int x = 0; x < VEC; x += 4)
                *reinterpret_cast<f4 *>(dst + x) = f4{v[x], v[x + 1], v[x + 2], v[x + 3]};
        }
    };

    const int64_t nrounds = (end - beg + TR - 1) / TR;
    fetch_round(beg);

    // fp16 storage at D = 128: the products run as split products on the
    // bf16 matrix cores (the block of A in three bf16 planes: a1[ks][e] + a2
    // + a3 = A[32*cb + j][16*ks + 8*h + e]), 8% faster per step than on the
    // fp32 matrix cores.  fp32 storage stays on the fp32 matrix cores: there
    // the same change gained 2%, and the extra power slowed the neighbouring
    // fp32 launches.  At D = 256 the planes would not fit in registers; at
    // D <= 64 the fp32 matrix cores were as fast.
    constexpr bool X3 = std::is_same<ST, StF16>::value && D == 128;
    constexpr int KS = D / 16;
    bf8x a1[X3 ? KS : 1], a2[X3 ? KS : 1], a3[X3 ? KS : 1];
    if constexpr (X3) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = 16 * ks + 8 * h + e;
                v[e] = colread ? st[k * D + 32 * cb + j] : st[(32 * cb + j) * D + k];
            }
            split3(v, a1[ks], a2[ks], a3[ks]);
        }
    }
    // else this wave's block of A in fp32: am[kb][r] = A[32*cb + j][kb*8 + 4*h + r]
    float am[X3 ? 1 : KB][4];
    if constexpr (!X3) {
        if (colread) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    am[kb][r] = st[(kb * 8 + 4 * h + r) * D + 32 * cb + j];
        } else {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f4 v =
                    *reinterpret_cast<const f4 *>(st + (32 * cb + j) * D + kb * 8 + 4 * h);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    am[kb][r] = v[r];
            }
        }
    }
    // epilogue vector at the lane's output columns 32*cb + 8*q + 4*h + (0..3):
    // u (forward), -r (dK) or t (dV)
    f4 ev[4];
    {
        const float *vec = st + D * D + ((KIND == 0 || (KIND == 2 && sub == 1)) ? D : 0);
        const float sgn = (KIND == 2 && sub == 0) ? -1.f : 1.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            ev[q] = sgn * *reinterpret_cast<const f4 *>(vec + 32 * cb + 8 * q + 4 * h);
    }
    if constexpr (KIND == 0)
        for (int e = tid; e < D; e += NT)
            vz[e] = st[D * D + e];
    stage_round(0);
    drain_loads();
    if (nrounds > 1)
        fetch_round(beg + TR);
    __syncthreads();

    // the previous round's output rows, stored during the next round (or,
    // with the LDS tile, the round's values put into the tile)
    f4 pend[4];
    int64_t prow = 0;
    bool pok = false;
    auto store_pending = [&](int q) {
        if (pok)
            io::store4(oh + prow * ol.sn + 32 * cb + 8 * q + 4 * h, pend[q]);
    };
    auto put_tile = [&](int tb) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            io::store4(&ot[tb][(32 * rg + j) * LDO + 32 * cb + 8 * q + 4 * h], pend[q]);
    };
    // 16-byte piece p of round rr's tile to global memory (consecutive lanes
    // take consecutive pieces of a row)
    auto store_tile = [&](int64_t rr, int p) {
        const int c = tid + p * NT;
        const int64_t grow = beg + rr * TR + c / CPR;
        if (grow < end)
            *reinterpret_cast<uint4 *>(oh + grow * ol.sn + VEC * (c % CPR)) =
                *reinterpret_cast<const uint4 *>(&ot[(int)(rr & 1)][(c / CPR) * LDO + VEC * (c % CPR)]);
    };

    for (int64_t round = 0; round < nrounds; ++round) {
        const int buf = (int)(round & 1);
        f16v acc = zero16();
        if constexpr (X3) {
            // B operand: the tile row's 8 consecutive values 16*ks + 8*h ..,
            // split into three bf16 planes, one k-step ahead of the MFMAs
            const float *xt = &xs[buf][(32 * rg + j) * LDX + 8 * h];
            f4 xn0 = *reinterpret_cast<const f4 *>(xt);
            f4 xn1 = *reinterpret_cast<const f4 *>(xt + 4);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const float xv[8] = {xn0[0], xn0[1], xn0[2], xn0[3],
                                     xn1[0], xn1[1], xn1[2], xn1[3]};
                if (ks + 1 < KS) {
                    xn0 = *reinterpret_cast<const f4 *>(xt + (ks + 1) * 16);
                    xn1 = *reinterpret_cast<const f4 *>(xt + (ks + 1) * 16 + 4);
                }
                bf8x b1, b2, b3;
                split3(xv, b1, b2, b3);
                acc = mma_split3(a1[ks], a2[ks], a3[ks], b1, b2, b3, acc);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (ks == q * (KS / 4))
                        store_pending(q);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            const float *xt = &xs[buf][(32 * rg + j) * LDX + 4 * h];
            // LDS operands one k-block ahead of the MFMAs; the scheduling
            // barrier per k-block stops the compiler from hoisting every read
            // of the tile
            f4 xn = *reinterpret_cast<const f4 *>(xt);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f4 x = xn;
                if (kb + 1 < KB)
                    xn = *reinterpret_cast<const f4 *>(xt + (kb + 1) * 8);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc = mma32(am[kb][r], x[r], acc);
                if constexpr (OT) {
#pragma unroll
                    for (int p = 0; p < PER; ++p)
                        if (round >= LAG && kb == (p * KB) / PER)
                            store_tile(round - LAG, p);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (kb == q * (KB / 4))
                            store_pending(q);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        const int64_t row = beg + round * TR + 32 * rg + j;
        if constexpr (KIND == 0) {
            // q.z over this wave's 32 columns (lane half h: 16 of them)
            const float *qr = &xs[buf][(32 * rg + j) * LDX + 32 * cb + 16 * h];
            const float *zr = &vz[32 * cb + 16 * h];
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < 16; e += 4)
                p += dot4(*reinterpret_cast<const f4 *>(qr + e), *reinterpret_cast<const f4 *>(zr + e));
            p = swap32_sum(p);
            if (h == 0)
                xch[buf][rg][cb][j] = p;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pend[q] = f4{acc[4 * q] + ev[q][0], acc[4 * q + 1] + ev[q][1],
                             acc[4 * q + 2] + ev[q][2], acc[4 * q + 3] + ev[q][3]};
            if constexpr (OT)
                put_tile(buf);
        }
        prow = row;
        pok = row < end;
        // stage the next round (its buffer was last read before the previous
        // barrier) and fetch the one after
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
                qz += xch[buf][rg][c2][j];
            const float den = (n0 + (float)N) + qz;
            const float inv = 1.f / den;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pend[q] = f4{(acc[4 * q] + ev[q][0]) * inv, (acc[4 * q + 1] + ev[q][1]) * inv,
                             (acc[4 * q + 2] + ev[q][2]) * inv, (acc[4 * q + 3] + ev[q][3]) * inv};
            if (den_out != nullptr && row < end && h == 0 && cb == 0)
                den_out[bh * N + row] = den;
            if constexpr (OT)
                put_tile(buf);
        }
    }
    if constexpr (OT) {
        __syncthreads();
        for (int64_t rr = nrounds - LAG < 0 ? 0 : nrounds - LAG; rr < nrounds; ++rr)
#pragma unroll
            for (int p = 0; p < PER; ++p)
                store_tile(rr, p);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            store_pending(q);
    }
}

// ============================================================ dQ + gradient record
// One pass over a segment's rows of Q and dO that produces dQ (as KIND 1 of
// k_apply_nc) and the segment's gradient record [dS | r | t] (as
// k_reduce_nc<GRAD = true>) without a second read of Q and dO:
//   a_i = g_i / den_i,  den_i = N + q_i.z,  y_i = S a_i,
//   c_i = (a_i.u + q_i.y_i) / den_i,  dq_i = y_i - c_i z,
//   dS = sum_i q_i a_i^T,  r = sum_i c_i q_i,  t = sum_i a_i.
// The workgroup has two roles of four waves each, so that no wave holds both
// a D x D slice of S (the dQ product) and one of dS (the reduction):
//   role 0 (waves 0-3): the dQ rows (y = S g as k_apply_nc applies its
//                       state), normalised after the round's barrier;
//   role 1 (waves 4-7): dS[:, 32*cb ..] over the round's rows, with
//                       a_i = g_i / den_i; r needs c_i, which role 0 hands
//                       over through LDS one round later.
// Both roles stage the rows (Q and dO, fp32, double-buffered), forming
// 1/den_i of each staged row on the way, and meet at one barrier per round:
// role 1 stages its half of the next round's rows before its MFMA chain and
// role 0 its half after its own, so that each role's staging runs beside the
// other role's chain on the SIMD they share.  With DS = false (D = 256,
// where a wave of either role needs 128 registers of state) the workgroup is
// eight dQ waves only, and it writes (c_i, 1/den_i) to part_out (as cbuf)
// for k_reduce_nc<GRAD = true>.
template <class ST, int D, bool DS = true>
__global__ __launch_bounds__(512) void k_bwd_q_nc(
    const typename ST::T *__restrict__ G, const typename ST::T *__restrict__ Q,
    typename ST::T *__restrict__ dQ, float *__restrict__ part_out,
    const float *__restrict__ rec, int64_t N, int64_t seg_len, int nseg, float n0, OutLay ol)
{
    typedef typename ST::T T;
    typedef IO<ST> io;
    static_assert(D >= 32, "32-column output blocks");
    constexpr int KB = D / 8;
    constexpr int NCB = D / 32;
    // waves of the dQ role: four next to four of the dS role, or (without
    // the dS role, D = 256) one per column block
    constexpr int NW0 = DS ? 4 : (NCB > 4 ? NCB : 4);
    constexpr int NT = DS ? 512 : 64 * NW0;
    static_assert(NT == 512 && NW0 % NCB == 0 && (!DS || NCB <= 4), "role layout");
    constexpr int NRG = NW0 / NCB;
    constexpr int TR = 32 * NRG;
    constexpr int LDX = D + 4;
    constexpr int VEC = 16 / sizeof(T);
    constexpr int CPR = D / VEC;
    constexpr int PER = TR * CPR / NT;
    static_assert(PER >= 1 && TR * CPR % NT == 0, "staging split");
    __shared__ __attribute__((aligned(16))) float xs[2][TR * LDX];  // dO rows
    __shared__ __attribute__((aligned(16))) float qs[2][TR * LDX];  // Q rows
    __shared__ __attribute__((aligned(16))) float vl[2 * D];        // z | u
    __shared__ float xch[2][NRG][NCB][32][2];  // dO.u and q.(S dO) partials
    __shared__ float cx[2][NRG][32];           // c_i of the round's rows
    __shared__ float ivx[2][TR];               // 1/den_i of the round's rows

    int64_t bh;
    int seg;
    xcd_unit(blockIdx.x, nseg, bh, seg);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
    const int role = DS ? (w >> 2) : 0, w0 = DS ? (w & 3) : w;
    const int cb = w0 % NCB, rg = w0 / NCB;
    const int64_t beg = (int64_t)seg * seg_len;
    const int64_t end = (beg + seg_len < N) ? beg + seg_len : N;
    const int64_t hoff = bh * N * D;
    const float *st = rec + bh * (int64_t)(D * D + 2 * D);
    const T *gh = G + hoff, *qh = Q + hoff;
    T *oh = dQ + ol.head(bh);

    // rows load through descriptors over the segment (rows past its end read
    // zeros); the lane's offsets are fixed, the round's is a scalar
    const int segb = (int)((end - beg) * D * sizeof(T));
    const __amdgpu_buffer_rsrc_t rsg =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(gh + beg * D), (short)0, segb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsq =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(qh + beg * D), (short)0, segb, 0x00020000);
    uint4 sg[PER], sq[PER];
    auto fetch_round = [&](int64_t r0) {
        const int so = __builtin_amdgcn_readfirstlane((int)((r0 - beg) * D * sizeof(T)));
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            const int vo = (int)(((c / CPR) * D + VEC * (c % CPR)) * sizeof(T));
            sg[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsg, vo, so, 0));
            sq[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsq, vo, so, 0));
        }
    };
    // widened chunk to LDS (rows past the segment end were loaded as zeros);
    // returns the values
    auto stage_one = [&](float *lds, const uint4 &src, int c, float (&v)[VEC]) {
        ST::widen(src, v);
        float *dst = lds + (c / CPR) * LDX + VEC * (c % CPR);
#pragma unroll
        for (int x = 0; x < VEC; x += 4)
            *reinterpret_cast<f4 *>(dst + x) = f4{v[x], v[x + 1], v[x + 2], v[x + 3]};
    };
    // Staging also forms den_i = N + q_i.z of every staged row, once per row
    // (the CPR consecutive threads that stage a row add their chunks' dot
    // products by shuffles: a row's chunks lie in one wave), stores the dO
    // row already divided by it, a_i = g_i / den_i, and keeps 1/den_i in LDS.
    static_assert(CPR <= 64 && 64 % CPR == 0, "a staged row lies in one wave");
    auto stage_round = [&](int buf) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int c = tid + p * NT;
            float qv[VEC];
            stage_one(qs[buf], sq[p], c, qv);
            const float *zc = &vl[VEC * (c % CPR)];
            float pz = 0.f;
#pragma unroll
            for (int x = 0; x < VEC; x += 4)
                pz += dot4(f4{qv[x], qv[x + 1], qv[x + 2], qv[x + 3]},
                           *reinterpret_cast<const f4 *>(zc + x));
            pz = group_sum<CPR>(pz);
            const float inv = 1.f / ((n0 + (float)N) + pz);
            if (c % CPR == 0)
                ivx[buf][c / CPR] = inv;
            float gv[VEC];
            ST::widen(sg[p], gv);
            float *dst = xs[buf] + (c / CPR) * LDX + VEC * (c % CPR);
#pragma unroll
            for (int x = 0; x < VEC; x += 4)
                *reinterpret_cast<f4 *>(dst + x) = f4{gv[x], gv[x + 1], gv[x + 2], gv[x + 3]} * inv;
        }
    };

    const int64_t nrounds = (end - beg + TR - 1) / TR;
    fetch_round(beg);
    for (int e = tid; e < 2 * D; e += NT)
        vl[e] = st[D * D + e];
    // Role 0's block of S (loaded by every wave so that the registers are
    // set on every path; dead in role 1).  For fp16 storage at D = 128 (as
    // in k_apply_nc) its product y = S a runs as split products on the bf16
    // matrix cores: s1[ks][e] + s2 + s3 = S[32*cb + j][16*ks + 8*h + e];
    // else in fp32: am[kb][r] = S[32*cb + j][kb*8 + 4*h + r].
    constexpr bool X3 = DS && std::is_same<ST, StF16>::value && D == 128;
    constexpr int KS = D / 16;
    bf8x s1[X3 ? KS : 1], s2[X3 ? KS : 1], s3[X3 ? KS : 1];
    float am[X3 ? 1 : KB][4];
    if constexpr (X3) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float *p = st + (32 * cb + j) * D + 16 * ks + 8 * h;
            const f4 v0 = *reinterpret_cast<const f4 *>(p), v1 = *reinterpret_cast<const f4 *>(p + 4);
            const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            split3(v, s1[ks], s2[ks], s3[ks]);
        }
    } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const f4 v = *reinterpret_cast<const f4 *>(st + (32 * cb + j) * D + kb * 8 + 4 * h);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                am[kb][r] = v[r];
        }
    }
    __syncthreads();  // z in LDS before the first staging reads it
    stage_round(0);
    drain_loads();
    if (nrounds > 1)
        fetch_round(beg + TR);
    __syncthreads();

    f16v gacc[NCB];
    float racc = 0.f, tacc = 0.f;
    float qcur[16], qprev[16];
    if (role == 0) {
        for (int64_t round = 0; round < nrounds; ++round) {
            const int buf = (int)(round & 1);
            const int64_t row = beg + round * TR + 32 * rg + j;
            // (read before the barrier: the slot is restaged one round later)
            const float inv = ivx[buf][32 * rg + j];
            f16v acc = zero16();
            if constexpr (X3) {
                // the row of a, 8 values 16*ks + 8*h .. per k-step, split
                // into three bf16 planes one k-step ahead of the MFMAs
                const float *xt = &xs[buf][(32 * rg + j) * LDX + 8 * h];
                f4 xn0 = *reinterpret_cast<const f4 *>(xt);
                f4 xn1 = *reinterpret_cast<const f4 *>(xt + 4);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const float xv[8] = {xn0[0], xn0[1], xn0[2], xn0[3],
                                         xn1[0], xn1[1], xn1[2], xn1[3]};
                    if (ks + 1 < KS) {
                        xn0 = *reinterpret_cast<const f4 *>(xt + (ks + 1) * 16);
                        xn1 = *reinterpret_cast<const f4 *>(xt + (ks + 1) * 16 + 4);
                    }
                    bf8x b1, b2, b3;
                    split3(xv, b1, b2, b3);
                    acc = mma_split3(s1[ks], s2[ks], s3[ks], b1, b2, b3, acc);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                const float *xt = &xs[buf][(32 * rg + j) * LDX + 4 * h];
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
            }
            // y' = S a in acc; partial a.u and q.y' over this block's columns
            {
                const float *xr = &xs[buf][(32 * rg + j) * LDX + 32 * cb + 4 * h];
                const float *qr = &qs[buf][(32 * rg + j) * LDX + 32 * cb + 4 * h];
                float p0 = 0.f, p2 = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f4 qv = *reinterpret_cast<const f4 *>(qr + 8 * q);
                    p0 += dot4(*reinterpret_cast<const f4 *>(xr + 8 * q),
                               *reinterpret_cast<const f4 *>(&vl[D + 32 * cb + 8 * q + 4 * h]));
                    p2 += qv[0] * acc[4 * q] + qv[1] * acc[4 * q + 1] + qv[2] * acc[4 * q + 2] +
                          qv[3] * acc[4 * q + 3];
                }
                p0 = swap32_sum(p0);
                p2 = swap32_sum(p2);
                if (h == 0) {
                    xch[buf][rg][cb][j][0] = p0;
                    xch[buf][rg][cb][j][1] = p2;
                }
            }
            if (round + 1 < nrounds) {
                stage_round(buf ^ 1);
                if (round + 2 < nrounds)
                    fetch_round(beg + (round + 2) * TR);
            }
            __syncthreads();
            float rz = 0.f, qy = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < NCB; ++c2) {
                rz += xch[buf][rg][c2][j][0];
                qy += xch[buf][rg][c2][j][1];
            }
            const float c = (rz + qy) * inv;  // (a.u + q.S a) / den
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f4 z = *reinterpret_cast<const f4 *>(&vl[32 * cb + 8 * q + 4 * h]);
                const f4 o = {acc[4 * q] - c * z[0], acc[4 * q + 1] - c * z[1],
                              acc[4 * q + 2] - c * z[2], acc[4 * q + 3] - c * z[3]};
                if (row < end)
                    io::store4(oh + row * ol.sn + 32 * cb + 8 * q + 4 * h, o);
            }
            if constexpr (DS) {
                if (cb == 0 && h == 0)
                    cx[buf][rg][j] = c;
            } else {
                // (c_i, 1/den_i) for the separate gradient reduction
                if (cb == 0 && h == 0 && row < end)
                    reinterpret_cast<float2 *>(part_out)[bh * N + row] = float2{c, inv};
            }
        }
    } else if constexpr (DS) {
#pragma unroll
        for (int t = 0; t < NCB; ++t)
            gacc[t] = zero16();
        for (int64_t round = 0; round < nrounds; ++round) {
            const int buf = (int)(round & 1);
            // this role's half of the next round's rows first (buffer
            // buf ^ 1 was last read before the previous barrier), while
            // role 0 runs its chain; role 0 stages its half after its chain
            if (round + 1 < nrounds) {
                stage_round(buf ^ 1);
                if (round + 2 < nrounds)
                    fetch_round(beg + (round + 2) * TR);
            }
            // dS[:, block cb] += Q^T A over the tile's rows (k = row; rows
            // 2kk + h per MFMA step), operands one step ahead.  Lane j reads
            // NCB consecutive columns NCB j .. of its q row as one vector:
            // tile t takes column NCB j + t, so its output row m is dS row
            // NCB m + t.
            const float *qt = &qs[buf][(32 * rg + h) * LDX + NCB * j];
            const float *qc = &qs[buf][(32 * rg + h) * LDX + 32 * cb + j];
            const float *gt = &xs[buf][(32 * rg + h) * LDX + 32 * cb + j];
            typedef float fv __attribute__((ext_vector_type(NCB)));
            fv an = *reinterpret_cast<const fv *>(qt);
            float gn = gt[0];
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const fv a = an;
                const float bv = gn;  // a_i = g_i / den_i, staged
                if (kk + 1 < 16) {
                    gn = gt[(2 * kk + 2) * LDX];
                    an = *reinterpret_cast<const fv *>(qt + (2 * kk + 2) * LDX);
                }
                tacc += bv;
#pragma unroll
                for (int t = 0; t < NCB; ++t)
                    gacc[t] = mma32(a[t], bv, gacc[t]);
                qcur[kk] = qc[2 * kk * LDX];
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
            // r += c_i q_i over the previous round's rows (c_i arrived in LDS
            // from role 0 before this barrier)
            if (round > 0) {
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    racc += cx[buf ^ 1][rg][2 * kk + h] * qprev[kk];
            }
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
                qprev[kk] = qcur[kk];
        }
    }
    if constexpr (!DS)
        return;
    __syncthreads();  // the last round's c_i is in LDS; staging buffers are free

    constexpr int PW = NCB * 16 * 64 + 64;  // floats per handing wave
    static_assert((NRG - 1) * NCB * PW <= 2 * TR * LDX, "merge space");
    float *red = &xs[0][0];
    if (role == 1) {
        if (nrounds > 0) {
            const int lb = (int)((nrounds - 1) & 1);
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
                racc += cx[lb][rg][2 * kk + h] * qprev[kk];
        }
        racc = swap32_sum(racc);
        tacc = swap32_sum(tacc);
        if (NRG > 1 && rg > 0) {
            float *dst = red + ((rg - 1) * NCB + cb) * PW;
#pragma unroll
            for (int t = 0; t < NCB; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    dst[(t * 16 + i) * 64 + lane] = gacc[t][i];
            if (h == 0) {
                dst[NCB * 16 * 64 + j] = racc;
                dst[NCB * 16 * 64 + 32 + j] = tacc;
            }
        }
    }
    __syncthreads();
    if (role == 1 && rg == 0) {
        for (int o = 1; o < NRG; ++o) {
            const float *src = red + ((o - 1) * NCB + cb) * PW;
#pragma unroll
            for (int t = 0; t < NCB; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    gacc[t][i] += src[(t * 16 + i) * 64 + lane];
            racc += src[NCB * 16 * 64 + j];
            tacc += src[NCB * 16 * 64 + 32 + j];
        }
        float *out = part_out + (bh * nseg + seg) * (int64_t)(D * D + 2 * D);
#pragma unroll
        for (int t = 0; t < NCB; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                out[(NCB * (8 * (i / 4) + 4 * h + (i % 4)) + t) * D + 32 * cb + j] = gacc[t][i];
        if (h == 0) {
            out[D * D + 32 * cb + j] = racc;
            out[D * D + D + 32 * cb + j] = tacc;
        }
    }
}

}  // namespace nc
}  // namespace la
